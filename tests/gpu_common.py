"""Shared helpers of the GPU parity tests: device transfer and the checkers that
compare GPU results with the oracle's."""
from __future__ import annotations

import numpy as np
import torch

from oracle import formats as F
from oracle.quant import element_codes, block_scale_codes, unpack_codes

DEV = torch.device("cuda:0")


def up(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(DEV)


def down(t):
    return t.detach().cpu().numpy()


def bf16_up(x32):
    """float32 values that are bf16 values -> bf16 GPU tensor (exact)."""
    return up(x32).to(torch.bfloat16)


def bf16_to_f32(t):
    return t.detach().float().cpu().numpy()


def assert_gemm_close(y_gpu, y_ref, absdot, bf16_out=False, what="gemm"):
    """|y - y_ref| <= 1e-3 * sum|a*b| + 1e-6 per element; a bfloat16 output also
    gets 2^-8 |y_ref| for its own rounding."""
    y_gpu = np.asarray(y_gpu, np.float64)
    tol = 1e-3 * absdot + 1e-6
    if bf16_out:
        tol = tol + 2.0 ** -8 * np.abs(y_ref)
    err = np.abs(y_gpu - y_ref)
    bad = err > tol
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance; first {tuple(i)}: "
                             f"gpu {y_gpu[tuple(i)]} ref {y_ref[tuple(i)]} tol {tol[tuple(i)]}")
    return float((err / np.maximum(tol, 1e-30)).max())


E2M1_MIDPOINTS = (F.E2M1_MAGNITUDES[:-1] + F.E2M1_MAGNITUDES[1:]) / 2
E4M3_MIDPOINTS = (F.E4M3_POS[:-1] + F.E4M3_POS[1:]) / 2


def check_requant(codes_gpu, scales_gpu, x_ref, g, tol_abs, max_flip_frac=1e-3, what="requant"):
    """GPU NVFP4 codes of a value the GPU computed itself (so it may differ from
    the oracle's value x_ref by up to tol_abs per element) against the oracle's
    encoding of x_ref.

    * a block scale may differ only by one code, and only where the oracle's
      t = (absmax/6)/g lies within the propagated tolerance of the E4M3
      decision point between the two codes; such blocks are checked by the
      error bound of the GPU's own encoding instead of code by code;
    * an element code may differ only by one magnitude step, and only where the
      oracle's |x|/(s*g) lies within tol of the E2M1 decision point between
      them (a zero may carry either sign when |x_ref| <= tol);
    * at most max_flip_frac of the elements may differ at all.
    Returns (number of scale flips, number of code flips)."""
    x32 = np.asarray(x_ref, np.float64).astype(np.float32)
    rows, cols = x32.shape
    tol_abs = np.broadcast_to(np.asarray(tol_abs, np.float64), x32.shape)
    g = np.float32(g)
    s_ref = block_scale_codes(x32, g)
    s_gpu = np.asarray(scales_gpu, np.uint8).reshape(rows, cols // 16)
    c_gpu = unpack_codes(np.asarray(codes_gpu, np.uint8).reshape(rows, cols // 2))

    # ---- block scales
    sdiff = s_gpu != s_ref
    nsflip = int(sdiff.sum())
    if nsflip:
        blk_abs = np.abs(x32).reshape(rows, -1, 16).astype(np.float64)
        amax = blk_abs.max(axis=2)
        tol_blk = tol_abs.reshape(rows, -1, 16).max(axis=2)
        t = amax / 6 / np.float64(g)
        tol_t = tol_blk / 6 / np.float64(g) + t * 2.0 ** -22
        lo = np.minimum(s_gpu, s_ref).astype(np.int64)
        adjacent = np.abs(s_gpu.astype(np.int64) - s_ref.astype(np.int64)) == 1
        mid = E4M3_MIDPOINTS[np.clip(lo, 0, len(E4M3_MIDPOINTS) - 1)]
        near = np.abs(t - mid) <= tol_t
        bad = sdiff & ~(adjacent & near)
        if bad.any():
            i = tuple(np.argwhere(bad)[0])
            raise AssertionError(f"{what}: block scale {i} gpu {s_gpu[i]:#x} ref {s_ref[i]:#x} t {t[i]} "
                                 f"tol {tol_t[i]}")
        # error bound of the GPU's own encoding in flipped blocks
        sv = np.repeat(F.e4m3_decode(s_gpu), 16, axis=1) * np.float64(g)
        deq = F.e2m1_decode(c_gpu) * sv
        blk = np.repeat(sdiff, 16, axis=1)
        v = np.abs(x32.astype(np.float64)) / np.where(sv > 0, sv, 1)
        hi = np.clip(np.searchsorted(F.E2M1_MAGNITUDES, v), 1, 7)
        gap = F.E2M1_MAGNITUDES[hi] - F.E2M1_MAGNITUDES[hi - 1]
        bound = np.where(v > 6, np.abs(x32) - 6 * sv, 0.5 * gap * sv) + tol_abs + 1e-30
        if np.any((np.abs(deq - x32) > bound * (1 + 1e-6))[blk]):
            raise AssertionError(f"{what}: codes of a flipped-scale block exceed the quantisation bound")

    # ---- element codes where the scales agree
    c_ref = element_codes(x32, s_ref, g)
    same_blk = np.repeat(~sdiff, 16, axis=1)
    cdiff = (c_gpu != c_ref) & same_blk
    ncflip = int(cdiff.sum())
    if ncflip:
        sv = np.repeat(F.e4m3_decode(s_ref), 16, axis=1) * np.float64(g)
        v = np.abs(x32.astype(np.float64)) / np.where(sv > 0, sv, 1)
        tol_v = tol_abs / np.where(sv > 0, sv, 1) + v * 2.0 ** -22
        mg, mr = (c_gpu & 7).astype(np.int64), (c_ref & 7).astype(np.int64)
        sign_ok = ((c_gpu & 8) == (c_ref & 8)) | ((mg == 0) & (mr == 0) & (np.abs(x32) <= tol_abs))
        adjacent = np.abs(mg - mr) <= 1
        mid = E2M1_MIDPOINTS[np.clip(np.minimum(mg, mr), 0, 6)]
        near = (mg == mr) | (np.abs(v - mid) <= tol_v)
        bad = cdiff & ~(sign_ok & adjacent & near)
        if bad.any():
            i = tuple(np.argwhere(bad)[0])
            raise AssertionError(f"{what}: code {i} gpu {c_gpu[i]:#x} ref {c_ref[i]:#x} v {v[i]} tol {tol_v[i]}")
    flips = nsflip * 16 + ncflip
    if flips > max_flip_frac * x32.size:
        raise AssertionError(f"{what}: {nsflip} scale flips and {ncflip} code flips in {x32.size} elements")
    return nsflip, ncflip


def check_requant_mx(codes_gpu, scales_gpu, x_ref, tol_abs, max_flip_frac=1e-3, what="mx requant"):
    """GPU MXFP4 codes of a value the GPU computed itself (within tol_abs of
    the oracle's x_ref per element) against the oracle's MXFP4 encoding of x_ref.

    * a block's E8M0 scale may differ by one code, and only where the oracle's
      block absmax lies within the block's tolerance of the power of two
      between the two exponents; such blocks are checked by the error bound of
      the GPU's own encoding;
    * an element code may differ by one magnitude step, and only where the
      oracle's |x| / 2^X lies within tol of the E2M1 decision point between them;
    * at most max_flip_frac of the elements may differ.
    Returns (scale flips, code flips)."""
    from oracle import mx as MXO
    x32 = np.asarray(x_ref, np.float64).astype(np.float32)
    rows, cols = x32.shape
    tol_abs = np.broadcast_to(np.asarray(tol_abs, np.float64), x32.shape)
    c_ref, s_ref = MXO.mx_quantize(x32)
    s_gpu = np.asarray(scales_gpu, np.uint8).reshape(rows, cols // 32)
    c_gpu = unpack_codes(np.asarray(codes_gpu, np.uint8).reshape(rows, cols // 2))
    c_ref = unpack_codes(c_ref)
    sdiff = s_gpu != s_ref
    nsflip = int(sdiff.sum())
    if nsflip:
        blk = np.abs(x32.astype(np.float64)).reshape(rows, -1, 32)
        amax = blk.max(axis=2)
        tol_blk = tol_abs.reshape(rows, -1, 32).max(axis=2) + amax * 2.0 ** -22
        hi = np.maximum(s_gpu, s_ref).astype(np.int64) - 127 + 2        # the power of two between
        adjacent = np.abs(s_gpu.astype(np.int64) - s_ref.astype(np.int64)) == 1
        near = np.abs(amax - np.exp2(hi.astype(np.float64))) <= tol_blk
        bad = sdiff & ~(adjacent & near)
        if bad.any():
            i = tuple(np.argwhere(bad)[0])
            raise AssertionError(f"{what}: block scale {i} gpu {s_gpu[i]} ref {s_ref[i]} amax {amax[i]} tol {tol_blk[i]}")
        sv = np.repeat(np.exp2(s_gpu.astype(np.float64) - 127), 32, axis=1)
        deq = F.e2m1_decode(c_gpu) * sv
        v = np.abs(x32.astype(np.float64)) / sv
        hi2 = np.clip(np.searchsorted(F.E2M1_MAGNITUDES, v), 1, 7)
        gap = F.E2M1_MAGNITUDES[hi2] - F.E2M1_MAGNITUDES[hi2 - 1]
        bound = np.where(v > 6, np.abs(x32) - 6 * sv, 0.5 * gap * sv) + tol_abs + 1e-30
        fb = np.repeat(sdiff, 32, axis=1)
        if np.any((np.abs(deq - x32) > bound * (1 + 1e-6))[fb]):
            raise AssertionError(f"{what}: codes of a flipped-scale block exceed the quantisation bound")
    same = np.repeat(~sdiff, 32, axis=1)
    cdiff = (c_gpu != c_ref) & same
    ncflip = int(cdiff.sum())
    if ncflip:
        sv = np.repeat(np.exp2(s_ref.astype(np.float64) - 127), 32, axis=1)
        v = np.abs(x32.astype(np.float64)) / sv
        tol_v = tol_abs / sv + v * 2.0 ** -22
        mg, mr = (c_gpu & 7).astype(np.int64), (c_ref & 7).astype(np.int64)
        sign_ok = ((c_gpu & 8) == (c_ref & 8)) | ((mg == 0) & (mr == 0) & (np.abs(x32) <= tol_abs))
        mid = E2M1_MIDPOINTS[np.clip(np.minimum(mg, mr), 0, 6)]
        near = (mg == mr) | (np.abs(v - mid) <= tol_v)
        bad = cdiff & ~(sign_ok & (np.abs(mg - mr) <= 1) & near)
        if bad.any():
            i = tuple(np.argwhere(bad)[0])
            raise AssertionError(f"{what}: code {i} gpu {c_gpu[i]:#x} ref {c_ref[i]:#x} v {v[i]} tol {tol_v[i]}")
    if nsflip * 32 + ncflip > max_flip_frac * x32.size:
        raise AssertionError(f"{what}: {nsflip} scale flips and {ncflip} code flips in {x32.size} elements")
    return nsflip, ncflip


def check_requant_fp8(codes_gpu, scales_gpu, x_ref, tol_abs, max_flip_frac=1e-3, what="fp8 requant"):
    """GPU FP8 (1 x 128 block) codes of a value the GPU computed itself (within
    tol_abs of the oracle's x_ref per element) against the oracle's FP8 encoding
    of x_ref.

    * a block's float32 scale s = absmax / 448 may differ from the oracle's by
      at most the block's tolerance / 448 (plus 2 ulp);
    * a differing element code must be the E4M3 rounding of some value within
      the element's tolerance (over s, plus the scale's relative difference)
      of the oracle's x / s: a code between the roundings of the interval's
      two ends, with the sign of x unless the interval holds 0;
    * at most max_flip_frac of the elements may differ.
    Returns (scale differences, code flips)."""
    from oracle import fp8 as F8
    x32 = np.asarray(x_ref, np.float64).astype(np.float32)
    rows, cols = x32.shape
    tol_abs = np.broadcast_to(np.asarray(tol_abs, np.float64), x32.shape)
    c_ref, s_ref = F8.fp8_quantize(x32, 1)
    s_gpu = np.asarray(scales_gpu, np.float32).reshape(rows, cols // 128).astype(np.float64)
    s_r = s_ref.astype(np.float64)
    c_gpu = np.asarray(codes_gpu, np.uint8).reshape(rows, cols)
    tol_blk = tol_abs.reshape(rows, -1, 128).max(axis=2) / 448.0 + s_r * 2.0 ** -22
    sbad = np.abs(s_gpu - s_r) > tol_blk
    if sbad.any():
        i = tuple(np.argwhere(sbad)[0])
        raise AssertionError(f"{what}: block scale {i} gpu {s_gpu[i]!r} ref {s_r[i]!r} tol {tol_blk[i]}")
    nsdiff = int((s_gpu != s_r).sum())
    cdiff = c_gpu != c_ref
    ncflip = int(cdiff.sum())
    if ncflip:
        sv = np.repeat(s_r, 128, axis=1)
        rel_s = np.repeat(np.abs(s_gpu - s_r) / s_r, 128, axis=1)
        xs = x32.astype(np.float64) / sv                       # signed quotient
        tol_v = tol_abs / sv + np.abs(xs) * (rel_s + 2.0 ** -22)
        lo, hi = xs - tol_v, xs + tol_v
        mag_g = F8.e4m3_decode(c_gpu & 0x7F)
        neg_g = (c_gpu & 0x80) != 0
        val_g = np.where(neg_g, -mag_g, mag_g)
        # the E4M3 roundings of the interval's ends, as signed grid values
        def rnd(t):
            m = F8.e4m3_decode(F8.e4m3_encode_satfinite(np.minimum(np.abs(t), F8.E4M3_MAX)))
            return np.where(t < 0, -m, m)
        r_lo, r_hi = rnd(lo), rnd(hi)
        in_range = (val_g >= r_lo) & (val_g <= r_hi)
        sign_ok = (neg_g == (xs < 0)) | (mag_g == 0) | ((lo <= 0) & (hi >= 0))
        bad = cdiff & ~(in_range & sign_ok)
        if bad.any():
            i = tuple(np.argwhere(bad)[0])
            raise AssertionError(f"{what}: code {i} gpu {c_gpu[i]:#x} ref {c_ref[i]:#x} x/s {xs[i]} tol {tol_v[i]}")
    if ncflip > max_flip_frac * x32.size:
        raise AssertionError(f"{what}: {ncflip} code flips in {x32.size} elements")
    return nsdiff, ncflip
