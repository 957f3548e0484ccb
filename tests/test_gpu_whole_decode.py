"""Whole-output parity of the kernel instances the benchmark times, at the
Zipf-skewed decode shape (T=2048, H=6144, I=256, E=256, top-8): every output
of every stage, element by element, in the benchmark's launch configuration
(packed weight tiles and no rows-per-expert hint, which select the decode tile,
cached weight loads and the light-chunk split that the layer step runs).

Each GPU stage is fed the oracle's previous-stage result; no oracle input comes
from the GPU.  The stages' inputs: the workload's routing (the oracle's, which
the routing tests show the GPU reproduces bit for bit), x quantised by the
oracle, weight operands drawn as seeded NVFP4 bytes (raw inputs of the GEMM),
h quantised by the oracle from its own y1, and the oracle's y2 rounded to bf16
for the combine.

Tolerances (from the GEMM contract, FP32 accumulation of exact block terms):
y1 and y2 within 1e-3 * sum|a^ b^| + 1e-6 (y2, stored as bf16, also 2^-8 |y|);
the combine within its float32 summation bound plus the bf16 rounding; the
fused SwiGLU requantisation code by code, a flip accepted only next to an
E2M1/E4M3 decision point within the propagated y1 tolerance, and, where y1 is
exact on both sides (constant block scales), only within 1e-6 relative of the
decision point."""
import functools

import numpy as np
import pytest
import torch

import block_scaled_fp4_permute_amd as m
import workloads
from oracle import moe as OM
from oracle import quant as OQ
from tests.gpu_common import DEV, assert_gemm_close, bf16_to_f32, check_requant, down, up

pytestmark = pytest.mark.gpu

CFG = workloads.CONFIGS[2]
G_GU = np.float32(2.0 ** -15)     # per-expert weight scales (powers of two)
G_DN = np.float32(2.0 ** -14)


@functools.lru_cache(maxsize=None)
def _inputs():
    c = CFG
    logits = workloads.logits(c)
    x = workloads.activations(c)
    ids, w = OM.route(logits, c.k)
    counts, offsets, src, perm_of, pw = OM.permute(ids, w, c.E)
    xq = OQ.quantize(x)
    gu = workloads.nvfp4_codes(c, 0, (c.E, 2 * c.I), c.H)
    dn = workloads.nvfp4_codes(c, 1, (c.E, c.H), c.I)
    return dict(ids=ids, w=w, counts=counts, offsets=offsets, src=src, perm_of=perm_of, xq=xq, gu=gu, dn=dn,
                g_gu=np.full(c.E, G_GU, np.float32), g_dn=np.full(c.E, G_DN, np.float32))


@functools.lru_cache(maxsize=None)
def _oracle_y1():
    d = _inputs()
    return OM.grouped_gemm(*d["xq"], *d["gu"], d["g_gu"], d["offsets"], a_rows=d["src"])


@functools.lru_cache(maxsize=None)
def _oracle_h():
    y1, _ = _oracle_y1()
    h64 = OM.swiglu(y1)
    g_h = np.float32(np.float32(np.abs(h64.astype(np.float32)).max()) / np.float32(2688.0))
    hq = OQ.quantize(h64.astype(np.float32), g=g_h)
    return h64, hq


@functools.lru_cache(maxsize=None)
def _oracle_y2():
    d = _inputs()
    _, hq = _oracle_h()
    return OM.grouped_gemm(*hq, *d["dn"], d["g_dn"], d["offsets"])


@functools.lru_cache(maxsize=None)
def _device():
    d = _inputs()
    xc, xs, xg = d["xq"]
    gu_c, gu_s = up(d["gu"][0]), up(d["gu"][1])
    dn_c, dn_s = up(d["dn"][0]), up(d["dn"][1])
    dev = dict(x=m.NVFP4Tensor(up(xc), up(xs), up(np.array([xg], np.float32))),
               gu_c=gu_c, gu_s=gu_s, gu_p=m.nvfp4_weight_repack(gu_c, gu_s), gu_g=up(d["g_gu"]),
               dn_c=dn_c, dn_s=dn_s, dn_p=m.nvfp4_weight_repack(dn_c, dn_s), dn_g=up(d["g_dn"]),
               offsets=up(d["offsets"]), src=up(d["src"]), perm_of=up(d["perm_of"]), w=up(d["w"]))
    torch.cuda.synchronize()
    return dev


def _swiglu_tol(y1_ref, absdot1):
    I = y1_ref.shape[1] // 2
    tol_y = 1e-3 * absdot1 + 1e-6
    g, u = y1_ref[:, :I].astype(np.float64), y1_ref[:, I:].astype(np.float64)
    silu = OM.silu(g)
    return 1.1 * tol_y[:, :I] * np.abs(u) + np.abs(silu) * tol_y[:, I:] + 2.0 ** -20 * np.abs(silu * u) + 1e-7


def test_whole_gate_up_f32():
    print("whole gate_up f32 (T=2048 Zipf decode shape)", flush=True)
    d, g = _inputs(), _device()
    M = CFG.T * CFG.k
    y = m.nvfp4_grouped_gemm(g["x"], g["gu_c"], g["gu_s"], g["gu_g"], g["offsets"], m_total=M, a_rows=g["src"],
                             epilogue=m.EPI_F32, b_packed=g["gu_p"])
    torch.cuda.synchronize()
    y_ref, absdot = _oracle_y1()
    worst = assert_gemm_close(down(y), y_ref, absdot, what="gate_up f32, all 16384 x 512")
    print(f"gate_up f32: worst |err|/tol {worst:.3g}", flush=True)


def test_whole_gate_up_fused_swiglu():
    # the benchmark's gate_up call: fused SwiGLU + NVFP4 requantisation
    print("whole gate_up + fused SwiGLU (T=2048 Zipf decode shape)", flush=True)
    d, g = _inputs(), _device()
    M = CFG.T * CFG.k
    y_ref, absdot = _oracle_y1()
    h64, hq_ref = _oracle_h()
    g_h = hq_ref[2]
    hq = m.nvfp4_grouped_gemm(g["x"], g["gu_c"], g["gu_s"], g["gu_g"], g["offsets"], m_total=M, a_rows=g["src"],
                              epilogue=m.EPI_SWIGLU_NVFP4, out_g=up(np.array([g_h], np.float32)),
                              b_packed=g["gu_p"])
    torch.cuda.synchronize()
    ns, nc = check_requant(down(hq.codes), down(hq.scales), h64, g_h, _swiglu_tol(y_ref, absdot),
                           max_flip_frac=1e-3, what="fused SwiGLU, all 16384 rows")
    print(f"fused SwiGLU: {ns} block-scale and {nc} code flips in {h64.size} values", flush=True)


def test_whole_gate_up_fused_swiglu_exact_accumulation():
    # constant block scales and power-of-two per-tensor scales: every FP32
    # partial sum is exact in any order, so y1 is identical on both sides and
    # the requantised h may differ only through silu's float32 rounding: a flip
    # is accepted only within 1e-6 relative of a decision point
    print("whole fused SwiGLU, exact accumulation (T=2048 Zipf decode shape)", flush=True)
    d = _inputs()
    c = CFG
    M = c.T * c.k
    xc, xs = workloads.nvfp4_codes(c, 2, (c.T,), c.H, const_scale=0x18)         # x scales 2^-4
    bc = d["gu"][0]
    bs = np.full(bc.shape[:2] + (c.H // 16,), 0x18, np.uint8)                     # weight scales 2^-4
    ones = np.ones(c.E, np.float32)
    y1, _ = OM.grouped_gemm(xc, xs, 1.0, bc, bs, ones, d["offsets"], a_rows=d["src"], want_absdot=False)
    h64 = OM.swiglu(y1)
    g_h = np.float32(np.float32(np.abs(h64.astype(np.float32)).max()) / np.float32(2688.0))
    g = _device()
    bct, bst = g["gu_c"], up(bs)
    x = m.NVFP4Tensor(up(xc), up(xs), up(np.ones(1, np.float32)))
    hq = m.nvfp4_grouped_gemm(x, bct, bst, up(ones), g["offsets"], m_total=M, a_rows=g["src"],
                              epilogue=m.EPI_SWIGLU_NVFP4, out_g=up(np.array([g_h], np.float32)),
                              b_packed=m.nvfp4_weight_repack(bct, bst))
    # the same accumulators through the float32 epilogue must equal the oracle's y1 bit for bit
    y = m.nvfp4_grouped_gemm(x, bct, bst, up(ones), g["offsets"], m_total=M, a_rows=g["src"],
                             epilogue=m.EPI_F32, b_packed=m.nvfp4_weight_repack(bct, bst))
    torch.cuda.synchronize()
    assert np.array_equal(down(y), y1)
    ns, nc = check_requant(down(hq.codes), down(hq.scales), h64, g_h, 1e-6 * np.abs(h64), max_flip_frac=1.0,
                           what="fused SwiGLU, exact y1")
    print(f"fused SwiGLU exact: {ns} block-scale and {nc} code flips in {h64.size} values", flush=True)


def test_whole_down_bf16():
    # the benchmark's down call (stream-N kernel, bf16 rows) on the oracle's h
    print("whole down bf16 (T=2048 Zipf decode shape)", flush=True)
    d, g = _inputs(), _device()
    M = CFG.T * CFG.k
    _, (hc, hs, g_h) = _oracle_h()
    hq = m.NVFP4Tensor(up(hc), up(hs), up(np.array([g_h], np.float32)))
    y2 = m.nvfp4_grouped_gemm(hq, g["dn_c"], g["dn_s"], g["dn_g"], g["offsets"], m_total=M,
                              epilogue=m.EPI_BF16, b_packed=g["dn_p"])
    torch.cuda.synchronize()
    y_ref, absdot = _oracle_y2()
    worst = assert_gemm_close(bf16_to_f32(y2), y_ref, absdot, bf16_out=True, what="down bf16, all 16384 x 6144")
    print(f"down bf16: worst |err|/tol {worst:.3g}", flush=True)


def test_whole_combine():
    print("whole combine (T=2048 Zipf decode shape)", flush=True)
    d, g = _inputs(), _device()
    y_ref, _ = _oracle_y2()
    y_bf = workloads.to_bf16_values(y_ref)
    out = m.moe_unpermute_combine(up(y_bf).to(torch.bfloat16), g["perm_of"], g["w"], CFG.T, CFG.k)
    torch.cuda.synchronize()
    ref64, _ = OM.combine(y_bf, d["perm_of"], d["w"])
    w = np.abs(d["w"].astype(np.float64))
    rows = np.abs(y_bf.astype(np.float64))[d["perm_of"].reshape(CFG.T, CFG.k)]
    bound = CFG.k * 2.0 ** -23 * np.einsum("tj,tjh->th", w, rows) + 2.0 ** -8 * np.abs(ref64) + 1e-30
    err = np.abs(bf16_to_f32(out) - ref64)
    assert np.all(err <= bound), f"combine: {int((err > bound).sum())} of {err.size} outside the bound"
