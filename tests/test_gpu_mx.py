"""GPU parity of the MXFP4 variant (mxfp4_quantize, mxfp4_grouped_gemm on
gfx950's block-scaled FP4 MFMA) against the MXFP4 oracle: quantiser bit for
bit, GEMM within 1e-3 sum|a^ b^| + 1e-6 (bf16 out: + 2^-8 |y|), bit for bit
where the float32 sum is order-free (one scale per operand), the fused SwiGLU +
MXFP4 requantisation code by code (flips only next to a decision point within
the propagated tolerance), and whole outputs at the Zipf decode gate_up and
down shapes.  Every GPU stage is fed the oracle's inputs."""
import numpy as np
import pytest
import torch

import block_scaled_fp4_permute_amd as m
import workloads
from oracle import moe as OM
from oracle import mx as MX
from tests.gpu_common import DEV, assert_gemm_close, bf16_to_f32, check_requant_mx, down, up

pytestmark = pytest.mark.gpu


def _mx_up(codes, scales):
    return m.MXFP4Tensor(up(codes), up(scales))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rows,cols", [(1, 32), (37, 256), (300, 6144)])
def test_mx_quantize_bit_exact(dtype, rows, cols):
    print(f"mx quantize {dtype} {rows}x{cols}", flush=True)
    rng = np.random.default_rng(rows + cols)
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    x *= np.exp2(rng.integers(-40, 40, (rows, cols // 32))).repeat(32, axis=1).astype(np.float32)
    x[0, :32] = -0.0                                  # a zero block of negative zeros
    if cols >= 64:
        x[0, 32] = -0.0
        x[0, 33:64] = 2.0 ** rng.integers(-5, 5, 31)   # powers of two: absmax on a scale boundary
    if dtype == "bf16":
        x = workloads.to_bf16_values(x)
    xt = up(x).to(torch.bfloat16) if dtype == "bf16" else up(x)
    q = m.mxfp4_quantize(xt)
    torch.cuda.synchronize()
    c_ref, s_ref = MX.mx_quantize(x)
    assert np.array_equal(down(q.scales), s_ref)
    assert np.array_equal(down(q.codes), c_ref)


def test_mx_quantize_decision_points():
    # values exactly on, and one float32 ulp either side of, every E2M1
    # decision point, under several shared exponents
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    vals = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(10))])
    rows = []
    for X in (-20, -3, 0, 7, 60):
        blk = np.zeros(32, np.float32)
        blk[0] = np.float32(4.0)                      # absmax 4 * 2^X: shared exponent X
        blk[1:1 + len(vals)] = vals
        blk[1 + len(vals):] = -vals[: 31 - len(vals)]
        rows.append(blk * np.float32(2.0 ** X))
    x = np.stack(rows)
    q = m.mxfp4_quantize(up(x))
    torch.cuda.synchronize()
    c_ref, s_ref = MX.mx_quantize(x)
    assert np.array_equal(down(q.scales), s_ref) and np.array_equal(down(q.codes), c_ref)


def _rand_mx(rng, shape_rows, K, lo=118, hi=136):
    codes = rng.integers(0, 256, shape_rows + (K // 2,), dtype=np.uint8)
    scales = rng.integers(lo, hi, shape_rows + (K // 32,), dtype=np.uint8)
    return codes, scales


CASES = [
    # E, counts, N, K, rows_a, hint
    (3, [5, 0, 17], 64, 256, 30, 0),
    (4, [1, 100, 64, 65], 48, 512, 300, 0),
    (2, [200, 3], 512, 6144, 203, 0),
    (8, [16, 31, 33, 64, 2, 0, 129, 8], 160, 256, 283, 100),
    (600, None, 64, 512, 500, 0),
    (3, [9, 40, 2], 48, 32, 60, 0),           # K below one step: one block per row
    (4, [20, 0, 70, 5], 64, 96, 100, 0),      # partial step, half a lane's blocks past K
    (2, [33, 80], 80, 416, 120, 0),           # one full step and a partial one
]


def _unpack_mx_tiles(packed, E, N, K):
    """Inverse of the documented MXFP4 tile layout (tile (e, rt, st) of 2176
    bytes; lane l = 16 g + n: row 16 rt + n, code bytes of blocks 2g, 2g+1 of
    the step at [16 l, +16) and [1024 + 16 l, +16), scale bytes at [2048 + 2 l, +2))."""
    ntr, nst = (N + 15) // 16, (K + 255) // 256
    t = np.asarray(packed, np.uint8)[: E * ntr * nst * 2176].reshape(E, ntr, nst, 2176)
    codes = np.zeros((E, ntr * 16, nst * 128), np.uint8)
    scales = np.zeros((E, ntr * 16, nst * 8), np.uint8)
    for l in range(64):
        n, g = l % 16, l // 16
        rows = np.arange(ntr) * 16 + n
        for st in range(nst):
            codes[:, rows, 128 * st + 32 * g: 128 * st + 32 * g + 16] = t[:, :, st, 16 * l: 16 * l + 16]
            codes[:, rows, 128 * st + 32 * g + 16: 128 * st + 32 * g + 32] = t[:, :, st, 1024 + 16 * l: 1024 + 16 * l + 16]
            scales[:, rows, 8 * st + 2 * g: 8 * st + 2 * g + 2] = t[:, :, st, 2048 + 2 * l: 2048 + 2 * l + 2]
    return codes, scales


@pytest.mark.parametrize("E,N,K", [(3, 48, 288), (1, 16, 32), (2, 512, 6144)])
def test_mx_weight_repack_layout(E, N, K):
    rng = np.random.default_rng(E * N + K)
    codes = rng.integers(0, 256, (E, N, K // 2), dtype=np.uint8)
    scales = rng.integers(0, 255, (E, N, K // 32), dtype=np.uint8)
    packed = down(m.mxfp4_weight_repack(_mx_up(codes, scales)))
    torch.cuda.synchronize()
    assert packed.size == m.lib().mxfp4_weight_packed_size(E, N, K)
    uc, us = _unpack_mx_tiles(packed, E, N, K)
    assert np.array_equal(uc[:, :N, :K // 2], codes) and np.array_equal(us[:, :N, :K // 32], scales)
    assert not uc[:, N:].any() and not uc[:, :, K // 2:].any()
    assert np.all(us[:, :, K // 32:] == 127) and np.all(us[:, N:] == 127)     # neutral scale in the padding


# hint (or the average) of at least 256 rows per expert, K a multiple of 256
# and packed weights: the 256 x 256 tile with both operands staged in LDS
LARGE_CASES = [
    # E, counts, N, K, rows_a, hint
    (3, [300, 0, 517], 320, 512, 400, 256),          # a partial column tile, an empty expert
    (1, [600], 512, 2048, 600, 0),                   # by the average; a partial row chunk
    (5, [256, 1, 1000, 0, 255], 256, 768, 700, 300),  # 1-row and 255-row experts, 4 chunks in one group
]


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("gather", [False, True])
@pytest.mark.parametrize("epi", ["f32", "bf16"])
@pytest.mark.parametrize("packed", [False, True])
def test_mx_gemm_random(case, gather, epi, packed):
    _run_mx_case(CASES[case], 200 + case, gather, epi, packed, f"case {case}")


@pytest.mark.parametrize("case", range(len(LARGE_CASES)))
@pytest.mark.parametrize("gather", [False, True])
@pytest.mark.parametrize("epi", ["f32", "bf16"])
def test_mx_gemm_large_tile(case, gather, epi):
    _run_mx_case(LARGE_CASES[case], 300 + case, gather, epi, True, f"large case {case}")


def _run_mx_case(spec, seed, gather, epi, packed, name):
    E, counts, N, K, rows_a, hint = spec
    rng = np.random.default_rng(seed)
    if counts is None:
        counts = rng.integers(0, 40, E) * (rng.random(E) < 0.7)
        counts[rng.choice(E, 4, replace=False)] = [150, 200, 65, 17]
    counts = np.asarray(counts, np.int64)
    M = int(counts.sum())
    print(f"mx gemm {name} gather={gather} epi={epi} packed={packed} E={E} M={M} N={N} K={K} hint={hint}", flush=True)
    if not gather:
        rows_a = max(M, 1)                     # row p of the GEMM reads A row p
    ac, as_ = _rand_mx(rng, (rows_a,), K)
    bc, bs = _rand_mx(rng, (E, N), K)
    a_rows = rng.integers(0, rows_a, M).astype(np.int32) if gather else None
    b_g = rng.uniform(0.5, 2.0, E).astype(np.float32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    b_t = _mx_up(bc, bs)
    y = m.mxfp4_grouped_gemm(_mx_up(ac, as_), b_t, up(offsets), m_total=M,
                             a_rows=None if a_rows is None else up(a_rows),
                             epilogue=m.EPI_F32 if epi == "f32" else m.EPI_BF16, a_g=up(np.array([0.75], np.float32)),
                             b_g=up(b_g), max_rows_per_expert_hint=hint,
                             b_packed=m.mxfp4_weight_repack(b_t) if packed else None)
    torch.cuda.synchronize()
    y_ref, absdot = MX.mx_grouped_gemm(ac, as_, bc, bs, offsets, a_rows=a_rows, a_g=0.75, b_g=b_g)
    got = down(y) if epi == "f32" else bf16_to_f32(y)
    assert_gemm_close(got, y_ref, absdot, bf16_out=epi == "bf16", what=f"mx {name} {epi}")


@pytest.mark.parametrize("K,large", [(256, False), (2048, False), (8192, False), (256, True), (512, True), (8192, True)])
def test_mx_gemm_constant_scales_bit_exact(K, large):
    # one scale per operand: every float32 partial sum is an exact multiple of
    # 0.25 * 2^(Xa + Xb), so the GPU must equal the oracle bit for bit
    rng = np.random.default_rng(K + large)
    E, counts, N = (2, [300, 520], 272) if large else (2, [37, 70], 80)
    M = sum(counts)
    ac = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    bc = rng.integers(0, 256, (E, N, K // 2), dtype=np.uint8)
    as_ = np.full((M, K // 32), 124, np.uint8)
    bs = np.full((E, N, K // 32), 129, np.uint8)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    b_t = _mx_up(bc, bs)
    y = m.mxfp4_grouped_gemm(_mx_up(ac, as_), b_t, up(offsets), m_total=M,
                             b_packed=m.mxfp4_weight_repack(b_t) if large else None)
    torch.cuda.synchronize()
    y_ref, _ = MX.mx_grouped_gemm(ac, as_, bc, bs, offsets)
    assert np.array_equal(down(y), y_ref)


@pytest.mark.parametrize("large", [False, True])
def test_mx_gemm_scale_per_block_single_term(large):
    # one nonzero 32-block per row pair at a time: each output is one exact
    # block term, so the per-lane scale selection (two blocks per lane, op_sel
    # picking the byte) must put every scale on its own block; large: 300 rows
    # and two K steps through the 256 x 256 tile (packed weights), whose A
    # blocks sit in LDS under a lane swizzle
    rng = np.random.default_rng(5)
    M, N, K = (300, 48, 512) if large else (16, 16, 256)
    for blk in range(K // 32):
        ac = np.zeros((M, K // 2), np.uint8)
        bc = np.zeros((1, N, K // 2), np.uint8)
        ac[:, 16 * blk:16 * blk + 16] = rng.integers(0, 256, (M, 16), dtype=np.uint8)
        bc[0, :, 16 * blk:16 * blk + 16] = rng.integers(0, 256, (N, 16), dtype=np.uint8)
        as_ = rng.integers(100, 150, (M, K // 32), dtype=np.uint8)
        bs = rng.integers(100, 150, (1, N, K // 32), dtype=np.uint8)
        offsets = np.array([0, M], np.int32)
        b_t = _mx_up(bc, bs)
        y = m.mxfp4_grouped_gemm(_mx_up(ac, as_), b_t, up(offsets), m_total=M,
                                 b_packed=m.mxfp4_weight_repack(b_t) if large else None)
        torch.cuda.synchronize()
        y_ref, _ = MX.mx_grouped_gemm(ac, as_, bc, bs, offsets)
        assert np.array_equal(down(y), y_ref), f"block {blk}"


def _swiglu_tol(y1, absdot):
    I = y1.shape[1] // 2
    tol_y = 1e-3 * absdot + 1e-6
    g, u = y1[:, :I].astype(np.float64), y1[:, I:].astype(np.float64)
    silu = OM.silu(g)
    return 1.1 * tol_y[:, :I] * np.abs(u) + np.abs(silu) * tol_y[:, I:] + 2.0 ** -20 * np.abs(silu * u) + 1e-9


@pytest.mark.parametrize("hint", [0, 100])
def test_mx_fused_swiglu(hint):
    rng = np.random.default_rng(31 + hint)
    E, counts, I, K = 4, [19, 45, 0, 130], 128, 512
    M = sum(counts)
    ac, as_ = _rand_mx(rng, (200,), K)
    bc, bs = _rand_mx(rng, (E, 2 * I), K)
    a_rows = rng.integers(0, 200, M).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    hq = m.mxfp4_grouped_gemm(_mx_up(ac, as_), _mx_up(bc, bs), up(offsets), m_total=M, a_rows=up(a_rows),
                              epilogue=m.EPI_SWIGLU_NVFP4, max_rows_per_expert_hint=hint)
    torch.cuda.synchronize()
    y1, absdot = MX.mx_grouped_gemm(ac, as_, bc, bs, offsets, a_rows=a_rows)
    _, _, h64 = MX.mx_swiglu_quantize(y1)
    check_requant_mx(down(hq.codes), down(hq.scales), h64, _swiglu_tol(y1, absdot), max_flip_frac=0.02,
                     what="mx fused swiglu")


def test_mx_fused_swiglu_large_tile():
    # 256 x 256 tiles (128 h columns each): I = 192 leaves the second h tile
    # half empty; a gathered A
    rng = np.random.default_rng(37)
    E, counts, I, K = 3, [260, 40, 700], 192, 1024
    M = sum(counts)
    ac, as_ = _rand_mx(rng, (900,), K)
    bc, bs = _rand_mx(rng, (E, 2 * I), K)
    a_rows = rng.integers(0, 900, M).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    b_t = _mx_up(bc, bs)
    hq = m.mxfp4_grouped_gemm(_mx_up(ac, as_), b_t, up(offsets), m_total=M, a_rows=up(a_rows),
                              epilogue=m.EPI_SWIGLU_NVFP4, max_rows_per_expert_hint=256,
                              b_packed=m.mxfp4_weight_repack(b_t))
    torch.cuda.synchronize()
    y1, absdot = MX.mx_grouped_gemm(ac, as_, bc, bs, offsets, a_rows=a_rows)
    _, _, h64 = MX.mx_swiglu_quantize(y1)
    check_requant_mx(down(hq.codes), down(hq.scales), h64, _swiglu_tol(y1, absdot), max_flip_frac=0.02,
                     what="mx fused swiglu, large tile")


def test_mx_dense_8192_sampled_rows():
    # the dense M = N = K = 8192 GEMM in the launch the benchmark times (large
    # tile, packed weights, bf16 out), checked on 24 sampled rows, every column
    rng = np.random.default_rng(8192)
    M = N = K = 8192
    print("mx dense 8192^3 sampled rows", flush=True)
    ac, as_ = _rand_mx(rng, (M,), K)
    bc, bs = _rand_mx(rng, (1, N), K)
    b_t = _mx_up(bc, bs)
    offsets = np.array([0, M], np.int32)
    y = m.mxfp4_grouped_gemm(_mx_up(ac, as_), b_t, up(offsets), m_total=M, epilogue=m.EPI_BF16,
                             b_packed=m.mxfp4_weight_repack(b_t))
    torch.cuda.synchronize()
    rows = np.sort(rng.choice(M, 24, replace=False))
    rows[0], rows[-1] = 0, M - 1
    got = bf16_to_f32(y[torch.as_tensor(rows, device=y.device)])
    y_ref, absdot = MX.mx_grouped_gemm(ac[rows], as_[rows], bc, bs, np.array([0, len(rows)], np.int32))
    assert_gemm_close(got, y_ref, absdot, bf16_out=True, what="mx dense 8192^3, sampled rows")


def test_mx_fused_swiglu_exact_accumulation():
    # one scale per operand: y1 is identical on both sides, h differs only by
    # silu's float32 rounding: flips only within 1e-6 relative of a decision point
    rng = np.random.default_rng(33)
    E, counts, I, K = 3, [40, 7, 90], 256, 1024
    M = sum(counts)
    ac = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    bc = rng.integers(0, 256, (E, 2 * I, K // 2), dtype=np.uint8)
    as_ = np.full((M, K // 32), 123, np.uint8)
    bs = np.full((E, 2 * I, K // 32), 123, np.uint8)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    hq = m.mxfp4_grouped_gemm(_mx_up(ac, as_), _mx_up(bc, bs), up(offsets), m_total=M,
                              epilogue=m.EPI_SWIGLU_NVFP4)
    torch.cuda.synchronize()
    y1, _ = MX.mx_grouped_gemm(ac, as_, bc, bs, offsets, want_absdot=False)
    _, _, h64 = MX.mx_swiglu_quantize(y1)
    ns, nc = check_requant_mx(down(hq.codes), down(hq.scales), h64, 1e-6 * np.abs(h64), max_flip_frac=1.0,
                              what="mx fused swiglu exact")
    print(f"mx swiglu exact: {ns} scale and {nc} code flips", flush=True)


def test_mx_whole_decode_gate_up_and_down():
    # the Zipf decode shape (T=2048, H=6144, I=256, E=256, top-8): every output
    # of the MXFP4 gate_up (f32 and fused SwiGLU) and down (bf16, on the
    # oracle's h), weights as seeded MXFP4 bytes, x quantised by the oracle
    c = workloads.CONFIGS[2]
    print("mx whole decode shape", flush=True)
    ids, w = OM.route(workloads.logits(c), c.k)
    counts, offsets, src, perm_of, pw = OM.permute(ids, w, c.E)
    M = c.T * c.k
    xc, xs = MX.mx_quantize(workloads.activations(c))
    guc, gus = workloads.nvfp4_codes(c, 3, (c.E, 2 * c.I), c.H, scale_lo=116, scale_hi=124, block=32)
    dnc, dns = workloads.nvfp4_codes(c, 4, (c.E, c.H), c.I, scale_lo=116, scale_hi=124, block=32)
    x_t, gu_t, dn_t = _mx_up(xc, xs), _mx_up(guc, gus), _mx_up(dnc, dns)
    gu_p, dn_p = m.mxfp4_weight_repack(gu_t), m.mxfp4_weight_repack(dn_t)
    off_t, src_t = up(offsets), up(src)
    y1g = m.mxfp4_grouped_gemm(x_t, gu_t, off_t, m_total=M, a_rows=src_t, b_packed=gu_p)
    hq = m.mxfp4_grouped_gemm(x_t, gu_t, off_t, m_total=M, a_rows=src_t, epilogue=m.EPI_SWIGLU_NVFP4, b_packed=gu_p)
    torch.cuda.synchronize()
    y1, ad1 = MX.mx_grouped_gemm(xc, xs, guc, gus, offsets, a_rows=src)
    assert_gemm_close(down(y1g), y1, ad1, what="mx gate_up f32, all 16384 x 512")
    hc_ref, hs_ref, h64 = MX.mx_swiglu_quantize(y1)
    check_requant_mx(down(hq.codes), down(hq.scales), h64, _swiglu_tol(y1, ad1), max_flip_frac=1e-3,
                     what="mx fused swiglu, all 16384 rows")
    y2g = m.mxfp4_grouped_gemm(_mx_up(hc_ref, hs_ref), dn_t, off_t, m_total=M, epilogue=m.EPI_BF16, b_packed=dn_p)
    torch.cuda.synchronize()
    y2, ad2 = MX.mx_grouped_gemm(hc_ref, hs_ref, dnc, dns, offsets)
    assert_gemm_close(bf16_to_f32(y2g), y2, ad2, bf16_out=True, what="mx down bf16, all 16384 x 6144")


@pytest.mark.parametrize("cfg_index", [0, 1])
def test_mx_layer_end_to_end(cfg_index):
    # MXMoELayer (the composition the MXFP4 bench times) against the oracle's
    # stages composed the same way; h values the GPU rounded the other way at
    # a decision point are first checked to be valid roundings, and the output
    # tolerance then carries their exact bound on the down GEMM
    from block_scaled_fp4_permute_amd.layer import MXMoELayer, quantize_expert_weights_mx
    c = workloads.CONFIGS[cfg_index]
    print(f"mx layer end to end cfg={cfg_index}", flush=True)
    logits, x = workloads.logits(c), workloads.activations(c)
    w_gu, w_dn = workloads.torch_expert_weights(c, DEV)
    wq = quantize_expert_weights_mx(w_gu, w_dn)
    layer = MXMoELayer(c.T, c.H, c.I, c.E, c.k, DEV)
    out = layer.forward(up(logits), up(x).to(torch.bfloat16), wq)
    torch.cuda.synchronize()
    ids, w = OM.route(logits, c.k)
    counts, offsets, src, perm_of, pw = OM.permute(ids, w, c.E)
    assert np.array_equal(down(layer.routing.perm_src_token), src)
    xc, xs = MX.mx_quantize(x)
    assert np.array_equal(down(layer.xq.codes), xc) and np.array_equal(down(layer.xq.scales), xs)
    gq = MX.mx_quantize(w_gu.reshape(-1, c.H).cpu().numpy())
    dq = MX.mx_quantize(w_dn.reshape(-1, c.I).cpu().numpy())
    gc, gs = gq[0].reshape(c.E, 2 * c.I, -1), gq[1].reshape(c.E, 2 * c.I, -1)
    dc, ds = dq[0].reshape(c.E, c.H, -1), dq[1].reshape(c.E, c.H, -1)
    assert np.array_equal(down(wq.gu.codes), gc) and np.array_equal(down(wq.dn.scales), ds)
    y1, ad1 = MX.mx_grouped_gemm(xc, xs, gc, gs, offsets, a_rows=src)
    hc, hs, h64 = MX.mx_swiglu_quantize(y1)
    hc_gpu, hs_gpu = down(layer.hq.codes), down(layer.hq.scales)
    check_requant_mx(hc_gpu, hs_gpu, h64, _swiglu_tol(y1, ad1), max_flip_frac=0.02, what="mx layer h")
    y2, ad2 = MX.mx_grouped_gemm(hc, hs, dc, ds, offsets)
    dh = np.abs(MX.mx_dequantize(hc_gpu, hs_gpu) - MX.mx_dequantize(hc, hs))
    tol_rows = 1e-3 * ad2 + 1e-6 + 2.0 ** -8 * np.abs(y2.astype(np.float64))
    for e in range(c.E):
        p0, p1 = int(offsets[e]), int(offsets[e + 1])
        if p1 > p0 and dh[p0:p1].any():
            tol_rows[p0:p1] += 1.001 * dh[p0:p1] @ np.abs(MX.mx_dequantize(dc[e], ds[e])).T
    out64, _ = OM.combine(y2, perm_of, w)
    tol = np.einsum("tj,tjh->th", np.abs(w.astype(np.float64)), tol_rows[perm_of.reshape(c.T, c.k)])
    tol = tol * (1 + 2.0 ** -8) + 2.0 ** -8 * np.abs(out64) + 1e-6
    err = np.abs(bf16_to_f32(out) - out64)
    assert np.all(err <= tol), f"mx layer: {int((err > tol).sum())} outputs outside tolerance"
