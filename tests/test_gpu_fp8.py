"""GPU parity of the FP8 block-scaled variant (fp8_quantize, fp8_weight_repack,
fp8_grouped_gemm on gfx950's FP8 MFMA with float32 block scales) against the
FP8 oracle: the quantiser bit for bit (1 x 128 and 128 x 128 blocks, ragged
row blocks, decision points, the subnormal range), the packed tile layout
byte for byte, the GEMM within 1e-3 sum|a^ b^| + 1e-6 (bf16 out: + 2^-8 |y|),
bit for bit where every float32 sum is exact, within two float32 ulps where
each output is a single block term (which pins each block's pair of scales),
whole outputs at the Zipf decode gate_up and down shapes, the SwiGLU + FP8
requantisation code by code (flips only next to a decision point), and the
FP8 layer (routing, permutation and combine of the NVFP4 path) end to end.  Every GPU
stage is fed the oracle's inputs or seeded raw bytes."""
import numpy as np
import pytest
import torch

import block_scaled_fp4_permute_amd as m
import workloads
from oracle import fp8 as F8
from oracle import moe as OM
from tests.gpu_common import DEV, assert_gemm_close, bf16_to_f32, check_requant_fp8, down, up

pytestmark = pytest.mark.gpu


def _a(codes, scales):
    return m.FP8Tensor(up(codes), up(scales), 1)


def _ragged_values(rng, rows, cols):
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    x *= np.exp2(rng.integers(-30, 30, (rows, cols // 128))).repeat(128, axis=1).astype(np.float32)
    x[0, :128] = -0.0                                   # a zero block of negative zeros
    if cols >= 256:
        x[0, 128:256] *= np.float32(2.0 ** -20)         # tiny block: codes in E4M3's subnormal range
        x[0, 130] = np.float32(3.0)                     # ... with one large value
    return x


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rows,cols", [(1, 128), (37, 256), (300, 6144)])
def test_fp8_quantize_rows_bit_exact(dtype, rows, cols):
    print(f"fp8 quantize 1x128 {dtype} {rows}x{cols}", flush=True)
    rng = np.random.default_rng(rows * 7 + cols)
    x = _ragged_values(rng, rows, cols)
    if dtype == "bf16":
        x = workloads.to_bf16_values(x)
    xt = up(x).to(torch.bfloat16) if dtype == "bf16" else up(x)
    q = m.fp8_quantize(xt, 1)
    torch.cuda.synchronize()
    c_ref, s_ref = F8.fp8_quantize(x, 1)
    assert np.array_equal(down(q.scales), s_ref)
    assert np.array_equal(down(q.codes), c_ref)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("E,N,K", [(1, 128, 128), (3, 200, 384), (2, 16, 256), (4, 512, 1024)])
def test_fp8_quantize_tiles_bit_exact(dtype, E, N, K):
    print(f"fp8 quantize 128x128 {dtype} E={E} N={N} K={K}", flush=True)
    rng = np.random.default_rng(E * 1000 + N + K)
    w = np.stack([_ragged_values(rng, N, K) for _ in range(E)])
    if dtype == "bf16":
        w = workloads.to_bf16_values(w)
    wt = up(w).to(torch.bfloat16) if dtype == "bf16" else up(w)
    q = m.fp8_quantize(wt, 128)
    torch.cuda.synchronize()
    for e in range(E):
        c_ref, s_ref = F8.fp8_quantize(w[e], 128)
        assert np.array_equal(down(q.scales[e]), s_ref), f"scales of matrix {e}"
        assert np.array_equal(down(q.codes[e]), c_ref), f"codes of matrix {e}"


def test_fp8_quantize_decision_points():
    # blocks with absmax 448 * 2^k (so s = 2^k exactly and every quotient is
    # exact), holding every E4M3 midpoint and its float32 neighbours, in the
    # normal and subnormal ranges
    pos = np.array(sorted({float(v) for v in F8.e4m3_decode(np.arange(0x7F, dtype=np.uint8))}))
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    vals = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9))])
    vals = vals[vals < 448]
    per = 127
    nblk = (len(vals) + per - 1) // per
    rows = []
    for k in (-20, -3, 0, 5):
        for b in range(nblk):
            blk = np.zeros(128, np.float32)
            blk[0] = np.float32(448.0)
            chunk = vals[b * per:(b + 1) * per]
            blk[1:1 + len(chunk)] = chunk * np.where(np.arange(len(chunk)) % 2 == 0, 1, -1).astype(np.float32)
            rows.append(blk * np.float32(2.0 ** k))
    x = np.stack(rows)
    q = m.fp8_quantize(up(x), 1)
    torch.cuda.synchronize()
    c_ref, s_ref = F8.fp8_quantize(x, 1)
    assert np.array_equal(down(q.scales), s_ref) and np.array_equal(down(q.codes), c_ref)


def _unpack_fp8_tiles(packed, E, N, K):
    """Inverse of the documented FP8 tile layout (tile (e, rt, st) of 2048
    bytes; lane l = 16 g + n: row 16 rt + n, K bytes [128 st + 32 g, +16) at
    [16 l, +16) and the next 16 at [1024 + 16 l, +16))."""
    ntr, nst = (N + 15) // 16, K // 128
    t = np.asarray(packed, np.uint8)[: E * ntr * nst * 2048].reshape(E, ntr, nst, 2048)
    codes = np.zeros((E, ntr * 16, K), np.uint8)
    for l in range(64):
        n, g = l % 16, l // 16
        r = np.arange(ntr) * 16 + n
        for st in range(nst):
            k0 = 128 * st + 32 * g
            codes[:, r, k0:k0 + 16] = t[:, :, st, 16 * l:16 * l + 16]
            codes[:, r, k0 + 16:k0 + 32] = t[:, :, st, 1024 + 16 * l:1024 + 16 * l + 16]
    return codes


@pytest.mark.parametrize("E,N,K", [(3, 48, 384), (1, 16, 128), (2, 512, 6144)])
def test_fp8_weight_repack_layout(E, N, K):
    rng = np.random.default_rng(E * N + K)
    codes = rng.integers(0, 256, (E, N, K), dtype=np.uint8)
    packed = down(m.fp8_weight_repack(up(codes)))
    torch.cuda.synchronize()
    assert packed.size == m.lib().fp8_weight_packed_size(E, N, K)
    assert np.array_equal(_unpack_fp8_tiles(packed, E, N, K)[:, :N], codes)


CASES = [
    # E, counts, N, K, rows_a, hint
    (3, [5, 0, 17], 64, 256, 30, 0),
    (4, [1, 100, 64, 65], 48, 512, 300, 0),
    (2, [200, 3], 512, 6144, 203, 0),
    (8, [16, 31, 33, 64, 2, 0, 129, 8], 160, 256, 283, 100),
    (600, None, 64, 512, 500, 0),
    (3, [9, 40, 2], 48, 128, 60, 0),          # one K step
    (2, [33, 80], 400, 384, 120, 0),          # odd step count, N past one weight block and not a multiple of 64
    # K <= 256 below 256 rows per expert: the stream-N kernel; 6160 columns are
    # 97 units of 64 (the last one 16 wide) over five workgroup column groups
    (4, [1, 64, 0, 37], 6160, 256, 110, 0),
    (3, [70, 2, 129], 6160, 128, 210, 64),    # one K step, cached weight loads
]


def _fp8_operands(cfg_stream, E, N, K, rows_a):
    c = workloads.CONFIGS[0]
    ac = workloads.fp8_codes(c, cfg_stream, (rows_a, K))
    as_ = workloads.fp8_scales(c, cfg_stream, (rows_a, K // 128), 2.0 ** -4, 2.0 ** 4)
    bc = workloads.fp8_codes(c, cfg_stream + 1, (E, N, K))
    bs = workloads.fp8_scales(c, cfg_stream + 1, (E, (N + 127) // 128, K // 128), 2.0 ** -4, 2.0 ** 4)
    return ac, as_, bc, bs


# hint (or the average) of at least 256 rows per expert: the 256 x 256 tile
# with both operands staged in LDS
LARGE_CASES = [
    # E, counts, N, K, rows_a, hint
    (3, [300, 0, 517], 400, 384, 400, 256),          # partial column tile past one weight block, odd steps
    (1, [600], 512, 2048, 600, 0),                   # by the average; a partial row chunk
    (5, [256, 1, 1000, 0, 255], 256, 640, 700, 300),  # five K steps; 1-row and 255-row experts
]


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("gather", [False, True])
@pytest.mark.parametrize("epi", ["f32", "bf16"])
def test_fp8_gemm_random(case, gather, epi):
    _run_fp8_case(CASES[case], 300 + case, 10 + 2 * case, gather, epi, f"case {case}")


@pytest.mark.parametrize("case", range(len(LARGE_CASES)))
@pytest.mark.parametrize("gather", [False, True])
@pytest.mark.parametrize("epi", ["f32", "bf16"])
def test_fp8_gemm_large_tile(case, gather, epi):
    _run_fp8_case(LARGE_CASES[case], 400 + case, 70 + 2 * case, gather, epi, f"large case {case}")


def _run_fp8_case(spec, seed, stream, gather, epi, name):
    E, counts, N, K, rows_a, hint = spec
    rng = np.random.default_rng(seed)
    if counts is None:
        counts = rng.integers(0, 40, E) * (rng.random(E) < 0.7)
        counts[rng.choice(E, 4, replace=False)] = [150, 200, 65, 17]
    counts = np.asarray(counts, np.int64)
    M = int(counts.sum())
    print(f"fp8 gemm {name} gather={gather} epi={epi} E={E} M={M} N={N} K={K} hint={hint}", flush=True)
    if not gather:
        rows_a = max(M, 1)
    ac, as_, bc, bs = _fp8_operands(stream, E, N, K, rows_a)
    a_rows = rng.integers(0, rows_a, M).astype(np.int32) if gather else None
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    y = m.fp8_grouped_gemm(_a(ac, as_), m.fp8_weight_repack(up(bc)), up(bs), up(offsets), N=N, m_total=M,
                           a_rows=None if a_rows is None else up(a_rows),
                           epilogue=m.EPI_F32 if epi == "f32" else m.EPI_BF16, max_rows_per_expert_hint=hint)
    torch.cuda.synchronize()
    y_ref, absdot = F8.fp8_grouped_gemm(ac, as_, bc, bs, offsets, a_rows=a_rows)
    got = down(y) if epi == "f32" else bf16_to_f32(y)
    assert_gemm_close(got, y_ref, absdot, bf16_out=epi == "bf16", what=f"fp8 {name} {epi}")


@pytest.mark.parametrize("K,large", [(128, False), (1024, False), (4096, False), (128, True), (4096, True)])
def test_fp8_gemm_exact_sums_bit_exact(K, large):
    # E4M3 values in [1, 3.75] (exponent fields 7 and 8) and block scales 1/2 or
    # 1: every scaled product is a multiple of 2^-8 of magnitude at most 14.07,
    # so any partial sum of at most 4096 of them is below 2^24 units of 2^-8 and
    # exact in float32 in any order: the GPU must equal the oracle bit for bit
    c = workloads.CONFIGS[0]
    E, counts, N = 2, ([300, 520] if large else [37, 70]), 272
    M = sum(counts)
    ac = workloads.fp8_codes(c, 40, (M, K), 7, 9)
    bc = workloads.fp8_codes(c, 41, (E, N, K), 7, 9)
    rng = np.random.default_rng(K)
    as_ = np.exp2(rng.integers(-1, 1, (M, K // 128))).astype(np.float32)
    bs = np.exp2(rng.integers(-1, 1, (E, (N + 127) // 128, K // 128))).astype(np.float32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    y = m.fp8_grouped_gemm(_a(ac, as_), m.fp8_weight_repack(up(bc)), up(bs), up(offsets), N=N, m_total=M)
    torch.cuda.synchronize()
    y_ref, _ = F8.fp8_grouped_gemm(ac, as_, bc, bs, offsets, want_absdot=False)
    assert np.array_equal(down(y), y_ref)


@pytest.mark.parametrize("shape", ["decode", "large", "stream_n"])
def test_fp8_gemm_single_block_term(shape):
    # one nonzero 128-block of K at a time, exact-sum codes, arbitrary float32
    # scales: each output is one block term part * sa * sb, which the GPU rounds
    # twice (sa * sb, then the product) - within two float32 ulps of the
    # oracle's exact term; a scale taken from the wrong row, tile or block is
    # far outside that (large: 300 rows through the 256 x 256 tile, whose A
    # rows and scales sit in LDS; stream_n: K = 256 with 1040 columns, nine
    # weight blocks over 17 streamed units)
    c = workloads.CONFIGS[0]
    M, N, K = {"decode": (80, 272, 512), "large": (300, 272, 512), "stream_n": (80, 1040, 256)}[shape]
    for blk in range(K // 128):
        ac = np.zeros((M, K), np.uint8)
        bc = np.zeros((1, N, K), np.uint8)
        ac[:, 128 * blk:128 * blk + 128] = workloads.fp8_codes(c, 50 + blk, (M, 128), 7, 9)
        bc[0, :, 128 * blk:128 * blk + 128] = workloads.fp8_codes(c, 60 + blk, (N, 128), 7, 9)
        as_ = workloads.fp8_scales(c, 50 + blk, (M, K // 128), 0.1, 10.0)
        bs = workloads.fp8_scales(c, 60 + blk, (1, (N + 127) // 128, K // 128), 0.1, 10.0)
        offsets = np.array([0, M], np.int32)
        y = m.fp8_grouped_gemm(_a(ac, as_), m.fp8_weight_repack(up(bc)), up(bs), up(offsets), N=N, m_total=M)
        torch.cuda.synchronize()
        y_ref, _ = F8.fp8_grouped_gemm(ac, as_, bc, bs, offsets, want_absdot=False)
        got = down(y).astype(np.float64)
        bad = np.abs(got - y_ref) > 2.0 ** -22 * np.abs(y_ref)
        if bad.any():
            i = tuple(np.argwhere(bad)[0])
            raise AssertionError(f"block {blk}: {int(bad.sum())} of {bad.size} outside two ulps; rows "
                                 f"{np.unique(np.argwhere(bad)[:, 0])[:20]} cols {np.unique(np.argwhere(bad)[:, 1])[:20]}; "
                                 f"first {i}: gpu {got[i]!r} ref {float(y_ref[i])!r}")


def test_fp8_dense_8192_sampled_rows():
    # the dense M = N = K = 8192 GEMM in the launch the benchmark times (large
    # tile, bf16 out), checked on 24 sampled rows, every column
    c = workloads.CONFIGS[0]
    M = N = K = 8192
    print("fp8 dense 8192^3 sampled rows", flush=True)
    ac = workloads.fp8_codes(c, 80, (M, K))
    as_ = workloads.fp8_scales(c, 80, (M, K // 128))
    bc = workloads.fp8_codes(c, 81, (1, N, K))
    bs = workloads.fp8_scales(c, 81, (1, N // 128, K // 128))
    offsets = np.array([0, M], np.int32)
    y = m.fp8_grouped_gemm(_a(ac, as_), m.fp8_weight_repack(up(bc)), up(bs), up(offsets), N=N, m_total=M,
                           epilogue=m.EPI_BF16)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(81).choice(M, 24, replace=False))
    rows[0], rows[-1] = 0, M - 1
    got = bf16_to_f32(y[torch.as_tensor(rows, device=y.device)])
    y_ref, absdot = F8.fp8_grouped_gemm(ac[rows], as_[rows], bc, bs, np.array([0, len(rows)], np.int32))
    assert_gemm_close(got, y_ref, absdot, bf16_out=True, what="fp8 dense 8192^3, sampled rows")


def test_fp8_whole_decode_gate_up_and_down():
    # the Zipf decode shape (T=2048, H=6144, I=256, E=256, top-8): every output
    # of the FP8 gate_up (f32) and down (bf16); x and h quantised by the oracle,
    # weights as seeded E4M3 bytes with log-uniform block scales
    c = workloads.CONFIGS[2]
    print("fp8 whole decode shape", flush=True)
    ids, w = OM.route(workloads.logits(c), c.k)
    counts, offsets, src, perm_of, pw = OM.permute(ids, w, c.E)
    M = c.T * c.k
    xc, xs = F8.fp8_quantize(workloads.activations(c), 1)
    guc = workloads.fp8_codes(c, 3, (c.E, 2 * c.I, c.H))
    gus = workloads.fp8_scales(c, 3, (c.E, 2 * c.I // 128, c.H // 128))
    dnc = workloads.fp8_codes(c, 4, (c.E, c.H, c.I))
    dns = workloads.fp8_scales(c, 4, (c.E, c.H // 128, c.I // 128))
    off_t = up(offsets)
    y1g = m.fp8_grouped_gemm(_a(xc, xs), m.fp8_weight_repack(up(guc)), up(gus), off_t, N=2 * c.I, m_total=M,
                             a_rows=up(src))
    torch.cuda.synchronize()
    y1, ad1 = F8.fp8_grouped_gemm(xc, xs, guc, gus, offsets, a_rows=src)
    assert_gemm_close(down(y1g), y1, ad1, what="fp8 gate_up f32, all 16384 x 512")
    del y1g
    hc, hs = F8.fp8_quantize(OM.swiglu(y1).astype(np.float32), 1)
    y2g = m.fp8_grouped_gemm(_a(hc, hs), m.fp8_weight_repack(up(dnc)), up(dns), off_t, N=c.H, m_total=M,
                             epilogue=m.EPI_BF16)
    torch.cuda.synchronize()
    y2, ad2 = F8.fp8_grouped_gemm(hc, hs, dnc, dns, offsets)
    assert_gemm_close(bf16_to_f32(y2g), y2, ad2, bf16_out=True, what="fp8 down bf16, all 16384 x 6144")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fp8_swiglu_quantize(dtype):
    # the oracle's gate_up rows in, h = silu(gate) * up requantised: the two
    # sides differ only by silu's float32 rounding (expf), so a code may flip
    # only within a few ulp of a decision point and a block scale only by
    # the rounding of its absmax
    rng = np.random.default_rng(21)
    M, I = 300, 256
    y1 = (rng.standard_normal((M, 2 * I)) * np.exp2(rng.integers(-6, 6, (M, 1)))).astype(np.float32)
    y1[0, :] = 0.0                                     # a zero row: h = 0, scale 1
    if dtype == "bf16":
        y1 = workloads.to_bf16_values(y1)
    yt = up(y1).to(torch.bfloat16) if dtype == "bf16" else up(y1)
    hq = m.fp8_swiglu_quantize(yt)
    torch.cuda.synchronize()
    _, _, h64 = F8.fp8_swiglu_quantize(y1)
    ns, nc = check_requant_fp8(down(hq.codes), down(hq.scales), h64, 2.0 ** -20 * np.abs(h64) + 1e-30,
                               max_flip_frac=1e-3, what="fp8 swiglu")
    assert down(hq.scales)[0].tolist() == [1.0, 1.0] and not down(hq.codes)[0].any()
    print(f"fp8 swiglu {dtype}: {ns} scale and {nc} code differences", flush=True)


# gate_up with SwiGLU + FP8 requant fused into its epilogue against the two
# calls it replaces (float32 rows, then fp8_swiglu_quantize): the same block
# sums in the same order, the same silu and block scale, so the same bits
SWIGLU_CASES = [
    # E, counts, I, K, rows_a, hint
    (3, [5, 0, 17], 128, 256, 30, 0),
    (4, [1, 100, 64, 65], 256, 512, 300, 0),
    (8, [16, 31, 33, 64, 2, 0, 129, 8], 384, 384, 283, 100),   # three h blocks, an odd step count
    (600, None, 128, 256, 500, 0),                              # many experts, several expert groups
    (2, [200, 3], 256, 6144, 203, 40),                          # the decode K, non-temporal loads
    (3, [300, 0, 517], 128, 256, 400, 512),                     # a large hint: still the decode tile
]


@pytest.mark.parametrize("case", range(len(SWIGLU_CASES)))
@pytest.mark.parametrize("gather", [False, True])
def test_fp8_fused_swiglu_matches_separate(case, gather):
    E, counts, I, K, rows_a, hint = SWIGLU_CASES[case]
    rng = np.random.default_rng(500 + case)
    if counts is None:
        counts = rng.integers(0, 40, E) * (rng.random(E) < 0.7)
        counts[rng.choice(E, 4, replace=False)] = [150, 200, 65, 17]
    counts = np.asarray(counts, np.int64)
    M = int(counts.sum())
    N = 2 * I
    print(f"fp8 fused swiglu case {case} gather={gather} E={E} M={M} I={I} K={K} hint={hint}", flush=True)
    if not gather:
        rows_a = max(M, 1)
    ac, as_, bc, bs = _fp8_operands(40 + 2 * case, E, N, K, rows_a)
    a_rows = up(rng.integers(0, rows_a, M).astype(np.int32)) if gather else None
    offsets = up(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32))
    A, bp, bst = _a(ac, as_), m.fp8_weight_repack(up(bc)), up(bs)
    y1 = m.fp8_grouped_gemm(A, bp, bst, offsets, N=N, m_total=M, a_rows=a_rows, epilogue=m.EPI_F32,
                            max_rows_per_expert_hint=min(hint, 255))
    ref = m.fp8_swiglu_quantize(y1)
    got = m.fp8_grouped_gemm(A, bp, bst, offsets, N=N, m_total=M, a_rows=a_rows, epilogue=m.EPI_SWIGLU_NVFP4,
                             max_rows_per_expert_hint=hint)
    torch.cuda.synchronize()
    assert torch.equal(got.scales, ref.scales), "block scales differ"
    diff = (got.codes != ref.codes).nonzero()
    assert diff.numel() == 0, f"{diff.shape[0]} codes differ, first at {diff[:5].tolist()}"


def test_fp8_fused_swiglu_full_decode_shape():
    # the fused gate_up the FP8 layer runs at the benchmark's decode workload
    # (T=2048, H=6144, I=256, E=256, top-8, Zipf routing, gathered rows)
    # against float32 rows + the separate SwiGLU kernel, every element
    c = workloads.CONFIGS[2]
    T, H, I, E, k = c.T, c.H, c.I, c.E, c.k
    M = T * k
    print(f"fp8 fused swiglu full shape T={T} H={H} I={I} E={E}", flush=True)
    r = m.moe_route_permute(up(workloads.logits(c)), k)
    ac, as_, bc, bs = _fp8_operands(70, E, 2 * I, H, T)
    A, bp, bst = _a(ac, as_), m.fp8_weight_repack(up(bc)), up(bs)
    y1 = m.fp8_grouped_gemm(A, bp, bst, r.offsets, N=2 * I, m_total=M, a_rows=r.perm_src_token, epilogue=m.EPI_F32,
                            max_rows_per_expert_hint=M // E)
    ref = m.fp8_swiglu_quantize(y1)
    del y1
    got = m.fp8_grouped_gemm(A, bp, bst, r.offsets, N=2 * I, m_total=M, a_rows=r.perm_src_token,
                             epilogue=m.EPI_SWIGLU_NVFP4, max_rows_per_expert_hint=M // E)
    torch.cuda.synchronize()
    assert torch.equal(got.scales, ref.scales)
    assert torch.equal(got.codes, ref.codes)


def _swiglu_tol(y1, absdot):
    I = y1.shape[1] // 2
    tol_y = 1e-3 * absdot + 1e-6
    g, u = y1[:, :I].astype(np.float64), y1[:, I:].astype(np.float64)
    silu = OM.silu(g)
    return 1.1 * tol_y[:, :I] * np.abs(u) + np.abs(silu) * tol_y[:, I:] + 2.0 ** -20 * np.abs(silu * u) + 1e-9


@pytest.mark.parametrize("cfg_index", [0, 1])
@pytest.mark.parametrize("swiglu", ["fused", "separate"])
def test_fp8_layer_end_to_end(cfg_index, swiglu):
    # FP8MoELayer against the oracle's stages composed the same way: routing
    # and x codes bit for bit, weight codes bit for bit, gate_up within the
    # GEMM tolerance, h flips only within the propagated window, and the output
    # within the down tolerance plus the exact bound of every h the GPU rounded
    # the other way
    from block_scaled_fp4_permute_amd.layer import FP8MoELayer, quantize_expert_weights_fp8
    c = workloads.CONFIGS[cfg_index]
    print(f"fp8 layer end to end cfg={cfg_index} swiglu={swiglu}", flush=True)
    logits, x = workloads.logits(c), workloads.activations(c)
    w_gu, w_dn = workloads.torch_expert_weights(c, DEV)
    wq = quantize_expert_weights_fp8(w_gu, w_dn)
    layer = FP8MoELayer(c.T, c.H, c.I, c.E, c.k, DEV, swiglu=swiglu)
    assert layer.fused == (swiglu == "fused")
    out = layer.forward(up(logits), up(x).to(torch.bfloat16), wq)
    torch.cuda.synchronize()
    ids, w = OM.route(logits, c.k)
    counts, offsets, src, perm_of, pw = OM.permute(ids, w, c.E)
    assert np.array_equal(down(layer.routing.perm_src_token), src)
    xb = workloads.to_bf16_values(x)                 # the layer quantises the bf16 activations
    xc, xs = F8.fp8_quantize(xb, 1)
    assert np.array_equal(down(layer.xq.codes), xc) and np.array_equal(down(layer.xq.scales), xs)
    wg, wd = w_gu.cpu().numpy(), w_dn.cpu().numpy()
    gq = [F8.fp8_quantize(wg[e], 128) for e in range(c.E)]
    dq = [F8.fp8_quantize(wd[e], 128) for e in range(c.E)]
    gc, gs = np.stack([q[0] for q in gq]), np.stack([q[1] for q in gq])
    dc, ds = np.stack([q[0] for q in dq]), np.stack([q[1] for q in dq])
    assert np.array_equal(down(wq.gu.codes), gc) and np.array_equal(down(wq.gu.scales), gs)
    assert np.array_equal(down(wq.dn.codes), dc) and np.array_equal(down(wq.dn.scales), ds)
    y1, ad1 = F8.fp8_grouped_gemm(xc, xs, gc, gs, offsets, a_rows=src)
    if layer.y1 is not None:                         # the float32 rows exist on the separate path only
        assert_gemm_close(down(layer.y1), y1, ad1, what="fp8 layer gate_up")
    hc, hs, h64 = F8.fp8_swiglu_quantize(y1)
    hc_gpu, hs_gpu = down(layer.hq.codes), down(layer.hq.scales)
    check_requant_fp8(hc_gpu, hs_gpu, h64, _swiglu_tol(y1, ad1), max_flip_frac=0.02, what="fp8 layer h")
    y2, ad2 = F8.fp8_grouped_gemm(hc, hs, dc, ds, offsets)
    dh = np.abs(F8.fp8_dequantize(hc_gpu, hs_gpu, 1) - F8.fp8_dequantize(hc, hs, 1))
    tol_rows = 1e-3 * ad2 + 1e-6 + 2.0 ** -8 * np.abs(y2.astype(np.float64))
    for e in range(c.E):
        p0, p1 = int(offsets[e]), int(offsets[e + 1])
        if p1 > p0 and dh[p0:p1].any():
            tol_rows[p0:p1] += 1.001 * dh[p0:p1] @ np.abs(F8.fp8_dequantize(dc[e], ds[e], 128)).T
    out64, _ = OM.combine(y2, perm_of, w)
    tol = np.einsum("tj,tjh->th", np.abs(w.astype(np.float64)), tol_rows[perm_of.reshape(c.T, c.k)])
    tol = tol * (1 + 2.0 ** -8) + 2.0 ** -8 * np.abs(out64) + 1e-6
    err = np.abs(bf16_to_f32(out) - out64)
    assert np.all(err <= tol), f"fp8 layer: {int((err > tol).sum())} outputs outside tolerance"
