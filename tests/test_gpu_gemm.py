"""GPU parity of the grouped NVFP4 GEMM and its epilogues against the oracle.

Inputs of every GPU stage here come from the seeded generators or from the
oracle (its quantiser, its previous stage), never from another GPU stage."""
import numpy as np
import pytest
import torch

import block_scaled_fp4_permute_amd as m
import workloads
from oracle import moe as OM
from oracle import quant as OQ
from tests.gpu_common import DEV, assert_gemm_close, bf16_to_f32, check_requant, down, up

pytestmark = pytest.mark.gpu


def _rand_nvfp4(rng, shape_rows, K, scale_lo=0x28, scale_hi=0x48):
    codes = rng.integers(0, 256, shape_rows + (K // 2,), dtype=np.uint8)
    scales = rng.integers(scale_lo, scale_hi, shape_rows + (K // 16,), dtype=np.uint8)
    return codes, scales


def _run_gemm(a_codes, a_scales, a_g, b_codes, b_scales, b_g, counts, a_rows=None, epilogue=m.EPI_F32,
              m_extra=0, hint=0, packed=False):
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    m_total = int(offsets[-1]) + m_extra
    a = m.NVFP4Tensor(up(a_codes), up(a_scales), up(np.array([a_g], np.float32)))
    bc, bs = up(b_codes), up(b_scales)
    bp = m.nvfp4_weight_repack(bc, bs) if packed else None
    y = m.nvfp4_grouped_gemm(a, bc, bs, up(np.asarray(b_g, np.float32)), up(offsets),
                             m_total=m_total, a_rows=None if a_rows is None else up(a_rows.astype(np.int32)),
                             epilogue=epilogue, max_rows_per_expert_hint=hint, b_packed=bp)
    torch.cuda.synchronize()
    return y, offsets


def _unpack_tiles(packed, E, N, K):
    """Inverse of the documented packed layout (tile (e, rt, st) of 2304 bytes;
    lane l = 16g + n holds row 16rt+n, code bytes [128st+32g, +32) at [16l, +16)
    and [1024+16l, +16), scale bytes [16st+4g, +4) at [2048+4l, +4))."""
    ntr, nst = (N + 15) // 16, (K + 255) // 256
    t = np.asarray(packed, np.uint8)[: E * ntr * nst * 2304].reshape(E, ntr, nst, 2304)
    codes = np.zeros((E, ntr * 16, nst * 128), np.uint8)
    scales = np.zeros((E, ntr * 16, nst * 16), np.uint8)
    for l in range(64):
        n, g = l % 16, l // 16
        rows = np.arange(ntr) * 16 + n
        for st in range(nst):
            codes[:, rows, 128 * st + 32 * g: 128 * st + 32 * g + 16] = t[:, :, st, 16 * l: 16 * l + 16]
            codes[:, rows, 128 * st + 32 * g + 16: 128 * st + 32 * g + 32] = t[:, :, st, 1024 + 16 * l: 1024 + 16 * l + 16]
            scales[:, rows, 16 * st + 4 * g: 16 * st + 4 * g + 4] = t[:, :, st, 2048 + 4 * l: 2048 + 4 * l + 4]
    return codes, scales


@pytest.mark.parametrize("E,N,K", [(3, 48, 288), (1, 16, 32), (2, 512, 6144), (4, 64, 256)])
def test_weight_repack_layout(E, N, K):
    rng = np.random.default_rng(E * N + K)
    codes = rng.integers(0, 256, (E, N, K // 2), dtype=np.uint8)
    scales = rng.integers(0, 256, (E, N, K // 16), dtype=np.uint8)
    packed = down(m.nvfp4_weight_repack(up(codes), up(scales)))
    torch.cuda.synchronize()
    assert packed.size == m.lib().nvfp4_weight_packed_size(E, N, K)
    uc, us = _unpack_tiles(packed, E, N, K)
    assert np.array_equal(uc[:, :N, :K // 2], codes) and np.array_equal(us[:, :N, :K // 16], scales)
    assert not uc[:, N:].any() and not uc[:, :, K // 2:].any() and not us[:, :, K // 16:].any()


GEMM_CASES = [
    # E, counts, N, K, rows_a, hint
    (3, [5, 0, 17], 64, 128, 30, 0),
    (4, [1, 100, 64, 65], 48, 32, 300, 0),
    (2, [200, 3], 512, 6144, 203, 0),
    (1, [300], 96, 96, 300, 16),
    (5, [0, 0, 0, 0, 7], 256, 256, 7, 0),
    (8, [16, 31, 33, 64, 2, 0, 129, 8], 160, 224, 283, 4),
]


@pytest.mark.parametrize("case", range(len(GEMM_CASES)))
@pytest.mark.parametrize("gather", [False, True])
@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("epi", ["f32", "bf16"])
def test_gemm_f32_random(case, gather, packed, epi):
    # with packed weights and K <= 256 the launcher picks the stream-N kernel
    # (whose bf16 rows leave through its LDS-staged store), otherwise stream-K
    E, counts, N, K, rows_a, hint = GEMM_CASES[case]
    print(f"gemm case {case} gather={gather} packed={packed} epi={epi} E={E} N={N} K={K}", flush=True)
    rng = np.random.default_rng(100 + case)
    a_codes, a_scales = _rand_nvfp4(rng, (rows_a,), K)
    b_codes, b_scales = _rand_nvfp4(rng, (E, N), K)
    a_g = np.float32(0.0123)
    b_g = rng.uniform(0.001, 0.01, E).astype(np.float32)
    M = int(np.sum(counts))
    a_rows = rng.integers(0, rows_a, M).astype(np.int32) if gather else None
    if not gather:
        a_codes, a_scales = a_codes[:max(M, 1)], a_scales[:max(M, 1)]
    y, offsets = _run_gemm(a_codes, a_scales, a_g, b_codes, b_scales, b_g, counts, a_rows, hint=hint, packed=packed,
                           epilogue=m.EPI_F32 if epi == "f32" else m.EPI_BF16)
    y_ref, absdot = OM.grouped_gemm(a_codes, a_scales, a_g, b_codes, b_scales, b_g, offsets, a_rows=a_rows)
    got = down(y)[:M] if epi == "f32" else bf16_to_f32(y)[:M]
    assert_gemm_close(got, y_ref, absdot, bf16_out=epi == "bf16", what=f"case {case} {epi}")


@pytest.mark.parametrize("hint", [0, 4096])
@pytest.mark.parametrize("packed", [False, True])
def test_gemm_many_experts_task_map(hint, packed):
    # more experts than threads in a work-group (the task map walks the
    # experts in several block-wide passes), many empty experts, a few with
    # several chunks; F32 (stream-K or stream-N) and fused SwiGLU (stream-K)
    rng = np.random.default_rng(7 + hint + int(packed))
    E, N, K = 600, 64, 512
    counts = rng.integers(0, 40, E) * (rng.random(E) < 0.7)
    counts[rng.choice(E, 6, replace=False)] = [150, 200, 64, 65, 129, 17]
    counts = counts.astype(np.int64)
    M = int(counts.sum())
    print(f"many experts: E={E} M={M} hint={hint} packed={packed}", flush=True)
    a_codes, a_scales = _rand_nvfp4(rng, (500,), K)
    b_codes, b_scales = _rand_nvfp4(rng, (E, N), K)
    b_g = rng.uniform(0.001, 0.01, E).astype(np.float32)
    a_rows = rng.integers(0, 500, M).astype(np.int32)
    for k_used in (K, 256):
        ac, as_ = a_codes[:, :k_used // 2].copy(), a_scales[:, :k_used // 16].copy()
        bc, bs = b_codes[:, :, :k_used // 2].copy(), b_scales[:, :, :k_used // 16].copy()
        y, offsets = _run_gemm(ac, as_, 0.02, bc, bs, b_g, counts, a_rows, hint=hint, packed=packed)
        y_ref, absdot = OM.grouped_gemm(ac, as_, 0.02, bc, bs, b_g, offsets, a_rows=a_rows)
        assert_gemm_close(down(y)[:M], y_ref, absdot, what=f"K={k_used}")
    y_ref, absdot = OM.grouped_gemm(a_codes, a_scales, 0.02, b_codes, b_scales, b_g, offsets, a_rows=a_rows)
    h64 = OM.swiglu(y_ref)
    g_h = np.float32(np.abs(h64.astype(np.float32)).max() / np.float32(2688))
    a = m.NVFP4Tensor(up(a_codes), up(a_scales), up(np.array([0.02], np.float32)))
    bct, bst = up(b_codes), up(b_scales)
    hq = m.nvfp4_grouped_gemm(a, bct, bst, up(b_g), up(offsets), m_total=M, a_rows=up(a_rows),
                              epilogue=m.EPI_SWIGLU_NVFP4, out_g=up(np.array([g_h], np.float32)),
                              max_rows_per_expert_hint=hint,
                              b_packed=m.nvfp4_weight_repack(bct, bst) if packed else None)
    torch.cuda.synchronize()
    check_requant(down(hq.codes), down(hq.scales), h64, g_h, _swiglu_tol(y_ref, absdot), max_flip_frac=0.02,
                  what="many experts swiglu")


@pytest.mark.parametrize("hint", [1, 200, 4096])
@pytest.mark.parametrize("packed", [False, True])
def test_gemm_decode_and_large_tile_shapes(hint, packed):
    # the rows-per-expert hint picks the decode (64-row) tile, the 128-row
    # 8-wave tile (128..255 rows, or row-major weights) or, with packed weights
    # from 256 rows, the 256 x 256 tile with both operands staged in LDS; all
    # must meet the oracle, with F32 and fused SwiGLU epilogues
    rng = np.random.default_rng(hint + int(packed))
    E, counts, N, K = 3, [150, 300, 7], 512, 1024
    M = sum(counts)
    a_codes, a_scales = _rand_nvfp4(rng, (400,), K)
    b_codes, b_scales = _rand_nvfp4(rng, (E, N), K)
    b_g = rng.uniform(0.001, 0.01, E).astype(np.float32)
    a_rows = rng.integers(0, 400, M).astype(np.int32)
    y, offsets = _run_gemm(a_codes, a_scales, 0.02, b_codes, b_scales, b_g, counts, a_rows, hint=hint,
                           packed=packed)
    y_ref, absdot = OM.grouped_gemm(a_codes, a_scales, 0.02, b_codes, b_scales, b_g, offsets, a_rows=a_rows)
    assert_gemm_close(down(y)[:M], y_ref, absdot, what=f"hint {hint}")
    h64 = OM.swiglu(y_ref)
    g_h = np.float32(np.abs(h64.astype(np.float32)).max() / np.float32(2688))
    a = m.NVFP4Tensor(up(a_codes), up(a_scales), up(np.array([0.02], np.float32)))
    bc, bs = up(b_codes), up(b_scales)
    hq = m.nvfp4_grouped_gemm(a, bc, bs, up(b_g), up(offsets), m_total=M, a_rows=up(a_rows),
                              epilogue=m.EPI_SWIGLU_NVFP4, out_g=up(np.array([g_h], np.float32)),
                              max_rows_per_expert_hint=hint, b_packed=m.nvfp4_weight_repack(bc, bs) if packed else None)
    torch.cuda.synchronize()
    check_requant(down(hq.codes), down(hq.scales), h64, g_h, _swiglu_tol(y_ref, absdot), max_flip_frac=0.02,
                  what=f"fused swiglu hint {hint}")


# packed weights, K a multiple of 256, hint (or average) >= 256: the 256 x 256
# tile (both operands in LDS, A decoded once per workgroup a quarter step at a time)
LARGE_CASES = [
    # E, counts, N, K, rows_a, hint
    (3, [300, 0, 517], 320, 512, 400, 256),          # a partial column tile, an empty expert
    (1, [600], 512, 2048, 600, 0),                   # by the average; a partial row chunk
    (5, [256, 1, 1000, 0, 255], 256, 768, 700, 300),  # 1-row and 255-row experts, 4 chunks in one group
]


@pytest.mark.parametrize("case", range(len(LARGE_CASES)))
@pytest.mark.parametrize("gather", [False, True])
@pytest.mark.parametrize("epi", ["f32", "bf16"])
def test_gemm_large_tile(case, gather, epi):
    E, counts, N, K, rows_a, hint = LARGE_CASES[case]
    print(f"gemm large case {case} gather={gather} epi={epi} E={E} N={N} K={K}", flush=True)
    rng = np.random.default_rng(500 + case)
    M = int(np.sum(counts))
    if not gather:
        rows_a = M                     # row p of the GEMM reads A row p
    a_codes, a_scales = _rand_nvfp4(rng, (rows_a,), K)
    b_codes, b_scales = _rand_nvfp4(rng, (E, N), K)
    a_g = np.float32(0.0123)
    b_g = rng.uniform(0.001, 0.01, E).astype(np.float32)
    a_rows = rng.integers(0, rows_a, M).astype(np.int32) if gather else None
    y, offsets = _run_gemm(a_codes, a_scales, a_g, b_codes, b_scales, b_g, counts, a_rows, hint=hint, packed=True,
                           epilogue=m.EPI_F32 if epi == "f32" else m.EPI_BF16)
    y_ref, absdot = OM.grouped_gemm(a_codes, a_scales, a_g, b_codes, b_scales, b_g, offsets, a_rows=a_rows)
    got = down(y)[:M] if epi == "f32" else bf16_to_f32(y)[:M]
    assert_gemm_close(got, y_ref, absdot, bf16_out=epi == "bf16", what=f"large case {case} {epi}")


def test_gemm_large_tile_fused_swiglu_and_combine():
    # SwiGLU + NVFP4 requant with I = 192 (the second 128-column h tile half
    # empty), then the float32 scatter-add combine epilogue, both on the
    # 256 x 256 tile
    rng = np.random.default_rng(41)
    E, counts, I, K = 3, [260, 40, 700], 192, 1024
    M = sum(counts)
    a_codes, a_scales = _rand_nvfp4(rng, (900,), K)
    b_codes, b_scales = _rand_nvfp4(rng, (E, 2 * I), K)
    b_g = rng.uniform(0.001, 0.01, E).astype(np.float32)
    a_rows = rng.integers(0, 900, M).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    y_ref, absdot = OM.grouped_gemm(a_codes, a_scales, 0.02, b_codes, b_scales, b_g, offsets, a_rows=a_rows)
    h64 = OM.swiglu(y_ref)
    g_h = np.float32(np.abs(h64.astype(np.float32)).max() / np.float32(2688))
    a = m.NVFP4Tensor(up(a_codes), up(a_scales), up(np.array([0.02], np.float32)))
    bc, bs = up(b_codes), up(b_scales)
    hq = m.nvfp4_grouped_gemm(a, bc, bs, up(b_g), up(offsets), m_total=M, a_rows=up(a_rows),
                              epilogue=m.EPI_SWIGLU_NVFP4, out_g=up(np.array([g_h], np.float32)),
                              max_rows_per_expert_hint=256, b_packed=m.nvfp4_weight_repack(bc, bs))
    torch.cuda.synchronize()
    check_requant(down(hq.codes), down(hq.scales), h64, g_h, _swiglu_tol(y_ref, absdot), max_flip_frac=0.02,
                  what="large-tile fused swiglu")
    # combine: rows scattered to 333 tokens with weights, N = 2I columns
    tok = rng.integers(0, 333, M).astype(np.int32)
    wt = rng.uniform(0.1, 1.0, M).astype(np.float32)
    acc = torch.zeros((333, 2 * I), dtype=torch.float32, device=DEV)
    m.nvfp4_grouped_gemm(a, bc, bs, up(b_g), up(offsets), m_total=M, a_rows=up(a_rows), epilogue=m.EPI_COMBINE_F32,
                         out=acc, out_rows=333, row_token=up(tok), row_weight=up(wt), max_rows_per_expert_hint=256,
                         b_packed=m.nvfp4_weight_repack(bc, bs))
    torch.cuda.synchronize()
    ref = np.zeros((333, 2 * I))
    tol = np.zeros((333, 2 * I))
    np.add.at(ref, tok, wt.astype(np.float64)[:, None] * y_ref)
    np.add.at(tol, tok, wt.astype(np.float64)[:, None] * (1e-3 * absdot + 1e-6))
    got = down(acc).astype(np.float64)
    # float32 atomics add the rows in any order: a few ulps of the running sums
    tol += 8 * 2.0 ** -24 * np.abs(ref) + 1e-30
    assert np.all(np.abs(got - ref) <= tol), "large-tile combine epilogue"


def test_gemm_dense_8192_sampled_rows():
    # the dense M = N = K = 8192 GEMM in the launch the benchmark times (256 x
    # 256 tile, packed weights, bf16 out), checked on 24 sampled rows
    rng = np.random.default_rng(8193)
    M = N = K = 8192
    print("nvfp4 dense 8192^3 sampled rows", flush=True)
    a_codes, a_scales = _rand_nvfp4(rng, (M,), K)
    b_codes, b_scales = _rand_nvfp4(rng, (1, N), K)
    a = m.NVFP4Tensor(up(a_codes), up(a_scales), up(np.array([0.01], np.float32)))
    bc, bs = up(b_codes), up(b_scales)
    offsets = np.array([0, M], np.int32)
    y = m.nvfp4_grouped_gemm(a, bc, bs, up(np.array([0.02], np.float32)), up(offsets), m_total=M,
                             epilogue=m.EPI_BF16, b_packed=m.nvfp4_weight_repack(bc, bs))
    torch.cuda.synchronize()
    rows = np.sort(rng.choice(M, 24, replace=False))
    rows[0], rows[-1] = 0, M - 1
    got = bf16_to_f32(y[torch.as_tensor(rows, device=y.device)])
    y_ref, absdot = OM.grouped_gemm(a_codes[rows], a_scales[rows], 0.01, b_codes, b_scales,
                                    np.array([0.02], np.float32), np.array([0, len(rows)], np.int32))
    assert_gemm_close(got, y_ref, absdot, bf16_out=True, what="nvfp4 dense 8192^3, sampled rows")


@pytest.mark.parametrize("epilogue", ["f32", "swiglu"])
def test_gemm_light_chunks_split_into_narrow_tasks(epilogue):
    # more whole-width tasks than resident workgroups, most experts with at
    # most 16 rows: with packed weights those chunks run as twice as many
    # half-width tasks; results must meet the oracle and equal, bit for bit,
    # the row-major path (which never splits and sums in the same order)
    rng = np.random.default_rng(11 + (epilogue == "swiglu"))
    E, N, K = 300, 512, 512
    counts = rng.integers(1, 17, E)
    counts[rng.choice(E, 40, replace=False)] = rng.integers(17, 200, 40)
    counts[rng.choice(E, 10, replace=False)] = 0
    M = int(counts.sum())
    print(f"light chunks: E={E} M={M} N={N} K={K} epilogue={epilogue}", flush=True)
    a_codes, a_scales = _rand_nvfp4(rng, (700,), K)
    b_codes, b_scales = _rand_nvfp4(rng, (E, N), K)
    b_g = rng.uniform(0.001, 0.01, E).astype(np.float32)
    a_rows = rng.integers(0, 700, M).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    y_ref, absdot = OM.grouped_gemm(a_codes, a_scales, 0.02, b_codes, b_scales, b_g, offsets, a_rows=a_rows)
    if epilogue == "f32":
        outs = []
        for packed in (True, False):
            y, _ = _run_gemm(a_codes, a_scales, 0.02, b_codes, b_scales, b_g, counts, a_rows, packed=packed)
            outs.append(down(y)[:M])
        assert_gemm_close(outs[0], y_ref, absdot, what="narrow tasks f32")
        assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
    else:
        h64 = OM.swiglu(y_ref)
        g_h = np.float32(np.abs(h64.astype(np.float32)).max() / np.float32(2688))
        a = m.NVFP4Tensor(up(a_codes), up(a_scales), up(np.array([0.02], np.float32)))
        bc, bs = up(b_codes), up(b_scales)
        outs = []
        for packed in (True, False):
            hq = m.nvfp4_grouped_gemm(a, bc, bs, up(b_g), up(offsets), m_total=M, a_rows=up(a_rows),
                                      epilogue=m.EPI_SWIGLU_NVFP4, out_g=up(np.array([g_h], np.float32)),
                                      b_packed=m.nvfp4_weight_repack(bc, bs) if packed else None)
            torch.cuda.synchronize()
            outs.append((down(hq.codes), down(hq.scales)))
        check_requant(outs[0][0], outs[0][1], h64, g_h, _swiglu_tol(y_ref, absdot), max_flip_frac=0.02,
                      what="narrow tasks swiglu")
        assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])


def test_gemm_bf16_epilogue_and_untouched_tail_rows():
    rng = np.random.default_rng(7)
    E, counts, N, K = 3, [9, 40, 2], 128, 256
    a_codes, a_scales = _rand_nvfp4(rng, (51,), K)
    b_codes, b_scales = _rand_nvfp4(rng, (E, N), K)
    b_g = np.array([0.5, 0.25, 0.125], np.float32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    a = m.NVFP4Tensor(up(a_codes), up(a_scales), up(np.array([0.01], np.float32)))
    out = torch.full((60, N), 7.0, dtype=torch.bfloat16, device=DEV)     # 9 rows past offsets[E]
    m.nvfp4_grouped_gemm(a, up(b_codes), up(b_scales), up(b_g), up(offsets), m_total=60, epilogue=m.EPI_BF16,
                         out=out)
    torch.cuda.synchronize()
    y_ref, absdot = OM.grouped_gemm(a_codes, a_scales, 0.01, b_codes, b_scales, b_g, offsets)
    got = bf16_to_f32(out)
    assert_gemm_close(got[:51], y_ref, absdot, bf16_out=True)
    assert np.all(got[51:] == 7.0)


@pytest.mark.parametrize("K,packed,large", [(32, False, False), (256, False, False), (4096, False, False),
                                             (6144, False, False), (32, True, False), (256, True, False),
                                             (4096, True, False), (6144, True, False), (256, True, True),
                                             (6144, True, True)])
def test_gemm_constant_scales_bit_exact(K, packed, large):
    # constant block scales and unit per-tensor scales make every FP32 partial
    # sum exact, so the GPU must reproduce the oracle bit for bit (large: the
    # 256 x 256 tile)
    rng = np.random.default_rng(K + large)
    E, counts, N = (2, [300, 520], 272) if large else (2, [37, 70], 80)
    M = sum(counts)
    a_codes = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    b_codes = rng.integers(0, 256, (E, N, K // 2), dtype=np.uint8)
    a_scales = np.full((M, K // 16), 0x3A, np.uint8)          # 1.25
    b_scales = np.full((E, N, K // 16), 0x30, np.uint8)       # 0.5
    y, offsets = _run_gemm(a_codes, a_scales, 1.0, b_codes, b_scales, np.ones(E, np.float32), counts, packed=packed,
                           hint=256 if large else 0)
    y_ref, _ = OM.grouped_gemm(a_codes, a_scales, 1.0, b_codes, b_scales, np.ones(E, np.float32), offsets)
    assert np.array_equal(down(y), y_ref)


@pytest.mark.parametrize("sa,sb", [(0x03, 0x05), (0x01, 0x7E), (0x07, 0x08), (0x00, 0x40)])
@pytest.mark.parametrize("packed,large", [(False, False), (True, False), (True, True)])
def test_gemm_subnormal_and_extreme_scales_bit_exact(sa, sb, packed, large):
    # E4M3 subnormal block scales (codes 1..7) pass through FP16 subnormals in
    # the decode; with one scale per operand and unit per-tensor scales the
    # float32 result is exact in any summation order, so it must match exactly
    rng = np.random.default_rng(sa * 256 + sb)
    E, counts, N, K = (2, [300, 280], 48, 1024) if large else (2, [21, 50], 48, 1024)
    M = sum(counts)
    a_codes = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    b_codes = rng.integers(0, 256, (E, N, K // 2), dtype=np.uint8)
    a_scales = np.full((M, K // 16), sa, np.uint8)
    b_scales = np.full((E, N, K // 16), sb, np.uint8)
    y, offsets = _run_gemm(a_codes, a_scales, 1.0, b_codes, b_scales, np.ones(E, np.float32), counts, packed=packed)
    y_ref, _ = OM.grouped_gemm(a_codes, a_scales, 1.0, b_codes, b_scales, np.ones(E, np.float32), offsets)
    assert np.array_equal(down(y), y_ref)


def test_gemm_single_block_products_exact():
    # K = 32 with extreme scales: each output is one or two exact block terms
    rng = np.random.default_rng(3)
    a_codes, a_scales = _rand_nvfp4(rng, (16,), 32, 0x01, 0x7F)
    b_codes, b_scales = _rand_nvfp4(rng, (1, 16), 32, 0x01, 0x7F)
    a_scales[:, 1] = 0                                      # second block contributes nothing
    y, offsets = _run_gemm(a_codes, a_scales, 1.0, b_codes, b_scales, np.ones(1, np.float32), [16])
    y_ref, _ = OM.grouped_gemm(a_codes, a_scales, 1.0, b_codes, b_scales, np.ones(1, np.float32), offsets)
    assert np.array_equal(down(y), y_ref)


# ------------------------------------------------------------------ config 0 stages
def _config0():
    c = workloads.CONFIGS[0]
    logits = workloads.logits(c)
    x = workloads.activations(c)
    wgu = OM.quantize_experts([workloads.gate_up_weight(c, e) for e in range(c.E)])
    wdn = OM.quantize_experts([workloads.down_weight(c, e) for e in range(c.E)])
    ids, w = OM.route(logits, c.k)
    counts, offsets, src, perm_of, pw = OM.permute(ids, w, c.E)
    xq = OQ.quantize(x)
    return c, logits, x, wgu, wdn, ids, w, counts, offsets, src, perm_of, pw, xq


def test_config0_gate_up_f32_gathered():
    c, logits, x, wgu, wdn, ids, w, counts, offsets, src, perm_of, pw, xq = _config0()
    y, _ = _run_gemm(xq[0], xq[1], xq[2], *wgu, counts, a_rows=src)
    y_ref, absdot = OM.grouped_gemm(*xq, *wgu, offsets, a_rows=src)
    assert_gemm_close(down(y), y_ref, absdot)


def _swiglu_tol(y1_ref, absdot1):
    I = y1_ref.shape[1] // 2
    tol_y = 1e-3 * absdot1 + 1e-6
    g, u = y1_ref[:, :I].astype(np.float64), y1_ref[:, I:].astype(np.float64)
    silu = OM.silu(g)
    h = silu * u
    return 1.1 * tol_y[:, :I] * np.abs(u) + np.abs(silu) * tol_y[:, I:] + 2.0 ** -20 * np.abs(h) + 1e-7


def test_swiglu_unfused_stage():
    c, logits, x, wgu, wdn, ids, w, counts, offsets, src, perm_of, pw, xq = _config0()
    y1, _ = OM.grouped_gemm(*xq, *wgu, offsets, a_rows=src)
    h64 = OM.swiglu(y1)
    g_h = np.float32(np.abs(h64.astype(np.float32)).max() / np.float32(2688))
    for dt in (torch.float32, torch.bfloat16):
        y_in = y1 if dt == torch.float32 else workloads.to_bf16_values(y1)
        hq = m.moe_swiglu(up(y_in).to(dt), g=up(np.array([g_h], np.float32)))
        torch.cuda.synchronize()
        h_ref = OM.swiglu(y_in)
        check_requant(down(hq.codes), down(hq.scales), h_ref, g_h, 2.0 ** -20 * np.abs(h_ref) + 1e-30,
                      what=f"moe_swiglu {dt}")
    # amax computed on the device
    hq = m.moe_swiglu(up(y1))
    torch.cuda.synchronize()
    g_dev = down(hq.g)[0]
    assert abs(g_dev - g_h) <= 2.0 ** -20 * g_h


@pytest.mark.parametrize("packed", [False, True])
def test_config0_gate_up_fused_swiglu(packed):
    c, logits, x, wgu, wdn, ids, w, counts, offsets, src, perm_of, pw, xq = _config0()
    y1, absdot1 = OM.grouped_gemm(*xq, *wgu, offsets, a_rows=src)
    h64 = OM.swiglu(y1)
    g_h = np.float32(np.abs(h64.astype(np.float32)).max() / np.float32(2688))
    a = m.NVFP4Tensor(up(xq[0]), up(xq[1]), up(np.array([xq[2]], np.float32)))
    bc, bs = up(wgu[0]), up(wgu[1])
    hq = m.nvfp4_grouped_gemm(a, bc, bs, up(wgu[2]), up(offsets), m_total=int(offsets[-1]),
                              a_rows=up(src), epilogue=m.EPI_SWIGLU_NVFP4, out_g=up(np.array([g_h], np.float32)),
                              b_packed=m.nvfp4_weight_repack(bc, bs) if packed else None)
    torch.cuda.synchronize()
    check_requant(down(hq.codes), down(hq.scales), h64, g_h, _swiglu_tol(y1, absdot1), max_flip_frac=0.02,
                  what="fused swiglu")


def test_fused_swiglu_exact_accumulation():
    # constant scales, unit per-tensor scales: y1 is exact on both sides, so
    # the fused re-quantisation differs from the oracle only through silu's
    # float32 rounding
    rng = np.random.default_rng(21)
    E, counts, I, K = 2, [19, 45], 64, 512
    M = sum(counts)
    a_codes = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    b_codes = rng.integers(0, 256, (E, 2 * I, K // 2), dtype=np.uint8)
    a_scales = np.full((M, K // 16), 0x20, np.uint8)         # 2^-3
    b_scales = np.full((E, 2 * I, K // 16), 0x28, np.uint8)   # 2^-2
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    y1, _ = OM.grouped_gemm(a_codes, a_scales, 1.0, b_codes, b_scales, np.ones(E, np.float32), offsets)
    h64 = OM.swiglu(y1)
    g_h = np.float32(np.abs(h64).max() / 2688)
    a = m.NVFP4Tensor(up(a_codes), up(a_scales), up(np.ones(1, np.float32)))
    hq = m.nvfp4_grouped_gemm(a, up(b_codes), up(b_scales), up(np.ones(E, np.float32)), up(offsets), m_total=M,
                              epilogue=m.EPI_SWIGLU_NVFP4, out_g=up(np.array([g_h], np.float32)))
    torch.cuda.synchronize()
    ns, nc = check_requant(down(hq.codes), down(hq.scales), h64, g_h, 2.0 ** -20 * np.abs(h64) + 1e-30,
                           max_flip_frac=1e-3, what="fused swiglu exact")


@pytest.mark.parametrize("packed", [False, True])
def test_config0_down_fused_combine_and_unfused_combine(packed):
    c, logits, x, wgu, wdn, ids, w, counts, offsets, src, perm_of, pw, xq = _config0()
    y1, _ = OM.grouped_gemm(*xq, *wgu, offsets, a_rows=src)
    h64 = OM.swiglu(y1)
    g_h = np.float32(np.abs(h64.astype(np.float32)).max() / np.float32(2688))
    hq = OQ.quantize(h64.astype(np.float32), g=g_h)
    y2, absdot2 = OM.grouped_gemm(*hq, *wdn, offsets)
    out64, out_ref = OM.combine(y2, perm_of, w)
    # tolerance: weighted GEMM tolerance of the k rows + bf16 rounding of the sum
    tol_rows = 1e-3 * absdot2 + 1e-6
    tol = np.einsum("tj,tjh->th", np.abs(w.astype(np.float64)), tol_rows[perm_of.reshape(w.shape)]) \
        + 2.0 ** -8 * np.abs(out64) + 1e-6
    # fused: scatter-add epilogue into a float32 accumulator, then to bf16
    a = m.NVFP4Tensor(up(hq[0]), up(hq[1]), up(np.array([hq[2]], np.float32)))
    acc = torch.zeros((c.T, c.H), dtype=torch.float32, device=DEV)
    bc, bs = up(wdn[0]), up(wdn[1])
    m.nvfp4_grouped_gemm(a, bc, bs, up(wdn[2]), up(offsets), m_total=int(offsets[-1]),
                         epilogue=m.EPI_COMBINE_F32, out=acc, out_rows=c.T, row_token=up(src), row_weight=up(pw),
                         b_packed=m.nvfp4_weight_repack(bc, bs) if packed else None)
    out = m.moe_unpermute_combine(acc, None, None, c.T, 1)
    torch.cuda.synchronize()
    assert np.all(np.abs(bf16_to_f32(out) - out64) <= tol), "fused combine"
    # unfused: combine of the oracle's y2 (float32 and bf16 inputs)
    for dt in (torch.float32, torch.bfloat16):
        y_in = y2 if dt == torch.float32 else workloads.to_bf16_values(y2)
        o = m.moe_unpermute_combine(up(y_in).to(dt), up(perm_of), up(w), c.T, c.k)
        torch.cuda.synchronize()
        ref64, _ = OM.combine(y_in, perm_of, w)
        t2 = 2.0 ** -8 * np.abs(ref64) + c.k * 2.0 ** -23 * np.einsum(
            "tj,tjh->th", np.abs(w.astype(np.float64)), np.abs(y_in.astype(np.float64))[perm_of.reshape(w.shape)]) + 1e-30
        assert np.all(np.abs(bf16_to_f32(o) - ref64) <= t2), f"unfused combine {dt}"
    # combine with k = 1, unit weights, identity permutation is exact conversion
    o = m.moe_unpermute_combine(up(y2), None, None, y2.shape[0], 1, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(down(o), y2)


@pytest.mark.parametrize("k", [1, 3, 8, 9, 17, 32])
@pytest.mark.parametrize("ydt", [torch.float32, torch.bfloat16])
def test_combine_any_k(k, ydt):
    # the combine fetches a token's rows in batches of 8: k below, at and
    # above a batch, and the largest k the router supports
    rng = np.random.default_rng(50 + k)
    T, H = 37, 272
    M = T * k
    y = rng.standard_normal((M, H)).astype(np.float32) * rng.uniform(0.1, 10, (M, 1)).astype(np.float32)
    if ydt == torch.bfloat16:
        y = workloads.to_bf16_values(y)
    perm_of = rng.permutation(M).astype(np.int32)
    w = rng.uniform(0, 1, (T, k)).astype(np.float32)
    print(f"combine k={k} y={ydt}", flush=True)
    ref64, _ = OM.combine(y, perm_of, w)
    bound = k * 2.0 ** -23 * np.einsum("tj,tjh->th", np.abs(w.astype(np.float64)),
                                        np.abs(y.astype(np.float64))[perm_of.reshape(T, k)]) + 1e-30
    o16 = m.moe_unpermute_combine(up(y).to(ydt), up(perm_of), up(w), T, k)
    o32 = m.moe_unpermute_combine(up(y).to(ydt), up(perm_of), up(w), T, k, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert np.all(np.abs(down(o32) - ref64) <= bound), "float32 out"
    assert np.all(np.abs(bf16_to_f32(o16) - ref64) <= bound + 2.0 ** -8 * np.abs(ref64)), "bf16 out"
