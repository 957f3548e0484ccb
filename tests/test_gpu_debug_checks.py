"""NVFP4MOE_DEBUG: with the variable set, the calls that read device index
arrays (expert offsets, gathered rows, combine rows) check them on the host
first and reject bad ones with NVFP4MOE_ERR_INVALID before any launch; valid
calls give the same results as without the checks.  Every bad input below is
rejected on the host, so no kernel ever runs on it."""
import numpy as np
import pytest
import torch

import block_scaled_fp4_permute_amd as m
from tests.gpu_common import DEV, up

pytestmark = pytest.mark.gpu


@pytest.fixture
def debug_on(monkeypatch):
    monkeypatch.setenv("NVFP4MOE_DEBUG", "1")


def _gemm_operands(rng, E=3, rows=40, N=64, K=128):
    a = m.NVFP4Tensor(up(rng.integers(0, 256, (rows, K // 2), dtype=np.uint8)),
                      up(rng.integers(0x30, 0x40, (rows, K // 16), dtype=np.uint8)), up(np.ones(1, np.float32)))
    bc = up(rng.integers(0, 256, (E, N, K // 2), dtype=np.uint8))
    bs = up(rng.integers(0x30, 0x40, (E, N, K // 16), dtype=np.uint8))
    bg = up(np.ones(E, np.float32))
    return a, bc, bs, bg


def _expect_invalid(fn, text):
    with pytest.raises(m.NVFP4MoEError) as ei:
        fn()
    assert ei.value.status == m.ERR_INVALID
    assert text in ei.value.detail, ei.value.detail


@pytest.mark.parametrize("offsets,text", [([0, 10, 5, 20], "offsets decrease at expert 1"),
                                          ([0, 10, 20, 41], "offsets[E] = 41 > m_total = 40"),
                                          ([3, 10, 20, 30], "offsets[0] = 3")])
def test_debug_rejects_bad_offsets(debug_on, offsets, text):
    rng = np.random.default_rng(1)
    a, bc, bs, bg = _gemm_operands(rng)
    off = up(np.array(offsets, np.int32))
    print(f"debug check offsets {offsets}", flush=True)
    _expect_invalid(lambda: m.nvfp4_grouped_gemm(a, bc, bs, bg, off, m_total=40), text)


def test_debug_rejects_gathered_rows_out_of_range(debug_on):
    rng = np.random.default_rng(2)
    a, bc, bs, bg = _gemm_operands(rng)
    off = up(np.array([0, 10, 20, 30], np.int32))
    rows = np.arange(40, dtype=np.int32) % 40
    rows[17] = 40                                   # one past the 40 rows of A
    _expect_invalid(lambda: m.nvfp4_grouped_gemm(a, bc, bs, bg, off, m_total=40, a_rows=up(rows)),
                    "a_rows[17] = 40 outside [0, 40)")
    rows[17] = 3
    rows[35] = -1                                   # past offsets[E] = 30: never read, not checked
    y = m.nvfp4_grouped_gemm(a, bc, bs, bg, off, m_total=40, a_rows=up(rows))
    torch.cuda.synchronize()
    assert y.shape == (40, 64)


def test_debug_rejects_combine_rows_out_of_range(debug_on):
    T, k, H = 6, 2, 64
    y = torch.randn((T * k, H), device=DEV).to(torch.bfloat16)
    w = torch.rand((T, k), device=DEV)
    perm = np.arange(T * k, dtype=np.int32)
    perm[5] = T * k
    _expect_invalid(lambda: m.moe_unpermute_combine(y, up(perm), w, T, k), "perm_of_assignment[5] = 12")


def test_debug_checks_leave_valid_calls_unchanged(monkeypatch):
    rng = np.random.default_rng(3)
    a, bc, bs, bg = _gemm_operands(rng)
    off = up(np.array([0, 13, 13, 40], np.int32))
    rows = up(rng.integers(0, 40, 40).astype(np.int32))
    monkeypatch.delenv("NVFP4MOE_DEBUG", raising=False)
    y0 = m.nvfp4_grouped_gemm(a, bc, bs, bg, off, m_total=40, a_rows=rows)
    for v in ("1", "yes"):
        monkeypatch.setenv("NVFP4MOE_DEBUG", v)
        y1 = m.nvfp4_grouped_gemm(a, bc, bs, bg, off, m_total=40, a_rows=rows)
        torch.cuda.synchronize()
        assert torch.equal(y0, y1)
    monkeypatch.setenv("NVFP4MOE_DEBUG", "0")       # "0" switches the checks off
    y2 = m.nvfp4_grouped_gemm(a, bc, bs, bg, off, m_total=40, a_rows=rows)
    torch.cuda.synchronize()
    assert torch.equal(y0, y2)


def test_debug_checks_on_the_other_calls(debug_on):
    # the FP8 and MXFP4 GEMMs and the expert FFN check their offsets too
    rng = np.random.default_rng(4)
    bad = up(np.array([0, 10, 5, 20], np.int32))
    xa = m.FP8Tensor(up(rng.integers(0, 120, (40, 128)).astype(np.uint8)), up(np.ones((40, 1), np.float32)), 1)
    bp = m.fp8_weight_repack(up(rng.integers(0, 120, (3, 64, 128)).astype(np.uint8)))
    bsf = up(np.ones((3, 1, 1), np.float32))
    _expect_invalid(lambda: m.fp8_grouped_gemm(xa, bp, bsf, bad, N=64, m_total=40), "offsets decrease")
    mx_a = m.MXFP4Tensor(up(rng.integers(0, 256, (40, 64), dtype=np.uint8)),
                         up(rng.integers(120, 130, (40, 4), dtype=np.uint8)))
    mx_b = m.MXFP4Tensor(up(rng.integers(0, 256, (3, 64, 64), dtype=np.uint8)),
                         up(rng.integers(120, 130, (3, 64, 4), dtype=np.uint8)))
    _expect_invalid(lambda: m.mxfp4_grouped_gemm(mx_a, mx_b, bad, m_total=40), "offsets decrease")
    E, H, I, M = 3, 256, 128, 40
    xq = m.NVFP4Tensor(up(rng.integers(0, 256, (M, H // 2), dtype=np.uint8)),
                       up(rng.integers(0x30, 0x40, (M, H // 16), dtype=np.uint8)), up(np.ones(1, np.float32)))
    gu_p = m.nvfp4_weight_repack(up(rng.integers(0, 256, (E, 2 * I, H // 2), dtype=np.uint8)),
                                 up(rng.integers(0x30, 0x40, (E, 2 * I, H // 16), dtype=np.uint8)))
    dn_p = m.nvfp4_weight_repack(up(rng.integers(0, 256, (E, H, I // 2), dtype=np.uint8)),
                                 up(rng.integers(0x30, 0x40, (E, H, I // 16), dtype=np.uint8)))
    g = up(np.ones(E, np.float32))
    src = np.arange(M, dtype=np.int32)
    src[2] = M + 5
    good = up(np.array([0, 10, 20, 40], np.int32))
    _expect_invalid(lambda: m.moe_expert_ffn(xq, up(src), good, gu_p, g, dn_p, g, g[:1], H=H, I=I, m_total=M),
                    "perm_src_token[2] = 45 outside [0, 40)")
