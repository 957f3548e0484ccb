"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every
function declared in include/*.h, and rejects invalid arguments on the host
before anything is enqueued (each case below fails validation, so no kernel is
ever launched here)."""
import ctypes
import glob
import os
import re

import pytest

import block_scaled_fp4_permute_amd as m

# The validation cases hand the library fake device addresses, relying on the
# host checks to reject every call before a launch.  Where a GPU is visible a
# regressed check would launch a kernel on them, so this module runs only on
# machines without one (the GPU parity tests cover the library there).
try:
    import torch
    _HAVE_GPU = torch.cuda.is_available()
except Exception:  # pragma: no cover
    _HAVE_GPU = False
pytestmark = pytest.mark.skipif(_HAVE_GPU, reason="fake device addresses: host-only checks, run without a GPU")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

FAKE = 1 << 20          # a non-null, 16-byte aligned address that is never dereferenced
FAKE_MIS = FAKE + 2     # non-null, misaligned


def _declared_functions():
    names = []
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for mt in re.finditer(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(", text, re.M):
            names.append(mt.group(1))
    return sorted(set(names))


def test_header_declares_the_five_calls():
    names = _declared_functions()
    for want in ("moe_route_permute", "nvfp4_quantize", "nvfp4_grouped_gemm", "moe_swiglu",
                 "moe_unpermute_combine"):
        assert want in names


def test_library_exports_every_declared_symbol():
    L = m.lib()
    missing = [n for n in _declared_functions() if not hasattr(L, n)]
    assert not missing, missing


def test_version_and_status_strings():
    L = m.lib()
    assert L.nvfp4moe_version() >= 100
    assert L.nvfp4moe_status_string(0) == b"ok"
    assert b"workspace" in L.nvfp4moe_status_string(3)
    assert L.nvfp4moe_status_string(99) == b"unknown status"


def _route(T=4, E=8, k=2, logits=FAKE, ws=FAKE, ws_bytes=None):
    L = m.lib()
    if ws_bytes is None:
        ws_bytes = L.moe_route_permute_workspace_size(T, E, k)
    return L.moe_route_permute(logits, T, E, k, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, ws, ws_bytes, None)


def test_route_validation():
    L = m.lib()
    assert _route(logits=None) == m.ERR_INVALID
    assert _route(T=0) == m.ERR_INVALID
    assert _route(k=9, E=8) == m.ERR_INVALID
    assert b"k=9" in L.nvfp4moe_last_error_detail()
    assert _route(k=33, E=64) == m.ERR_UNSUPPORTED
    assert _route(E=5000, k=2) == m.ERR_UNSUPPORTED
    assert _route(ws_bytes=4) == m.ERR_WORKSPACE
    assert _route(ws=None) == m.ERR_WORKSPACE
    assert L.moe_route_permute_workspace_size(256, 256, 8) >= 256 * 8 * 4 + 2 * 256 * 4


def _route_quantize(logits=FAKE, T=16, E=8, k=2, x=FAKE, x_dtype=m.BF16, cols=64, codes=FAKE, ws=FAKE,
                    ws_bytes=1 << 20):
    L = m.lib()
    return L.moe_route_quantize(logits, T, E, k, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, x, x_dtype, cols, None,
                                None, codes, FAKE, ws, ws_bytes, None)


def test_route_quantize_validation():
    # every check runs before any launch: no GPU needed
    L = m.lib()
    assert _route_quantize(logits=None) == m.ERR_INVALID
    assert _route_quantize(x=None) == m.ERR_INVALID
    assert _route_quantize(T=0) == m.ERR_INVALID
    assert _route_quantize(k=9, E=8) == m.ERR_INVALID
    assert _route_quantize(k=33, E=64) == m.ERR_UNSUPPORTED
    assert _route_quantize(cols=48) == m.ERR_INVALID
    assert b"cols=48" in L.nvfp4moe_last_error_detail()
    assert _route_quantize(x_dtype=7) == m.ERR_INVALID
    assert _route_quantize(x=FAKE + 8) == m.ERR_INVALID          # x not 16-byte aligned
    assert _route_quantize(ws_bytes=4) == m.ERR_WORKSPACE
    assert _route_quantize(ws=None) == m.ERR_WORKSPACE
    need = L.moe_route_quantize_workspace_size(256, 256, 8)
    assert need == L.moe_route_permute_workspace_size(256, 256, 8) + 1024 * 4
    assert L.moe_route_quantize_workspace_size(0, 256, 8) == 0


def test_quantize_validation():
    L = m.lib()
    q = L.nvfp4_quantize
    assert q(None, m.BF16, 4, 64, None, None, FAKE, FAKE, FAKE, 256, None) == m.ERR_INVALID
    assert q(FAKE, 7, 4, 64, None, None, FAKE, FAKE, FAKE, 256, None) == m.ERR_INVALID
    assert q(FAKE, m.BF16, 4, 48, None, None, FAKE, FAKE, FAKE, 256, None) == m.ERR_INVALID
    assert q(FAKE, m.BF16, 0, 64, None, None, FAKE, FAKE, FAKE, 256, None) == m.ERR_INVALID
    assert q(FAKE_MIS, m.BF16, 4, 64, None, None, FAKE, FAKE, FAKE, 256, None) == m.ERR_INVALID
    assert q(FAKE, m.BF16, 4, 64, None, None, FAKE, FAKE, None, 0, None) == m.ERR_WORKSPACE
    assert q(FAKE, m.F32, 4, 64, None, None, FAKE, FAKE, FAKE, 8, None) == m.ERR_WORKSPACE


def _gemm_args(**over):
    a = m.GemmArgs(a_codes=FAKE, a_scales=FAKE, a_g=FAKE, a_rows=None, a_rows_total=16, b_codes=FAKE,
                   b_scales=FAKE, b_g=FAKE, offsets=FAKE, E=4, N=64, K=128, m_total=16,
                   epilogue=m.EPI_F32, out=FAKE, out_rows=0)
    for k_, v in over.items():
        setattr(a, k_, v)
    return a


def _gemm(**over):
    return m.lib().nvfp4_grouped_gemm(ctypes.byref(_gemm_args(**over)), None)


def test_gemm_validation():
    L = m.lib()
    assert L.nvfp4_grouped_gemm(None, None) == m.ERR_INVALID
    assert _gemm(K=48) == m.ERR_INVALID
    assert _gemm(N=24) == m.ERR_INVALID
    assert _gemm(E=0) == m.ERR_INVALID
    assert _gemm(b_codes=None) == m.ERR_INVALID
    assert _gemm(a_codes=FAKE_MIS) == m.ERR_INVALID
    assert _gemm(epilogue=9) == m.ERR_INVALID
    assert _gemm(epilogue=m.EPI_SWIGLU_NVFP4, out_codes=FAKE, out_scales=FAKE) == m.ERR_INVALID
    assert _gemm(epilogue=m.EPI_SWIGLU_NVFP4, N=48, out_codes=FAKE, out_scales=FAKE, out_g=FAKE) == m.ERR_INVALID
    assert _gemm(epilogue=m.EPI_COMBINE_F32, out_rows=4) == m.ERR_INVALID
    assert _gemm(E=1 << 16, N=1 << 16) == m.ERR_UNSUPPORTED
    assert _gemm(m_total=1 << 31) == m.ERR_UNSUPPORTED
    # 32-bit byte offsets: A codes stay below 2 GiB
    assert _gemm(a_rows_total=1 << 20, K=4096) == m.ERR_UNSUPPORTED
    # an empty problem is valid and enqueues nothing
    assert _gemm(m_total=0) == m.OK


def test_gemm_output_alignment():
    # the F32 / BF16 epilogues write rows as 16-byte vector stores
    assert _gemm(out=FAKE + 8) == m.ERR_INVALID
    assert b"out not 16-byte aligned" in m.lib().nvfp4moe_last_error_detail()
    assert _gemm(epilogue=m.EPI_BF16, out=FAKE_MIS) == m.ERR_INVALID
    assert b"out not 16-byte aligned" in m.lib().nvfp4moe_last_error_detail()


def _mx(**over):
    return m.lib().mxfp4_grouped_gemm(ctypes.byref(_gemm_args(**over)), None)


def test_mx_gemm_validation():
    L = m.lib()
    assert L.mxfp4_grouped_gemm(None, None) == m.ERR_INVALID
    assert _mx(K=48) == m.ERR_INVALID
    assert _mx(N=24) == m.ERR_INVALID
    assert _mx(E=0) == m.ERR_INVALID
    assert _mx(a_codes=FAKE_MIS) == m.ERR_INVALID
    assert _mx(out=None) == m.ERR_INVALID
    assert _mx(out=FAKE + 4) == m.ERR_INVALID
    assert b"out not 16-byte aligned" in L.nvfp4moe_last_error_detail()
    assert _mx(epilogue=m.EPI_SWIGLU_NVFP4, N=96, out_codes=FAKE, out_scales=FAKE) == m.ERR_INVALID
    assert _mx(epilogue=m.EPI_SWIGLU_NVFP4, out_codes=None, out_scales=FAKE) == m.ERR_INVALID
    assert _mx(epilogue=m.EPI_COMBINE_F32, out_rows=4, row_token=FAKE, row_weight=FAKE) == m.ERR_UNSUPPORTED


def _fp8(**over):
    a = m.Fp8GemmArgs(a_codes=FAKE, a_scales=FAKE, a_rows=None, a_rows_total=16, b_packed=FAKE, b_scales=FAKE,
                      offsets=FAKE, E=4, N=64, K=256, m_total=16, epilogue=m.EPI_BF16, out=FAKE,
                      max_rows_per_expert_hint=0)
    for k_, v in over.items():
        setattr(a, k_, v)
    return m.lib().fp8_grouped_gemm(ctypes.byref(a), None)


def test_fp8_gemm_validation():
    L = m.lib()
    assert L.fp8_grouped_gemm(None, None) == m.ERR_INVALID
    assert _fp8(K=64) == m.ERR_INVALID
    assert _fp8(N=24) == m.ERR_INVALID
    assert _fp8(E=0) == m.ERR_INVALID
    assert _fp8(b_packed=None) == m.ERR_INVALID
    assert _fp8(a_codes=FAKE_MIS) == m.ERR_INVALID
    assert _fp8(a_scales=FAKE_MIS) == m.ERR_INVALID
    assert _fp8(out=None) == m.ERR_INVALID
    assert _fp8(out=FAKE + 8) == m.ERR_INVALID
    assert b"out not 16-byte aligned" in L.nvfp4moe_last_error_detail()
    assert _fp8(epilogue=m.EPI_COMBINE_F32) == m.ERR_UNSUPPORTED
    assert _fp8(epilogue=m.EPI_SWIGLU_NVFP4) == m.ERR_INVALID              # N = 64: I not a multiple of 128
    assert _fp8(epilogue=m.EPI_SWIGLU_NVFP4, N=512) == m.ERR_INVALID       # no out_codes / out_scales
    assert _fp8(epilogue=m.EPI_SWIGLU_NVFP4, N=512, out_codes=FAKE, out_scales=FAKE_MIS) == m.ERR_INVALID
    assert _fp8(E=5000) == m.ERR_UNSUPPORTED


def test_swiglu_and_combine_validation():
    L = m.lib()
    assert L.moe_swiglu(FAKE, m.F32, 4, 24, FAKE, None, FAKE, FAKE, None, 0, None) == m.ERR_INVALID
    assert L.moe_swiglu(FAKE, m.F32, 4, 32, None, None, FAKE, FAKE, None, 0, None) == m.ERR_WORKSPACE
    assert L.moe_swiglu(None, m.F32, 4, 32, FAKE, None, FAKE, FAKE, None, 0, None) == m.ERR_INVALID
    c = L.moe_unpermute_combine
    assert c(FAKE, m.BF16, FAKE, FAKE, 4, 2, 12, FAKE, m.BF16, None) == m.ERR_INVALID
    assert c(FAKE, 5, FAKE, FAKE, 4, 2, 16, FAKE, m.BF16, None) == m.ERR_INVALID
    assert c(None, m.BF16, FAKE, FAKE, 4, 2, 16, FAKE, m.BF16, None) == m.ERR_INVALID
    assert c(FAKE, m.BF16, FAKE, FAKE, 0, 2, 16, FAKE, m.BF16, None) == m.ERR_INVALID


def test_binding_has_no_oracle_or_fallback():
    # the product path must not import the oracle or route through a CPU fallback
    import sys
    pkg = os.path.join(ROOT, "block_scaled_fp4_permute_amd")
    for f in glob.glob(os.path.join(pkg, "*.py")):
        src = open(f).read()
        assert "oracle" not in src.replace("no oracle", ""), f
        assert "import numpy" not in src, f


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(m, "_lib", None)
    monkeypatch.setattr(m, "LIB_PATH", str(tmp_path / "libnvfp4moe.so"))
    with pytest.raises(ImportError):
        m.lib()


def test_route_quantize_noalloc_validation():
    # the no-allocation variant checks the same arguments, and rejects a
    # problem whose scratch exceeds the library's fixed per-device block,
    # all before touching a device
    L = m.lib()
    cap = L.moe_route_quantize_noalloc_max_workspace()
    assert cap == 4 << 20

    def call(logits=FAKE, T=16, E=8, k=2, cols=64, x=FAKE):
        return L.moe_route_quantize_noalloc(logits, T, E, k, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, x, m.BF16,
                                            cols, None, None, FAKE, FAKE, None)
    assert call(logits=None) == m.ERR_INVALID
    assert call(k=9, E=8) == m.ERR_INVALID
    assert call(cols=48) == m.ERR_INVALID
    assert call(x=FAKE + 8) == m.ERR_INVALID
    T_big = 200_000
    assert L.moe_route_quantize_workspace_size(T_big, 256, 8) > cap
    assert call(T=T_big, E=256, k=8) == m.ERR_UNSUPPORTED
    assert b"scratch" in L.nvfp4moe_last_error_detail()
    assert L.moe_route_quantize_workspace_size(16384, 256, 8) <= cap      # the prefill workload fits


def _ffn_args(**over):
    a = m.FfnArgs(x_codes=FAKE, x_scales=FAKE, x_g=FAKE, x_rows=64, perm_src_token=FAKE, offsets=FAKE, E=8, H=512,
                  I=256, m_total=128, w_gu_packed=FAKE, g_gu=FAKE, w_dn_packed=FAKE, g_dn=FAKE, g_h=FAKE,
                  h_codes=FAKE, h_scales=FAKE, y=FAKE, max_rows_per_expert_hint=0)
    for k_, v in over.items():
        setattr(a, k_, v)
    return a


def test_expert_ffn_validation():
    L = m.lib()
    need = L.moe_expert_ffn_workspace_size(8, 128, 512, 256)
    assert need > 0 and L.moe_expert_ffn_workspace_size(0, 128, 512, 256) == 0

    def call(ws=FAKE, ws_bytes=None, **over):
        return L.moe_expert_ffn(ctypes.byref(_ffn_args(**over)), ws, need if ws_bytes is None else ws_bytes, None)
    assert L.moe_expert_ffn(None, FAKE, need, None) == m.ERR_INVALID
    assert call(x_codes=None) == m.ERR_INVALID
    assert call(y=None) == m.ERR_INVALID
    assert call(E=0) == m.ERR_INVALID
    assert call(H=500) == m.ERR_INVALID
    assert call(I=24) == m.ERR_INVALID
    assert call(I=512) == m.ERR_UNSUPPORTED          # down GEMM is one K step
    assert call(E=5000) == m.ERR_UNSUPPORTED
    assert call(x_codes=FAKE_MIS) == m.ERR_INVALID
    assert call(ws_bytes=need - 1) == m.ERR_WORKSPACE
    assert call(ws=None) == m.ERR_WORKSPACE
    assert call(ws=FAKE + 16) == m.ERR_INVALID         # workspace must be 256-byte aligned
    assert call(m_total=0) == m.OK                     # nothing to do, nothing enqueued
    # the fused combine: out needs perm_of_assignment, topk_w and T * k == m_total
    assert call(out=FAKE) == m.ERR_INVALID
    comb = dict(out=FAKE, perm_of_assignment=FAKE, topk_w=FAKE)
    assert call(T=3, k=8, **comb) == m.ERR_INVALID
    assert call(T=16, k=0, **comb) == m.ERR_INVALID
    assert call(T=16, k=8, out=FAKE_MIS, perm_of_assignment=FAKE, topk_w=FAKE) == m.ERR_INVALID
    assert call(T=16, k=8, out=FAKE, perm_of_assignment=None, topk_w=FAKE) == m.ERR_INVALID
