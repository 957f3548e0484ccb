"""Python binding of libnvfp4moe, the NVFP4 block-scaled MoE layer for MI355X.

Argument marshalling only: each function checks tensor devices/dtypes/shapes,
allocates outputs with torch (device memory is all torch is used for), and
calls the C entry point of the same name on the current HIP stream.  Every
step of the computation runs in the library's HIP kernels; there is no CPU or
eager-PyTorch fallback, and importing a function whose library is missing
raises.

C entry points (include/nvfp4moe.h): moe_route_permute, nvfp4_quantize,
nvfp4_grouped_gemm, moe_swiglu, moe_unpermute_combine, moe_route_quantize
(routing and activation quantisation in shared launches) and moe_expert_ffn
(gate_up + SwiGLU requant + down for all experts, one persistent launch at
decode sizes).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libnvfp4moe.so")

OK, ERR_INVALID, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = range(5)
F32, BF16 = 0, 1
EPI_F32, EPI_BF16, EPI_SWIGLU_NVFP4, EPI_COMBINE_F32 = range(4)


class NVFP4MoEError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"nvfp4moe status {status}: {detail}")
        self.status = status
        self.detail = detail


class FfnArgs(ctypes.Structure):
    """Mirror of nvfp4moe_ffn_args."""
    _fields_ = [
        ("x_codes", ctypes.c_void_p), ("x_scales", ctypes.c_void_p), ("x_g", ctypes.c_void_p),
        ("x_rows", ctypes.c_int64), ("perm_src_token", ctypes.c_void_p), ("offsets", ctypes.c_void_p),
        ("E", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32), ("m_total", ctypes.c_int64),
        ("w_gu_packed", ctypes.c_void_p), ("g_gu", ctypes.c_void_p),
        ("w_dn_packed", ctypes.c_void_p), ("g_dn", ctypes.c_void_p), ("g_h", ctypes.c_void_p),
        ("h_codes", ctypes.c_void_p), ("h_scales", ctypes.c_void_p), ("y", ctypes.c_void_p),
        ("max_rows_per_expert_hint", ctypes.c_int32),
        ("out", ctypes.c_void_p), ("perm_of_assignment", ctypes.c_void_p), ("topk_w", ctypes.c_void_p),
        ("T", ctypes.c_int32), ("k", ctypes.c_int32),
    ]


class GemmArgs(ctypes.Structure):
    """Mirror of nvfp4moe_gemm_args."""
    _fields_ = [
        ("a_codes", ctypes.c_void_p), ("a_scales", ctypes.c_void_p), ("a_g", ctypes.c_void_p),
        ("a_rows", ctypes.c_void_p), ("a_rows_total", ctypes.c_int64),
        ("b_codes", ctypes.c_void_p), ("b_scales", ctypes.c_void_p), ("b_g", ctypes.c_void_p),
        ("offsets", ctypes.c_void_p),
        ("E", ctypes.c_int32), ("N", ctypes.c_int32), ("K", ctypes.c_int32),
        ("m_total", ctypes.c_int64), ("epilogue", ctypes.c_int32),
        ("out", ctypes.c_void_p), ("out_rows", ctypes.c_int64),
        ("out_codes", ctypes.c_void_p), ("out_scales", ctypes.c_void_p), ("out_g", ctypes.c_void_p),
        ("row_token", ctypes.c_void_p), ("row_weight", ctypes.c_void_p),
        ("max_rows_per_expert_hint", ctypes.c_int32),
        ("b_packed", ctypes.c_void_p),
    ]


class Fp8GemmArgs(ctypes.Structure):
    """Mirror of nvfp4moe_fp8_gemm_args."""
    _fields_ = [
        ("a_codes", ctypes.c_void_p), ("a_scales", ctypes.c_void_p), ("a_rows", ctypes.c_void_p),
        ("a_rows_total", ctypes.c_int64), ("b_packed", ctypes.c_void_p), ("b_scales", ctypes.c_void_p),
        ("offsets", ctypes.c_void_p), ("E", ctypes.c_int32), ("N", ctypes.c_int32), ("K", ctypes.c_int32),
        ("m_total", ctypes.c_int64), ("epilogue", ctypes.c_int32), ("out", ctypes.c_void_p),
        ("max_rows_per_expert_hint", ctypes.c_int32), ("out_codes", ctypes.c_void_p), ("out_scales", ctypes.c_void_p),
    ]


_lib = None

_SIGNATURES = {
    "moe_route_permute_workspace_size": (ctypes.c_size_t, [ctypes.c_int32] * 3),
    "moe_route_permute": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
                          + [ctypes.c_void_p] * 8 + [ctypes.c_size_t, ctypes.c_void_p]),
    "nvfp4_quantize_workspace_size": (ctypes.c_size_t, []),
    "nvfp4_quantize": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64]
                       + [ctypes.c_void_p] * 5 + [ctypes.c_size_t, ctypes.c_void_p]),
    "nvfp4_grouped_gemm": (ctypes.c_int, [ctypes.POINTER(GemmArgs), ctypes.c_void_p]),
    "nvfp4_weight_packed_size": (ctypes.c_size_t, [ctypes.c_int32] * 3),
    "nvfp4_weight_repack": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "moe_swiglu_workspace_size": (ctypes.c_size_t, []),
    "moe_swiglu": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32]
                   + [ctypes.c_void_p] * 5 + [ctypes.c_size_t, ctypes.c_void_p]),
    "moe_unpermute_combine": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                             ctypes.c_int32, ctypes.c_void_p]),
    "moe_route_quantize_workspace_size": (ctypes.c_size_t, [ctypes.c_int32] * 3),
    "moe_route_quantize": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
                           + [ctypes.c_void_p] * 7 + [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64]
                           + [ctypes.c_void_p] * 4 + [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "moe_route_quantize_noalloc_max_workspace": (ctypes.c_size_t, []),
    "moe_route_quantize_noalloc": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
                                   + [ctypes.c_void_p] * 7 + [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64]
                                   + [ctypes.c_void_p] * 4 + [ctypes.c_void_p]),
    "moe_expert_ffn_workspace_size": (ctypes.c_size_t, [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                                                        ctypes.c_int32]),
    "moe_expert_ffn": (ctypes.c_int, [ctypes.POINTER(FfnArgs), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "mxfp4_quantize": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "mxfp4_grouped_gemm": (ctypes.c_int, [ctypes.POINTER(GemmArgs), ctypes.c_void_p]),
    "mxfp4_weight_packed_size": (ctypes.c_size_t, [ctypes.c_int32] * 3),
    "mxfp4_weight_repack": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "fp8_quantize": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                    ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "fp8_swiglu_quantize": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                                           ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "fp8_weight_packed_size": (ctypes.c_size_t, [ctypes.c_int32] * 3),
    "fp8_weight_repack": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                         ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "fp8_grouped_gemm": (ctypes.c_int, [ctypes.POINTER(Fp8GemmArgs), ctypes.c_void_p]),
    "nvfp4moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "nvfp4moe_last_error_detail": (ctypes.c_char_p, []),
    "nvfp4moe_version": (ctypes.c_int, []),
}


def lib() -> ctypes.CDLL:
    """Load libnvfp4moe.so (built in-tree by block_scaled_fp4_permute_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: run `python -m block_scaled_fp4_permute_amd.build` "
                              "(there is no fallback implementation)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(status: int):
    if status != OK:
        detail = lib().nvfp4moe_last_error_detail().decode()
        raise NVFP4MoEError(status, detail)


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _need(t, dtype, name, device=None):
    import torch
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")


def _dtype_code(t):
    import torch
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


# --------------------------------------------------------------------------- route
@dataclass
class Routing:
    topk_ids: "object"
    topk_w: "object"
    counts: "object"
    offsets: "object"
    perm_src_token: "object"
    perm_of_assignment: "object"
    perm_weight: "object"


def moe_route_permute(logits, k: int, out: Routing | None = None, workspace=None, stream=None) -> Routing:
    """logits float32 [T, E] -> Routing (see include/nvfp4moe.h)."""
    import torch
    _need(logits, torch.float32, "logits")
    T, E = logits.shape
    dev = logits.device
    if out is None:
        i32 = dict(dtype=torch.int32, device=dev)
        out = Routing(torch.empty((T, k), **i32), torch.empty((T, k), dtype=torch.float32, device=dev),
                      torch.empty(E, **i32), torch.empty(E + 1, **i32), torch.empty(T * k, **i32),
                      torch.empty(T * k, **i32), torch.empty(T * k, dtype=torch.float32, device=dev))
    nbytes = lib().moe_route_permute_workspace_size(T, E, k)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
    _check(lib().moe_route_permute(
        logits.data_ptr(), T, E, k, out.topk_ids.data_ptr(), out.topk_w.data_ptr(), out.counts.data_ptr(),
        out.offsets.data_ptr(), out.perm_src_token.data_ptr(), out.perm_of_assignment.data_ptr(),
        _ptr(out.perm_weight), workspace.data_ptr(), workspace.numel(), _stream(stream)))
    return out


# ------------------------------------------------------------------------ quantise
@dataclass
class NVFP4Tensor:
    codes: "object"     # uint8 [rows, cols/2]
    scales: "object"    # uint8 [rows, cols/16]
    g: "object"         # float32 [1] (device)


def nvfp4_quantize(x, g=None, out: NVFP4Tensor | None = None, workspace=None, stream=None) -> NVFP4Tensor:
    """x bf16/float32 [rows, cols] -> NVFP4Tensor.  g: optional device float32[1]
    per-tensor scale (None: amax/2688 computed on the device)."""
    import torch
    if x.dim() != 2:
        raise ValueError("x must be 2-D")
    _need(x, x.dtype, "x")
    rows, cols = x.shape
    dev = x.device
    if out is None:
        out = NVFP4Tensor(torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev),
                          torch.empty((rows, cols // 16), dtype=torch.uint8, device=dev),
                          torch.empty(1, dtype=torch.float32, device=dev))
    if workspace is None:
        workspace = torch.empty(lib().nvfp4_quantize_workspace_size(), dtype=torch.uint8, device=dev)
    _check(lib().nvfp4_quantize(x.data_ptr(), _dtype_code(x), rows, cols, _ptr(g), _ptr(out.g),
                                out.codes.data_ptr(), out.scales.data_ptr(), workspace.data_ptr(),
                                workspace.numel(), _stream(stream)))
    return out


# ------------------------------------------------------------------ packed weights
def nvfp4_weight_repack(codes, scales, out=None, stream=None):
    """Row-major NVFP4 weights codes uint8 [E, N, K/2], scales uint8 [E, N, K/16]
    -> packed tile layout (uint8 tensor) read by nvfp4_grouped_gemm(b_packed=...)."""
    import torch
    _need(codes, torch.uint8, "codes")
    _need(scales, torch.uint8, "scales")
    E, N, K2 = codes.shape
    nbytes = lib().nvfp4_weight_packed_size(E, N, 2 * K2)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=codes.device)
    _check(lib().nvfp4_weight_repack(codes.data_ptr(), scales.data_ptr(), E, N, 2 * K2, out.data_ptr(),
                                     out.numel(), _stream(stream)))
    return out


# ------------------------------------------------------------------ route + quantise
def moe_route_quantize(logits, k: int, x, g=None, out: Routing | None = None, xq: NVFP4Tensor | None = None,
                       workspace=None, stream=None) -> tuple[Routing, NVFP4Tensor]:
    """moe_route_permute(logits, k) and nvfp4_quantize(x, g) in one call whose
    kernels share launches; the outputs are those of the two calls."""
    import torch
    _need(logits, torch.float32, "logits")
    _need(x, x.dtype, "x")
    T, E = logits.shape
    if x.dim() != 2 or x.shape[0] != T:
        raise ValueError("x must be [T, cols] with the logits' T rows")
    cols = x.shape[1]
    dev = logits.device
    if out is None:
        i32 = dict(dtype=torch.int32, device=dev)
        out = Routing(torch.empty((T, k), **i32), torch.empty((T, k), dtype=torch.float32, device=dev),
                      torch.empty(E, **i32), torch.empty(E + 1, **i32), torch.empty(T * k, **i32),
                      torch.empty(T * k, **i32), torch.empty(T * k, dtype=torch.float32, device=dev))
    if xq is None:
        xq = NVFP4Tensor(torch.empty((T, cols // 2), dtype=torch.uint8, device=dev),
                         torch.empty((T, cols // 16), dtype=torch.uint8, device=dev),
                         torch.empty(1, dtype=torch.float32, device=dev))
    nbytes = lib().moe_route_quantize_workspace_size(T, E, k)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
    _check(lib().moe_route_quantize(
        logits.data_ptr(), T, E, k, out.topk_ids.data_ptr(), out.topk_w.data_ptr(), out.counts.data_ptr(),
        out.offsets.data_ptr(), out.perm_src_token.data_ptr(), out.perm_of_assignment.data_ptr(),
        _ptr(out.perm_weight), x.data_ptr(), _dtype_code(x), cols, _ptr(g), _ptr(xq.g), xq.codes.data_ptr(),
        xq.scales.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream(stream)))
    return out, xq


def moe_route_quantize_noalloc(logits, k: int, x, out: Routing, xq: NVFP4Tensor, g=None, stream=None):
    """moe_route_quantize with the library's per-device scratch instead of a
    workspace: allocates nothing (outputs are the caller's ``out`` and ``xq``)."""
    import torch
    _need(logits, torch.float32, "logits")
    _need(x, x.dtype, "x")
    T, E = logits.shape
    if x.dim() != 2 or x.shape[0] != T:
        raise ValueError("x must be [T, cols] with the logits' T rows")
    cols = x.shape[1]
    if tuple(out.topk_ids.shape) != (T, k) or out.perm_src_token.numel() < T * k or out.offsets.numel() < E + 1:
        raise ValueError("routing outputs do not match T, E, k")
    if tuple(xq.codes.shape) != (T, cols // 2) or tuple(xq.scales.shape) != (T, cols // 16):
        raise ValueError("xq does not match x")
    _check(lib().moe_route_quantize_noalloc(
        logits.data_ptr(), T, E, k, out.topk_ids.data_ptr(), out.topk_w.data_ptr(), out.counts.data_ptr(),
        out.offsets.data_ptr(), out.perm_src_token.data_ptr(), out.perm_of_assignment.data_ptr(),
        _ptr(out.perm_weight), x.data_ptr(), _dtype_code(x), cols, _ptr(g), _ptr(xq.g), xq.codes.data_ptr(),
        xq.scales.data_ptr(), _stream(stream)))
    return out, xq


# ---------------------------------------------------------------------------- gemm
def nvfp4_grouped_gemm(a: NVFP4Tensor, b_codes, b_scales, b_g, offsets, *, m_total: int, a_rows=None,
                       epilogue: int = EPI_F32, out=None, out_rows: int = 0, out_codes=None,
                       out_scales=None, out_g=None, row_token=None, row_weight=None,
                       max_rows_per_expert_hint: int = 0, b_packed=None, stream=None):
    """Grouped NVFP4 GEMM (see include/nvfp4moe.h).  b_codes uint8 [E, N, K/2],
    b_scales uint8 [E, N, K/16], b_g float32 [E], offsets int32 [E+1] (device).
    With b_packed (from nvfp4_weight_repack), b_codes/b_scales give only the
    shapes (they may be meta or empty-strided tensors) and are not read."""
    import torch
    E, N, K2 = b_codes.shape
    K = 2 * K2
    _need(a.codes, torch.uint8, "a.codes")
    _need(a.scales, torch.uint8, "a.scales")
    if b_packed is None:
        _need(b_codes, torch.uint8, "b_codes")
        _need(b_scales, torch.uint8, "b_scales")
    else:
        _need(b_packed, torch.uint8, "b_packed")
        if b_packed.numel() < lib().nvfp4_weight_packed_size(E, N, K):
            raise ValueError("b_packed is smaller than the packed size of [E, N, K]")
    _need(b_g, torch.float32, "b_g")
    _need(offsets, torch.int32, "offsets")
    if a.codes.shape[1] != K2 or tuple(b_scales.shape) != (E, N, K // 16):
        raise ValueError("operand shapes disagree")
    a_rows_total = a.codes.shape[0]
    if tuple(a.scales.shape) != (a_rows_total, K // 16):
        raise ValueError(f"a.scales: expected [{a_rows_total}, {K // 16}], got {list(a.scales.shape)}")
    if a.g.numel() < 1 or b_g.numel() < E:
        raise ValueError("a.g needs 1 and b_g needs E float32 values")
    if offsets.numel() < E + 1:
        raise ValueError(f"offsets: {offsets.numel()} values, expected E+1 = {E + 1}")
    if a_rows is not None:
        _need(a_rows, torch.int32, "a_rows")
        if a_rows.numel() < m_total:
            raise ValueError(f"a_rows: {a_rows.numel()} values, expected m_total = {m_total}")
    dev = b_codes.device
    I = N // 2
    if epilogue in (EPI_F32, EPI_BF16):
        want = torch.float32 if epilogue == EPI_F32 else torch.bfloat16
        if out is None:
            out = torch.empty((m_total, N), dtype=want, device=dev)
        else:
            _need(out, want, "out")
            if tuple(out.shape) != (m_total, N):
                raise ValueError(f"out: expected [{m_total}, {N}], got {list(out.shape)}")
    if epilogue == EPI_SWIGLU_NVFP4:
        if out_g is None:
            raise ValueError("EPI_SWIGLU_NVFP4 needs out_g (the per-tensor scale of h)")
        _need(out_g, torch.float32, "out_g")
        if out_codes is None:
            out_codes = torch.empty((m_total, I // 2), dtype=torch.uint8, device=dev)
            out_scales = torch.empty((m_total, I // 16), dtype=torch.uint8, device=dev)
        _need(out_codes, torch.uint8, "out_codes")
        _need(out_scales, torch.uint8, "out_scales")
        if tuple(out_codes.shape) != (m_total, I // 2) or tuple(out_scales.shape) != (m_total, I // 16):
            raise ValueError(f"out_codes/out_scales: expected [{m_total}, {I // 2}] and [{m_total}, {I // 16}]")
    if epilogue == EPI_COMBINE_F32:
        if out is None or row_token is None or row_weight is None:
            raise ValueError("EPI_COMBINE_F32 needs out, row_token and row_weight")
        _need(out, torch.float32, "out")
        _need(row_token, torch.int32, "row_token")
        _need(row_weight, torch.float32, "row_weight")
        if tuple(out.shape) != (out_rows, N) or row_token.numel() < m_total or row_weight.numel() < m_total:
            raise ValueError(f"combine epilogue: out must be [out_rows={out_rows}, {N}], row_token and row_weight "
                             f"at least m_total = {m_total} long")
    args = GemmArgs(
        a_codes=a.codes.data_ptr(), a_scales=a.scales.data_ptr(), a_g=a.g.data_ptr(), a_rows=_ptr(a_rows),
        a_rows_total=a_rows_total,
        b_codes=None if b_packed is not None else b_codes.data_ptr(),
        b_scales=None if b_packed is not None else b_scales.data_ptr(), b_packed=_ptr(b_packed),
        b_g=b_g.data_ptr(), offsets=offsets.data_ptr(), E=E, N=N, K=K, m_total=m_total, epilogue=epilogue,
        out=_ptr(out), out_rows=out_rows, out_codes=_ptr(out_codes), out_scales=_ptr(out_scales),
        out_g=_ptr(out_g), row_token=_ptr(row_token), row_weight=_ptr(row_weight),
        max_rows_per_expert_hint=max_rows_per_expert_hint)
    _check(lib().nvfp4_grouped_gemm(ctypes.byref(args), _stream(stream)))
    if epilogue == EPI_SWIGLU_NVFP4:
        return NVFP4Tensor(out_codes, out_scales, out_g)
    return out


# ---------------------------------------------------------------------- expert FFN
def moe_expert_ffn_workspace(E: int, m_total: int, H: int, I: int, device):
    import torch
    n = lib().moe_expert_ffn_workspace_size(E, m_total, H, I)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def moe_expert_ffn(xq: NVFP4Tensor, perm_src_token, offsets, w_gu_packed, g_gu, w_dn_packed, g_dn, g_h, *, H: int,
                   I: int, m_total: int, h: NVFP4Tensor | None = None, y=None, workspace=None,
                   max_rows_per_expert_hint: int = 0, perm_of_assignment=None, topk_w=None, k: int = 0, out=None,
                   stream=None):
    """gate_up + SwiGLU/requant + down for all experts (see include/nvfp4moe.h):
    returns (h NVFP4Tensor [m_total, I], y bf16 [m_total, H]); with
    perm_of_assignment, topk_w ([T, k]) and k also the weighted top-k combine
    out bf16 [T, H] (fused into the launch in the one-launch regime), returned
    as a third element."""
    import torch
    E = offsets.numel() - 1
    dev = offsets.device
    _need(xq.codes, torch.uint8, "x codes")
    _need(xq.scales, torch.uint8, "x scales")
    if tuple(xq.codes.shape[1:]) != (H // 2,) or tuple(xq.scales.shape) != (xq.codes.shape[0], H // 16):
        raise ValueError("x codes/scales do not match H")
    _need(perm_src_token, torch.int32, "perm_src_token")
    _need(offsets, torch.int32, "offsets")
    if perm_src_token.numel() < m_total:
        raise ValueError("perm_src_token shorter than m_total")
    for t, name, n in ((w_gu_packed, "w_gu_packed", lib().nvfp4_weight_packed_size(E, 2 * I, H)),
                       (w_dn_packed, "w_dn_packed", lib().nvfp4_weight_packed_size(E, H, I))):
        _need(t, torch.uint8, name)
        if t.numel() < n:
            raise ValueError(f"{name}: {t.numel()} bytes, the packed size is {n}")
    for t, name, n in ((g_gu, "g_gu", E), (g_dn, "g_dn", E), (g_h, "g_h", 1)):
        _need(t, torch.float32, name)
        if t.numel() < n:
            raise ValueError(f"{name}: needs {n} values")
    if h is None:
        h = NVFP4Tensor(torch.empty((m_total, I // 2), dtype=torch.uint8, device=dev),
                        torch.empty((m_total, I // 16), dtype=torch.uint8, device=dev), g_h)
    if tuple(h.codes.shape) != (m_total, I // 2) or tuple(h.scales.shape) != (m_total, I // 16):
        raise ValueError("h codes/scales must be [m_total, I/2] and [m_total, I/16]")
    if y is None:
        y = torch.empty((m_total, H), dtype=torch.bfloat16, device=dev)
    _need(y, torch.bfloat16, "y")
    if tuple(y.shape) != (m_total, H):
        raise ValueError("y must be bf16 [m_total, H]")
    T = 0
    if perm_of_assignment is not None:
        if topk_w is None or k <= 0 or m_total % k:
            raise ValueError("the combine needs topk_w and k > 0 dividing m_total")
        T = m_total // k
        _need(perm_of_assignment, torch.int32, "perm_of_assignment")
        _need(topk_w, torch.float32, "topk_w")
        if perm_of_assignment.numel() < m_total or topk_w.numel() < m_total:
            raise ValueError("perm_of_assignment and topk_w need T * k values")
        if out is None:
            out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        _need(out, torch.bfloat16, "out")
        if tuple(out.shape) != (T, H):
            raise ValueError("out must be bf16 [T, H]")
    if workspace is None:
        workspace = moe_expert_ffn_workspace(E, m_total, H, I, dev)
    args = FfnArgs(x_codes=xq.codes.data_ptr(), x_scales=xq.scales.data_ptr(), x_g=xq.g.data_ptr(),
                   x_rows=xq.codes.shape[0], perm_src_token=perm_src_token.data_ptr(), offsets=offsets.data_ptr(),
                   E=E, H=H, I=I, m_total=m_total, w_gu_packed=w_gu_packed.data_ptr(), g_gu=g_gu.data_ptr(),
                   w_dn_packed=w_dn_packed.data_ptr(), g_dn=g_dn.data_ptr(), g_h=g_h.data_ptr(),
                   h_codes=h.codes.data_ptr(), h_scales=h.scales.data_ptr(), y=y.data_ptr(),
                   max_rows_per_expert_hint=max_rows_per_expert_hint,
                   out=out.data_ptr() if T else None,
                   perm_of_assignment=perm_of_assignment.data_ptr() if T else None,
                   topk_w=topk_w.data_ptr() if T else None, T=T, k=k if T else 0)
    _check(lib().moe_expert_ffn(ctypes.byref(args), workspace.data_ptr(), workspace.numel(), _stream(stream)))
    if T:
        return NVFP4Tensor(h.codes, h.scales, g_h), y, out
    return NVFP4Tensor(h.codes, h.scales, g_h), y


# --------------------------------------------------------------------------- MXFP4
@dataclass
class MXFP4Tensor:
    codes: "object"     # uint8 [rows, cols/2]
    scales: "object"    # uint8 [rows, cols/32], E8M0


def mxfp4_quantize(x, out: MXFP4Tensor | None = None, stream=None) -> MXFP4Tensor:
    """x bf16/float32 [rows, cols] (or [..., cols]) -> MXFP4Tensor (E8M0 scale per 32 values)."""
    import torch
    _need(x, x.dtype, "x")
    cols = x.shape[-1]
    rows = x.numel() // cols
    dev = x.device
    if out is None:
        out = MXFP4Tensor(torch.empty(x.shape[:-1] + (cols // 2,), dtype=torch.uint8, device=dev),
                          torch.empty(x.shape[:-1] + (cols // 32,), dtype=torch.uint8, device=dev))
    if out.codes.numel() != rows * (cols // 2) or out.scales.numel() != rows * (cols // 32):
        raise ValueError("out codes/scales do not match x")
    _need(out.codes, torch.uint8, "out.codes")
    _need(out.scales, torch.uint8, "out.scales")
    _check(lib().mxfp4_quantize(x.data_ptr(), _dtype_code(x), rows, cols, out.codes.data_ptr(), out.scales.data_ptr(),
                                _stream(stream)))
    return out


def mxfp4_weight_repack(b: MXFP4Tensor, out=None, stream=None):
    """MXFP4 weights codes [E, N, K/2], scales [E, N, K/32] -> packed tiles
    (uint8 tensor) for mxfp4_grouped_gemm(b_packed=...)."""
    import torch
    _need(b.codes, torch.uint8, "codes")
    _need(b.scales, torch.uint8, "scales")
    E, N, K2 = b.codes.shape
    nbytes = lib().mxfp4_weight_packed_size(E, N, 2 * K2)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=b.codes.device)
    _check(lib().mxfp4_weight_repack(b.codes.data_ptr(), b.scales.data_ptr(), E, N, 2 * K2, out.data_ptr(),
                                     out.numel(), _stream(stream)))
    return out


def mxfp4_grouped_gemm(a: MXFP4Tensor, b: MXFP4Tensor, offsets, *, m_total: int, a_rows=None, epilogue: int = EPI_F32,
                       out=None, out_codes=None, out_scales=None, a_g=None, b_g=None,
                       max_rows_per_expert_hint: int = 0, b_packed=None, stream=None):
    """Grouped MXFP4 GEMM (see include/nvfp4moe.h): a [rows, K], b [E, N, K]
    (codes/scales), offsets int32 [E+1].  Epilogues F32, BF16, or
    EPI_SWIGLU_NVFP4 read as SwiGLU + MXFP4 requantisation (returns an
    MXFP4Tensor of h).  a_g / b_g: optional float32 multipliers (1 / E values)."""
    import torch
    E, N, K2 = b.codes.shape
    K = 2 * K2
    dev = b.codes.device
    for t, name in ((a.codes, "a.codes"), (a.scales, "a.scales")):
        _need(t, torch.uint8, name)
    if b_packed is None:
        _need(b.codes, torch.uint8, "b.codes")
        _need(b.scales, torch.uint8, "b.scales")
    else:
        _need(b_packed, torch.uint8, "b_packed")
        if b_packed.numel() < lib().mxfp4_weight_packed_size(E, N, K):
            raise ValueError("b_packed is smaller than the packed size of [E, N, K]")
    _need(offsets, torch.int32, "offsets")
    rows_a = a.codes.shape[0]
    if tuple(a.codes.shape) != (rows_a, K2) or tuple(a.scales.shape) != (rows_a, K // 32) \
            or tuple(b.scales.shape) != (E, N, K // 32):
        raise ValueError("operand shapes disagree")
    if offsets.numel() < E + 1:
        raise ValueError("offsets needs E+1 values")
    if a_rows is not None:
        _need(a_rows, torch.int32, "a_rows")
        if a_rows.numel() < m_total:
            raise ValueError("a_rows shorter than m_total")
    if a_g is None:
        a_g = torch.ones(1, dtype=torch.float32, device=dev)
    if b_g is None:
        b_g = torch.ones(E, dtype=torch.float32, device=dev)
    _need(a_g, torch.float32, "a_g")
    _need(b_g, torch.float32, "b_g")
    I = N // 2
    if epilogue in (EPI_F32, EPI_BF16):
        want = torch.float32 if epilogue == EPI_F32 else torch.bfloat16
        if out is None:
            out = torch.empty((m_total, N), dtype=want, device=dev)
        _need(out, want, "out")
        if tuple(out.shape) != (m_total, N):
            raise ValueError("out must be [m_total, N]")
    elif epilogue == EPI_SWIGLU_NVFP4:
        if out_codes is None:
            out_codes = torch.empty((m_total, I // 2), dtype=torch.uint8, device=dev)
            out_scales = torch.empty((m_total, I // 32), dtype=torch.uint8, device=dev)
        if tuple(out_codes.shape) != (m_total, I // 2) or tuple(out_scales.shape) != (m_total, I // 32):
            raise ValueError("out_codes/out_scales must be [m_total, I/2] and [m_total, I/32]")
    args = GemmArgs(a_codes=a.codes.data_ptr(), a_scales=a.scales.data_ptr(), a_g=a_g.data_ptr(), a_rows=_ptr(a_rows),
                    a_rows_total=rows_a, b_codes=None if b_packed is not None else b.codes.data_ptr(),
                    b_scales=None if b_packed is not None else b.scales.data_ptr(), b_packed=_ptr(b_packed),
                    b_g=b_g.data_ptr(), offsets=offsets.data_ptr(), E=E, N=N, K=K, m_total=m_total,
                    epilogue=epilogue, out=_ptr(out), out_rows=0, out_codes=_ptr(out_codes),
                    out_scales=_ptr(out_scales), out_g=None, row_token=None, row_weight=None,
                    max_rows_per_expert_hint=max_rows_per_expert_hint)
    _check(lib().mxfp4_grouped_gemm(ctypes.byref(args), _stream(stream)))
    if epilogue == EPI_SWIGLU_NVFP4:
        return MXFP4Tensor(out_codes, out_scales)
    return out


# --------------------------------------------------------------------------- FP8
FP8_BLOCK = 128


@dataclass
class FP8Tensor:
    codes: "object"     # uint8 [..., rows, cols], E4M3 bytes
    scales: "object"    # float32 [..., ceil(rows/block_rows), cols/128]
    block_rows: int     # 1 (activations) or 128 (weights)


def fp8_quantize(x, block_rows: int = 1, out: FP8Tensor | None = None, stream=None) -> FP8Tensor:
    """x bf16/float32 [rows, cols] (block_rows 1) or [batch, rows, cols]
    (block_rows 128: one scale per 128 x 128 tile of each matrix) -> FP8Tensor."""
    import torch
    _need(x, x.dtype, "x")
    cols = x.shape[-1]
    if block_rows == 1:
        batch, rows = 1, x.numel() // cols
        sshape = x.shape[:-1] + (cols // FP8_BLOCK,)
    else:
        rows = x.shape[-2]
        batch = x.numel() // (rows * cols)
        sshape = x.shape[:-2] + ((rows + FP8_BLOCK - 1) // FP8_BLOCK, cols // FP8_BLOCK)
    dev = x.device
    if out is None:
        out = FP8Tensor(torch.empty(x.shape, dtype=torch.uint8, device=dev),
                        torch.empty(sshape, dtype=torch.float32, device=dev), block_rows)
    if out.codes.numel() != x.numel() or tuple(out.scales.shape) != tuple(sshape):
        raise ValueError("out codes/scales do not match x")
    _need(out.codes, torch.uint8, "out.codes")
    _need(out.scales, torch.float32, "out.scales")
    _check(lib().fp8_quantize(x.data_ptr(), _dtype_code(x), batch, rows, cols, block_rows, out.codes.data_ptr(),
                              out.scales.data_ptr(), _stream(stream)))
    return out


def fp8_swiglu_quantize(gate_up, out: FP8Tensor | None = None, stream=None) -> FP8Tensor:
    """gate_up float32/bf16 [M, 2I] -> FP8 h = silu(gate) * up with 1 x 128 blocks."""
    import torch
    _need(gate_up, gate_up.dtype, "gate_up")
    M, N2 = gate_up.shape
    I = N2 // 2
    dev = gate_up.device
    if out is None:
        out = FP8Tensor(torch.empty((M, I), dtype=torch.uint8, device=dev),
                        torch.empty((M, I // FP8_BLOCK), dtype=torch.float32, device=dev), 1)
    if tuple(out.codes.shape) != (M, I) or tuple(out.scales.shape) != (M, I // FP8_BLOCK):
        raise ValueError("out codes/scales must be [M, I] and [M, I/128]")
    _need(out.codes, torch.uint8, "out.codes")
    _need(out.scales, torch.float32, "out.scales")
    _check(lib().fp8_swiglu_quantize(gate_up.data_ptr(), _dtype_code(gate_up), M, I, out.codes.data_ptr(),
                                     out.scales.data_ptr(), _stream(stream)))
    return out


def fp8_weight_repack(codes, out=None, stream=None):
    """FP8 weight codes [E, N, K] -> packed tiles (uint8 tensor) for fp8_grouped_gemm."""
    import torch
    _need(codes, torch.uint8, "codes")
    E, N, K = codes.shape
    nbytes = lib().fp8_weight_packed_size(E, N, K)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=codes.device)
    _check(lib().fp8_weight_repack(codes.data_ptr(), E, N, K, out.data_ptr(), out.numel(), _stream(stream)))
    return out


def fp8_grouped_gemm(a: FP8Tensor, b_packed, b_scales, offsets, *, N: int, m_total: int, a_rows=None,
                     epilogue: int = EPI_F32, out=None, max_rows_per_expert_hint: int = 0, stream=None):
    """Grouped FP8 GEMM (see include/nvfp4moe.h): a [rows, K] (1 x 128 blocks),
    b_packed from fp8_weight_repack, b_scales float32 [E, ceil(N/128), K/128],
    offsets int32 [E+1].  Epilogues F32 or BF16 (returns out), or
    EPI_SWIGLU_NVFP4 read as SwiGLU + FP8 requant of h (N = 2I, I % 128 == 0;
    out: an FP8Tensor for h or None; returns it)."""
    import torch
    rows_a, K = a.codes.shape
    E = b_scales.shape[0]
    dev = a.codes.device
    if a.block_rows != 1:
        raise ValueError("A must be quantised with 1 x 128 blocks")
    _need(a.codes, torch.uint8, "a.codes")
    _need(a.scales, torch.float32, "a.scales")
    _need(b_packed, torch.uint8, "b_packed")
    _need(b_scales, torch.float32, "b_scales")
    _need(offsets, torch.int32, "offsets")
    if tuple(a.scales.shape) != (rows_a, K // FP8_BLOCK) or \
            tuple(b_scales.shape) != (E, (N + FP8_BLOCK - 1) // FP8_BLOCK, K // FP8_BLOCK):
        raise ValueError("operand shapes disagree")
    if b_packed.numel() < lib().fp8_weight_packed_size(E, N, K):
        raise ValueError("b_packed is smaller than the packed size of [E, N, K]")
    if offsets.numel() < E + 1:
        raise ValueError("offsets needs E+1 values")
    if a_rows is not None:
        _need(a_rows, torch.int32, "a_rows")
        if a_rows.numel() < m_total:
            raise ValueError("a_rows shorter than m_total")
    if epilogue == EPI_SWIGLU_NVFP4:
        if N % (2 * FP8_BLOCK) != 0:
            raise ValueError("fp8_grouped_gemm: SwiGLU needs N = 2I with I % 128 == 0")
        I = N // 2
        if out is None:
            out = FP8Tensor(torch.empty((m_total, I), dtype=torch.uint8, device=dev),
                            torch.empty((m_total, I // FP8_BLOCK), dtype=torch.float32, device=dev), 1)
        _need(out.codes, torch.uint8, "out.codes")
        _need(out.scales, torch.float32, "out.scales")
        if tuple(out.codes.shape) != (m_total, I) or tuple(out.scales.shape) != (m_total, I // FP8_BLOCK):
            raise ValueError("out codes/scales must be [m_total, I] and [m_total, I/128]")
        args = Fp8GemmArgs(a_codes=a.codes.data_ptr(), a_scales=a.scales.data_ptr(), a_rows=_ptr(a_rows),
                           a_rows_total=rows_a, b_packed=b_packed.data_ptr(), b_scales=b_scales.data_ptr(),
                           offsets=offsets.data_ptr(), E=E, N=N, K=K, m_total=m_total, epilogue=epilogue, out=None,
                           max_rows_per_expert_hint=max_rows_per_expert_hint, out_codes=out.codes.data_ptr(),
                           out_scales=out.scales.data_ptr())
        _check(lib().fp8_grouped_gemm(ctypes.byref(args), _stream(stream)))
        return out
    if epilogue not in (EPI_F32, EPI_BF16):
        raise ValueError("fp8_grouped_gemm: epilogue F32, BF16 or SwiGLU")
    want = torch.float32 if epilogue == EPI_F32 else torch.bfloat16
    if out is None:
        out = torch.empty((m_total, N), dtype=want, device=dev)
    _need(out, want, "out")
    if tuple(out.shape) != (m_total, N):
        raise ValueError("out must be [m_total, N]")
    args = Fp8GemmArgs(a_codes=a.codes.data_ptr(), a_scales=a.scales.data_ptr(), a_rows=_ptr(a_rows),
                       a_rows_total=rows_a, b_packed=b_packed.data_ptr(), b_scales=b_scales.data_ptr(),
                       offsets=offsets.data_ptr(), E=E, N=N, K=K, m_total=m_total, epilogue=epilogue,
                       out=out.data_ptr(), max_rows_per_expert_hint=max_rows_per_expert_hint)
    _check(lib().fp8_grouped_gemm(ctypes.byref(args), _stream(stream)))
    return out


# -------------------------------------------------------------------------- swiglu
def moe_swiglu(gate_up, g=None, out: NVFP4Tensor | None = None, workspace=None, stream=None) -> NVFP4Tensor:
    """gate_up float32/bf16 [M, 2I] -> NVFP4 h = silu(gate) * up."""
    import torch
    _need(gate_up, gate_up.dtype, "gate_up")
    M, N2 = gate_up.shape
    I = N2 // 2
    dev = gate_up.device
    if out is None:
        out = NVFP4Tensor(torch.empty((M, I // 2), dtype=torch.uint8, device=dev),
                          torch.empty((M, I // 16), dtype=torch.uint8, device=dev),
                          torch.empty(1, dtype=torch.float32, device=dev))
    if workspace is None:
        workspace = torch.empty(lib().moe_swiglu_workspace_size(), dtype=torch.uint8, device=dev)
    _check(lib().moe_swiglu(gate_up.data_ptr(), _dtype_code(gate_up), M, I, _ptr(g), _ptr(out.g),
                            out.codes.data_ptr(), out.scales.data_ptr(), workspace.data_ptr(), workspace.numel(),
                            _stream(stream)))
    return out


# ------------------------------------------------------------------------- combine
def moe_unpermute_combine(y, perm_of_assignment, topk_w, T: int, k: int, out=None, out_dtype=None, stream=None):
    """out[t] = sum_j topk_w[t, j] * y[perm_of_assignment[t*k + j]] (bf16 by default)."""
    import torch
    _need(y, y.dtype, "y")
    H = y.shape[1]
    if out is None:
        out = torch.empty((T, H), dtype=out_dtype or torch.bfloat16, device=y.device)
    if tuple(out.shape) != (T, H):
        raise ValueError(f"out: expected [{T}, {H}], got {list(out.shape)}")
    _need(out, out.dtype, "out")
    if perm_of_assignment is not None:
        _need(perm_of_assignment, torch.int32, "perm_of_assignment")
        if perm_of_assignment.numel() < T * k:
            raise ValueError(f"perm_of_assignment: {perm_of_assignment.numel()} values, expected T*k = {T * k}")
    elif y.shape[0] < T * k:
        raise ValueError(f"y has {y.shape[0]} rows, fewer than T*k = {T * k} (and no perm_of_assignment)")
    if topk_w is not None:
        _need(topk_w, torch.float32, "topk_w")
        if topk_w.numel() < T * k:
            raise ValueError(f"topk_w: {topk_w.numel()} values, expected T*k = {T * k}")
    _check(lib().moe_unpermute_combine(y.data_ptr(), _dtype_code(y), _ptr(perm_of_assignment), _ptr(topk_w),
                                       T, k, H, out.data_ptr(), _dtype_code(out), _stream(stream)))
    return out


__all__ = ["lib", "moe_route_permute", "moe_route_quantize", "moe_route_quantize_noalloc", "nvfp4_quantize", "nvfp4_grouped_gemm", "moe_swiglu", "nvfp4_weight_repack",
           "moe_unpermute_combine", "moe_expert_ffn", "moe_expert_ffn_workspace", "mxfp4_quantize",
           "mxfp4_grouped_gemm", "mxfp4_weight_repack", "MXFP4Tensor", "fp8_quantize", "fp8_swiglu_quantize", "fp8_weight_repack",
           "fp8_grouped_gemm", "FP8Tensor", "Fp8GemmArgs", "NVFP4Tensor", "Routing", "GemmArgs", "NVFP4MoEError",
           "F32", "BF16", "EPI_F32", "EPI_BF16", "EPI_SWIGLU_NVFP4", "EPI_COMBINE_F32"]
