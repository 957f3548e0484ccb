"""The NVFP4 MoE layer forward, composed from the five C entry points.

route + permute -> quantise x -> gate_up grouped GEMM (rows gathered by token)
-> SwiGLU + NVFP4 re-quantisation -> down grouped GEMM -> weighted combine back
to token order, bfloat16 out.

Choices:
  ffn="one_launch" (default) gate_up + SwiGLU/requant + down through
                   moe_expert_ffn: one persistent launch from 48 rows per
                   expert (down tasks start as soon as their chunk's h rows
                   exist), the two grouped-GEMM launches below that;
  ffn="two_launch" the two grouped-GEMM calls, with the choices below;
  swiglu="fused"   (two_launch) the gate_up GEMM epilogue computes SwiGLU and
                   writes NVFP4 h directly;
  swiglu="separate" float32 gate_up output, then moe_swiglu;
  combine="gather" (default) the down GEMM writes bf16 rows, then
                   moe_unpermute_combine gathers each token's k rows
                   (deterministic);
  combine="atomic" the down GEMM epilogue scatter-adds weighted rows into a
                   float32 accumulator (float32 atomics), then converts it;
  combine="fused"  (one_launch) moe_expert_ffn combines too: in its
                   persistent launch the down task that writes a token's last
                   row of a column group combines that group (the same
                   arithmetic as moe_unpermute_combine, bit for bit); in the
                   two-launch regimes the combine kernel follows on the stream.

Buffers are allocated once per layer object (torch device memory); a forward
allocates nothing.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import (BF16, EPI_BF16, EPI_COMBINE_F32, EPI_F32, EPI_SWIGLU_NVFP4, F32, NVFP4Tensor, Routing, lib,
               moe_expert_ffn, moe_expert_ffn_workspace, moe_route_permute, moe_route_quantize, moe_swiglu,
               moe_unpermute_combine, nvfp4_grouped_gemm, nvfp4_quantize, nvfp4_weight_repack)


@dataclass
class ExpertWeights:
    """Per-expert NVFP4 weights: gate_up [E, 2I, H] and down [E, H, I]."""
    gu_codes: torch.Tensor
    gu_scales: torch.Tensor
    gu_g: torch.Tensor
    dn_codes: torch.Tensor
    dn_scales: torch.Tensor
    dn_g: torch.Tensor
    gu_packed: torch.Tensor | None = None    # tile layout from nvfp4_weight_repack
    dn_packed: torch.Tensor | None = None

    def pack(self) -> "ExpertWeights":
        """Repack both matrices into the GEMM's streaming tile layout (once, offline)."""
        self.gu_packed = nvfp4_weight_repack(self.gu_codes, self.gu_scales)
        self.dn_packed = nvfp4_weight_repack(self.dn_codes, self.dn_scales)
        return self

    @property
    def E(self):
        return self.gu_codes.shape[0]

    @property
    def I(self):
        return self.gu_codes.shape[1] // 2

    @property
    def H(self):
        return self.dn_codes.shape[1]

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in
                   (self.gu_codes, self.gu_scales, self.dn_codes, self.dn_scales))


def quantize_expert_weights(w_gu: torch.Tensor, w_dn: torch.Tensor) -> ExpertWeights:
    """Quantise float32/bf16 weights [E, 2I, H] and [E, H, I] on the GPU with
    one per-tensor scale per expert matrix (nvfp4_quantize per expert)."""
    E, I2, H = w_gu.shape
    dev = w_gu.device
    out = ExpertWeights(
        torch.empty((E, I2, H // 2), dtype=torch.uint8, device=dev),
        torch.empty((E, I2, H // 16), dtype=torch.uint8, device=dev),
        torch.empty(E, dtype=torch.float32, device=dev),
        torch.empty((E, H, I2 // 4), dtype=torch.uint8, device=dev),
        torch.empty((E, H, I2 // 32), dtype=torch.uint8, device=dev),
        torch.empty(E, dtype=torch.float32, device=dev))
    ws = torch.empty(lib().nvfp4_quantize_workspace_size(), dtype=torch.uint8, device=dev)
    for e in range(E):
        nvfp4_quantize(w_gu[e], out=NVFP4Tensor(out.gu_codes[e], out.gu_scales[e], out.gu_g[e:e + 1]), workspace=ws)
        nvfp4_quantize(w_dn[e], out=NVFP4Tensor(out.dn_codes[e], out.dn_scales[e], out.dn_g[e:e + 1]), workspace=ws)
    return out


class MoELayer:
    """Preallocated NVFP4 MoE layer for T tokens."""

    def __init__(self, T: int, H: int, I: int, E: int, k: int, device, swiglu: str = "fused",
                 combine: str = "gather", ffn: str = "one_launch"):
        assert swiglu in ("fused", "separate") and combine in ("gather", "atomic", "fused")
        assert ffn in ("one_launch", "two_launch")
        if ffn == "one_launch" and (swiglu, combine) not in (("fused", "gather"), ("fused", "fused")):
            ffn = "two_launch"     # the one-launch FFN has the fused SwiGLU and bf16 rows
        if ffn == "two_launch" and combine == "fused":
            combine = "gather"
        self.T, self.H, self.I, self.E, self.k = T, H, I, E, k
        self.swiglu, self.combine, self.ffn = swiglu, combine, ffn
        dev = torch.device(device)
        i32 = dict(dtype=torch.int32, device=dev)
        f32 = dict(dtype=torch.float32, device=dev)
        u8 = dict(dtype=torch.uint8, device=dev)
        M = T * k
        self.routing = Routing(torch.empty((T, k), **i32), torch.empty((T, k), **f32), torch.empty(E, **i32),
                               torch.empty(E + 1, **i32), torch.empty(M, **i32), torch.empty(M, **i32),
                               torch.empty(M, **f32))
        self.route_ws = torch.empty(max(16, lib().moe_route_quantize_workspace_size(T, E, k)), **u8)
        self.small_ws = torch.empty(lib().nvfp4_quantize_workspace_size(), **u8)
        self.xq = NVFP4Tensor(torch.empty((T, H // 2), **u8), torch.empty((T, H // 16), **u8),
                              torch.empty(1, **f32))
        self.hq = NVFP4Tensor(torch.empty((M, I // 2), **u8), torch.empty((M, I // 16), **u8), None)
        self.out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        if swiglu == "separate":
            self.y1 = torch.empty((M, 2 * I), **f32)
        if combine == "atomic":
            self.acc = torch.empty((T, H), **f32)
        else:
            self.y2 = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
        if self.ffn == "one_launch":
            self.ffn_ws = moe_expert_ffn_workspace(E, M, H, I, dev)

    def forward(self, logits: torch.Tensor, x: torch.Tensor, w: ExpertWeights, g_h: torch.Tensor,
                stream=None, marks=None) -> torch.Tensor:
        """One layer step.  ``marks``: optional list of 6 torch.cuda.Event (or None
        entries) recorded on the launch stream before routing and after each
        stage: route+permute and the quantisation of x (one call whose kernels
        share launches; marks 1 and 2 both follow it), gate_up, down,
        to-bf16/combine.  With the one-launch FFN, marks 3 and 4 both follow
        the gate_up + down call."""
        T, k, M = self.T, self.k, self.T * self.k
        hq = NVFP4Tensor(self.hq.codes, self.hq.scales, g_h)

        def mark(i):
            if marks is not None and marks[i] is not None:
                marks[i].record(stream)

        mark(0)
        r, _ = moe_route_quantize(logits, k, x, out=self.routing, xq=self.xq, workspace=self.route_ws, stream=stream)
        mark(1)
        mark(2)
        if self.ffn == "one_launch" and w.gu_packed is not None and w.dn_packed is not None:
            if self.combine == "fused":
                moe_expert_ffn(self.xq, r.perm_src_token, r.offsets, w.gu_packed, w.gu_g, w.dn_packed, w.dn_g, g_h,
                               H=self.H, I=self.I, m_total=M, h=hq, y=self.y2, workspace=self.ffn_ws,
                               perm_of_assignment=r.perm_of_assignment, topk_w=r.topk_w, k=k, out=self.out,
                               stream=stream)
                mark(3)
                mark(4)
                mark(5)
                return self.out
            moe_expert_ffn(self.xq, r.perm_src_token, r.offsets, w.gu_packed, w.gu_g, w.dn_packed, w.dn_g, g_h,
                           H=self.H, I=self.I, m_total=M, h=hq, y=self.y2, workspace=self.ffn_ws, stream=stream)
            mark(3)
            mark(4)
            moe_unpermute_combine(self.y2, r.perm_of_assignment, r.topk_w, T, k, out=self.out, stream=stream)
            mark(5)
            return self.out
        if self.swiglu == "fused":
            nvfp4_grouped_gemm(self.xq, w.gu_codes, w.gu_scales, w.gu_g, r.offsets, m_total=M,
                               a_rows=r.perm_src_token, epilogue=EPI_SWIGLU_NVFP4, out_codes=self.hq.codes,
                               out_scales=self.hq.scales, out_g=g_h, b_packed=w.gu_packed, stream=stream)
        else:
            nvfp4_grouped_gemm(self.xq, w.gu_codes, w.gu_scales, w.gu_g, r.offsets, m_total=M,
                               a_rows=r.perm_src_token, epilogue=EPI_F32, out=self.y1, b_packed=w.gu_packed,
                               stream=stream)
            moe_swiglu(self.y1, g=g_h, out=self.hq, workspace=self.small_ws, stream=stream)
        mark(3)
        if self.combine == "atomic":
            self.acc.zero_()
            nvfp4_grouped_gemm(hq, w.dn_codes, w.dn_scales, w.dn_g, r.offsets, m_total=M,
                               epilogue=EPI_COMBINE_F32, out=self.acc, out_rows=T, row_token=r.perm_src_token,
                               row_weight=r.perm_weight, b_packed=w.dn_packed, stream=stream)
            mark(4)
            moe_unpermute_combine(self.acc, None, None, T, 1, out=self.out, stream=stream)
        else:
            nvfp4_grouped_gemm(hq, w.dn_codes, w.dn_scales, w.dn_g, r.offsets, m_total=M,
                               epilogue=EPI_BF16, out=self.y2, b_packed=w.dn_packed, stream=stream)
            mark(4)
            moe_unpermute_combine(self.y2, r.perm_of_assignment, r.topk_w, T, k, out=self.out, stream=stream)
        mark(5)
        return self.out


def capture_step(layer: "MoELayer", logits: torch.Tensor, x: torch.Tensor, w: ExpertWeights, g_h: torch.Tensor):
    """Record one layer step (``layer.forward`` on these exact tensors) into a
    HIP graph and return it (a ``torch.cuda.CUDAGraph``; ``replay()`` re-runs
    the step's kernels on the same buffers with one launch of the graph).
    Nothing in the step synchronises with the host or allocates: the routing
    counts stay on the device and every buffer is the layer's own, so the
    recorded kernels are exactly the eager step's.  The inputs' contents may
    change between replays; their addresses may not."""
    side = torch.cuda.Stream(device=logits.device)
    side.wait_stream(torch.cuda.current_stream(logits.device))
    with torch.cuda.stream(side):          # the capture runs on a side stream, as torch requires
        layer.forward(logits, x, w, g_h)   # one eager step on that stream first
    torch.cuda.current_stream(logits.device).wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer.forward(logits, x, w, g_h)
    return graph


# ------------------------------------------------------------------ MXFP4 variant
@dataclass
class MXExpertWeights:
    """Per-expert MXFP4 weights (E8M0 scale per 32 along K, no per-tensor scale):
    gate_up codes [E, 2I, H/2], scales [E, 2I, H/32]; down [E, H, I/2], [E, H, I/32]."""
    gu: "object"
    dn: "object"
    gu_packed: "object" = None     # streaming tiles from mxfp4_weight_repack
    dn_packed: "object" = None

    def pack(self) -> "MXExpertWeights":
        from . import mxfp4_weight_repack
        self.gu_packed = mxfp4_weight_repack(self.gu)
        self.dn_packed = mxfp4_weight_repack(self.dn)
        return self

    @property
    def E(self):
        return self.gu.codes.shape[0]

    def nbytes(self) -> int:
        return sum(t.numel() for t in (self.gu.codes, self.gu.scales, self.dn.codes, self.dn.scales))


def quantize_expert_weights_mx(w_gu: torch.Tensor, w_dn: torch.Tensor) -> MXExpertWeights:
    """Quantise float32/bf16 weights [E, 2I, H] and [E, H, I] to MXFP4 on the GPU."""
    from . import mxfp4_quantize
    return MXExpertWeights(mxfp4_quantize(w_gu.contiguous()), mxfp4_quantize(w_dn.contiguous())).pack()


class MXMoELayer:
    """Preallocated MXFP4 MoE layer for T tokens: route + permute, MXFP4
    quantisation of x, gate_up grouped GEMM with the fused SwiGLU + MXFP4
    requantisation, down grouped GEMM (bf16 rows), weighted gather combine."""

    def __init__(self, T: int, H: int, I: int, E: int, k: int, device):
        from . import MXFP4Tensor
        self.T, self.H, self.I, self.E, self.k = T, H, I, E, k
        dev = torch.device(device)
        i32 = dict(dtype=torch.int32, device=dev)
        f32 = dict(dtype=torch.float32, device=dev)
        u8 = dict(dtype=torch.uint8, device=dev)
        M = T * k
        self.routing = Routing(torch.empty((T, k), **i32), torch.empty((T, k), **f32), torch.empty(E, **i32),
                               torch.empty(E + 1, **i32), torch.empty(M, **i32), torch.empty(M, **i32),
                               torch.empty(M, **f32))
        self.route_ws = torch.empty(max(16, lib().moe_route_permute_workspace_size(T, E, k)), **u8)
        self.xq = MXFP4Tensor(torch.empty((T, H // 2), **u8), torch.empty((T, H // 32), **u8))
        self.hq = MXFP4Tensor(torch.empty((M, I // 2), **u8), torch.empty((M, I // 32), **u8))
        self.y2 = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
        self.out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        self.ones = torch.ones(max(E, 1), **f32)

    def forward(self, logits: torch.Tensor, x: torch.Tensor, w: MXExpertWeights, stream=None,
                marks=None) -> torch.Tensor:
        """One layer step; ``marks``: optional 6 events (as MoELayer.forward:
        route, quantise x, gate_up, down, combine)."""
        from . import mxfp4_grouped_gemm, mxfp4_quantize
        T, k, M = self.T, self.k, self.T * self.k

        def mark(i):
            if marks is not None and marks[i] is not None:
                marks[i].record(stream)

        mark(0)
        r = moe_route_permute(logits, k, out=self.routing, workspace=self.route_ws, stream=stream)
        mark(1)
        mxfp4_quantize(x, out=self.xq, stream=stream)
        mark(2)
        mxfp4_grouped_gemm(self.xq, w.gu, r.offsets, m_total=M, a_rows=r.perm_src_token, epilogue=EPI_SWIGLU_NVFP4,
                           out_codes=self.hq.codes, out_scales=self.hq.scales, a_g=self.ones[:1], b_g=self.ones,
                           b_packed=w.gu_packed, stream=stream)
        mark(3)
        mxfp4_grouped_gemm(self.hq, w.dn, r.offsets, m_total=M, epilogue=EPI_BF16, out=self.y2, a_g=self.ones[:1],
                           b_g=self.ones, b_packed=w.dn_packed, stream=stream)
        mark(4)
        moe_unpermute_combine(self.y2, r.perm_of_assignment, r.topk_w, T, k, out=self.out, stream=stream)
        mark(5)
        return self.out


# ------------------------------------------------------------------ FP8 block-scaled variant
@dataclass
class FP8ExpertWeights:
    """Per-expert FP8 weights with one float32 scale per 128 x 128 block:
    gate_up codes [E, 2I, H] and scales [E, 2I/128, H/128], down [E, H, I] and
    [E, H/128, I/128], with each matrix's packed tiles (fp8_weight_repack)."""
    gu: "object"
    dn: "object"
    gu_packed: "object" = None
    dn_packed: "object" = None

    def pack(self) -> "FP8ExpertWeights":
        from . import fp8_weight_repack
        self.gu_packed = fp8_weight_repack(self.gu.codes)
        self.dn_packed = fp8_weight_repack(self.dn.codes)
        return self


def quantize_expert_weights_fp8(w_gu: torch.Tensor, w_dn: torch.Tensor) -> FP8ExpertWeights:
    """Quantise float32/bf16 weights [E, 2I, H] and [E, H, I] to FP8 (128 x 128
    blocks) on the GPU and repack them."""
    from . import fp8_quantize
    return FP8ExpertWeights(fp8_quantize(w_gu.contiguous(), 128), fp8_quantize(w_dn.contiguous(), 128)).pack()


class FP8MoELayer:
    """Preallocated FP8 block-scaled MoE layer for T tokens, reusing the routing,
    permutation and combine of the NVFP4 layer: route + permute, FP8
    quantisation of x (1 x 128 blocks), gate_up grouped GEMM (A gathered
    through the permutation) with SwiGLU + FP8 requantisation of h, down
    grouped GEMM (bf16 rows), weighted gather combine.

    ``swiglu``: "fused" runs the SwiGLU + requant as gate_up's epilogue below
    256 rows per expert (at and above that gate_up runs the 256 x 256 tile,
    which writes float32 rows for the separate kernel); "separate" always
    writes the float32 rows.  Both give the same h, bit for bit."""

    def __init__(self, T: int, H: int, I: int, E: int, k: int, device, swiglu: str = "fused"):
        from . import FP8_BLOCK, FP8Tensor
        if swiglu not in ("fused", "separate"):
            raise ValueError("swiglu: 'fused' or 'separate'")
        self.T, self.H, self.I, self.E, self.k = T, H, I, E, k
        self.fused = swiglu == "fused" and (T * k) // E < 256 and I % FP8_BLOCK == 0
        dev = torch.device(device)
        i32 = dict(dtype=torch.int32, device=dev)
        f32 = dict(dtype=torch.float32, device=dev)
        u8 = dict(dtype=torch.uint8, device=dev)
        M = T * k
        self.routing = Routing(torch.empty((T, k), **i32), torch.empty((T, k), **f32), torch.empty(E, **i32),
                               torch.empty(E + 1, **i32), torch.empty(M, **i32), torch.empty(M, **i32),
                               torch.empty(M, **f32))
        self.route_ws = torch.empty(max(16, lib().moe_route_permute_workspace_size(T, E, k)), **u8)
        self.xq = FP8Tensor(torch.empty((T, H), **u8), torch.empty((T, H // FP8_BLOCK), **f32), 1)
        self.y1 = None if self.fused else torch.empty((M, 2 * I), **f32)
        self.hq = FP8Tensor(torch.empty((M, I), **u8), torch.empty((M, I // FP8_BLOCK), **f32), 1)
        self.y2 = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
        self.out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)

    def forward(self, logits: torch.Tensor, x: torch.Tensor, w: FP8ExpertWeights, stream=None,
                marks=None) -> torch.Tensor:
        """One layer step; ``marks``: optional 7 events recorded before routing
        and after each stage (route, quantise x, gate_up, SwiGLU + requant,
        down, combine; with the fused SwiGLU marks 3 and 4 both follow
        gate_up)."""
        from . import EPI_SWIGLU_NVFP4, fp8_grouped_gemm, fp8_quantize, fp8_swiglu_quantize
        T, k, M = self.T, self.k, self.T * self.k
        hint = M // self.E

        def mark(i):
            if marks is not None and marks[i] is not None:
                marks[i].record(stream)

        mark(0)
        r = moe_route_permute(logits, k, out=self.routing, workspace=self.route_ws, stream=stream)
        mark(1)
        fp8_quantize(x, 1, out=self.xq, stream=stream)
        mark(2)
        if self.fused:
            fp8_grouped_gemm(self.xq, w.gu_packed, w.gu.scales, r.offsets, N=2 * self.I, m_total=M,
                             a_rows=r.perm_src_token, epilogue=EPI_SWIGLU_NVFP4, out=self.hq,
                             max_rows_per_expert_hint=hint, stream=stream)
            mark(3)
            mark(4)
        else:
            fp8_grouped_gemm(self.xq, w.gu_packed, w.gu.scales, r.offsets, N=2 * self.I, m_total=M,
                             a_rows=r.perm_src_token, epilogue=EPI_F32, out=self.y1, max_rows_per_expert_hint=hint,
                             stream=stream)
            mark(3)
            fp8_swiglu_quantize(self.y1, out=self.hq, stream=stream)
            mark(4)
        fp8_grouped_gemm(self.hq, w.dn_packed, w.dn.scales, r.offsets, N=self.H, m_total=M, epilogue=EPI_BF16,
                         out=self.y2, max_rows_per_expert_hint=hint, stream=stream)
        mark(5)
        moe_unpermute_combine(self.y2, r.perm_of_assignment, r.topk_w, T, k, out=self.out, stream=stream)
        mark(6)
        return self.out
