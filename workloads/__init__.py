"""Seeded synthetic inputs for the NVFP4 MoE layer.

This module only draws random numbers and fixes shapes.  It holds none of the
method's arithmetic (no quantisation, routing, GEMM or combine): both the CPU
oracle and the GPU path receive exactly the arrays produced here.

Every stream is ``numpy.random.default_rng(SeedSequence([2026, cfg, stream, ...]))``
with streams 0 = router logits, 1 = expert popularity ranks, 2 = activations,
3 = gate_up weights (one sub-stream per expert), 4 = down weights (one per
expert), 5/6 = dense A/B, 7 = NVFP4 operand bytes drawn directly.  Activations are drawn in float32 and rounded to
bfloat16 (round to nearest even, by torch), because the layer's input is a
bfloat16 tensor; the float32 copy returned here holds the same values.

The workloads stand in for one GPU's share of a 256-expert MoE layer served
with 8-way tensor parallelism (the per-GPU expert width of 256 comes from
"Discovering SM120-Specific CUTLASS MoE Kernels", section "Assumptions and
Potential Missteps": E=256, N=256 at TP8); hidden size 6144 and top-8 routing
are the stated workload sizes.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

SEED = 2026


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int          # tokens
    H: int          # hidden size (K of gate_up, N of down)
    I: int          # per-expert intermediate size (gate_up has 2I rows)
    E: int          # experts
    k: int          # experts per token
    routing: str = "uniform"          # "uniform" or "zipf"
    zipf_s: float = 1.1
    zipf_alpha: float = 0.55
    zipf_r0: int = 32
    logit_std: float = 1.0
    weight_std: float = 0.02
    dense: bool = False               # single dense GEMM (E=1, no routing)
    index: int = 0
    extra: dict = field(default_factory=dict)


CONFIGS = {
    0: MoEConfig("tiny", T=8, H=256, I=128, E=4, k=2, index=0),
    1: MoEConfig("decode_T256", T=256, H=6144, I=256, E=256, k=8, index=1),
    2: MoEConfig("decode_T2048_zipf", T=2048, H=6144, I=256, E=256, k=8,
                 routing="zipf", index=2),
    3: MoEConfig("prefill_T16384", T=16384, H=6144, I=256, E=256, k=8, index=3),
    # dense GEMM: M=T rows of A, N=H rows of B, K=I reduction
    4: MoEConfig("dense_8192", T=8192, H=8192, I=8192, E=1, k=1, dense=True, index=4),
}


def rng(cfg_index: int, stream: int, *sub: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([SEED, cfg_index, stream, *sub]))


def to_bf16_values(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), returned as float32."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def expert_bias(cfg: MoEConfig) -> np.ndarray:
    """Per-expert additive logit bias giving a Zipf-like expert popularity.

    b_e = -alpha * s * ln(max(rank_e, r0)) where rank_e is a seeded permutation
    of 1..E.  Uniform routing gets zeros.
    """
    if cfg.routing == "uniform":
        return np.zeros(cfg.E, dtype=np.float32)
    ranks = rng(cfg.index, 1).permutation(cfg.E) + 1
    b = -cfg.zipf_alpha * cfg.zipf_s * np.log(np.maximum(ranks, cfg.zipf_r0).astype(np.float64))
    return b.astype(np.float32)


def logits(cfg: MoEConfig, T: int | None = None) -> np.ndarray:
    T = cfg.T if T is None else T
    g = rng(cfg.index, 0)
    l = g.standard_normal((T, cfg.E), dtype=np.float32) * np.float32(cfg.logit_std)
    return (l + expert_bias(cfg)[None, :]).astype(np.float32)


def activations(cfg: MoEConfig, T: int | None = None) -> np.ndarray:
    """x ~ N(0,1), rounded to bfloat16, as float32 [T, H]."""
    T = cfg.T if T is None else T
    x = rng(cfg.index, 2).standard_normal((T, cfg.H), dtype=np.float32)
    return to_bf16_values(x)


def gate_up_weight(cfg: MoEConfig, e: int) -> np.ndarray:
    """float32 [2I, H] ~ N(0, weight_std): rows [0, I) gate, [I, 2I) up."""
    w = rng(cfg.index, 3, e).standard_normal((2 * cfg.I, cfg.H), dtype=np.float32)
    return w * np.float32(cfg.weight_std)


def down_weight(cfg: MoEConfig, e: int) -> np.ndarray:
    """float32 [H, I] ~ N(0, weight_std)."""
    w = rng(cfg.index, 4, e).standard_normal((cfg.H, cfg.I), dtype=np.float32)
    return w * np.float32(cfg.weight_std)


def dense_operands(cfg: MoEConfig, M: int | None = None, N: int | None = None,
                   K: int | None = None) -> tuple[np.ndarray, np.ndarray]:
    """A [M, K] and B [N, K] ~ N(0,1) float32 for the single dense GEMM."""
    M = cfg.T if M is None else M
    N = cfg.H if N is None else N
    K = cfg.I if K is None else K
    a = rng(cfg.index, 5).standard_normal((M, K), dtype=np.float32)
    b = rng(cfg.index, 6).standard_normal((N, K), dtype=np.float32)
    return a, b


def small_variant(cfg: MoEConfig, **over) -> MoEConfig:
    """Same recipe, other sizes (for parity cases the oracle finishes quickly)."""
    d = dict(cfg.__dict__)
    d.update(over)
    return MoEConfig(**d)


def torch_expert_weights(cfg: MoEConfig, device, copy: int = 0):
    """float32 gate_up [E, 2I, H] and down [E, H, I] ~ N(0, weight_std) drawn on
    ``device`` with torch's seeded generator (for the full-size workloads, where
    drawing 1.2e9 normals on the host would dominate).  Deterministic for a given
    (cfg, copy, device type)."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(SEED * 1000 + cfg.index * 10 + copy)
    w_gu = torch.randn((cfg.E, 2 * cfg.I, cfg.H), generator=gen, device=device, dtype=torch.float32)
    w_gu.mul_(cfg.weight_std)
    w_dn = torch.randn((cfg.E, cfg.H, cfg.I), generator=gen, device=device, dtype=torch.float32)
    w_dn.mul_(cfg.weight_std)
    return w_gu, w_dn


def torch_dense_operands(cfg: MoEConfig, device):
    """A [M, K] and B [N, K] ~ N(0, 1) float32 on ``device`` (seeded torch generator)."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(SEED * 1000 + cfg.index * 10 + 7)
    a = torch.randn((cfg.T, cfg.I), generator=gen, device=device, dtype=torch.float32)
    b = torch.randn((cfg.H, cfg.I), generator=gen, device=device, dtype=torch.float32)
    return a, b


def nvfp4_codes(cfg: MoEConfig, stream: int, shape_rows: tuple, K: int, scale_lo: int = 0x60,
                scale_hi: int = 0x7F, const_scale: int | None = None, block: int = 16):
    """Random FP4 operand bytes: codes uint8 [*shape_rows, K/2] uniform over all
    256 byte values (two 4-bit codes each) and block-scale bytes uint8
    [*shape_rows, K/block] uniform in [scale_lo, scale_hi) (for NVFP4, E4M3
    codes with 16-value blocks: the default range 0x60..0x7E is where block
    scales of quantised Gaussian weights land, about 64..448; for MXFP4, E8M0
    codes with block=32), or all equal to ``const_scale``.  Raw input bytes,
    drawn from stream ``stream`` (7 = GEMM operands given directly as codes);
    no arithmetic of the method is involved."""
    g = rng(cfg.index, 7, stream)
    codes = g.integers(0, 256, tuple(shape_rows) + (K // 2,), dtype=np.uint8)
    if const_scale is None:
        scales = g.integers(scale_lo, scale_hi, tuple(shape_rows) + (K // block,), dtype=np.uint8)
    else:
        scales = np.full(tuple(shape_rows) + (K // block,), const_scale, np.uint8)
    return codes, scales


def fp8_codes(cfg: MoEConfig, stream: int, shape: tuple, exp_lo: int = 0, exp_hi: int = 16):
    """Random E4M3 bytes uint8 [*shape]: random sign, exponent field uniform in
    [exp_lo, exp_hi), mantissa uniform, the NaN pattern (exponent 15, mantissa
    7) replaced by 448's.  Raw input bytes from stream ``stream`` of generator
    family 8; no arithmetic of the method is involved."""
    g = rng(cfg.index, 8, stream)
    if exp_lo == 0 and exp_hi == 16:
        codes = g.integers(0, 256, shape, dtype=np.uint8)       # every byte value: all signs and fields
    else:
        e = g.integers(exp_lo, exp_hi, shape, dtype=np.uint8)
        codes = (e << 3) | g.integers(0, 8, shape, dtype=np.uint8) | (g.integers(0, 2, shape, dtype=np.uint8) << 7)
    codes[(codes & 0x7F) == 0x7F] ^= 1
    return codes.astype(np.uint8, copy=False)


def fp8_scales(cfg: MoEConfig, stream: int, shape: tuple, lo: float = 2.0 ** -12, hi: float = 2.0 ** -6):
    """Random positive float32 block scales [*shape], log-uniform in [lo, hi)
    (stream ``stream`` of generator family 9)."""
    g = rng(cfg.index, 9, stream)
    return np.exp2(g.uniform(np.log2(lo), np.log2(hi), shape)).astype(np.float32)


# Static calibration of the intermediate's per-tensor scale: an expected
# absolute maximum of h = silu(gate) * up for each workload (gate and up are
# roughly N(0, (sqrt(H) * 0.02)^2) for x ~ N(0,1)).  Both sides receive the same
# per-tensor scale derived from it.
H_CALIBRATION_AMAX = {0: 0.5, 1: 24.0, 2: 32.0, 3: 40.0}
