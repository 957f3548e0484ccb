"""The NVFP4 MoE layer, step by step, on the CPU (oracle; test infrastructure).

Steps, in the order the layer runs them:

route     top-k experts per token from the router logits, softmax weights
          renormalised over the chosen k.  The pages describe a router choosing
          a few of 256 experts per token ("Discovering SM120-Specific CUTLASS MoE
          Kernels", section "Input Knowledge Required").
permute   expert-first layout: a per-expert histogram, its exclusive prefix sum
          (expert offsets) and a stable scatter of assignments into expert
          order ("From Empirical Limits to Research-Driven Optimization",
          section "Sections 5-6: Algorithmic Techniques": expert-first layout,
          token reordering with fused reduction).
gemm      per expert, a block-scaled NVFP4 GEMM of its contiguous rows, float32
          result (the MMA of section "Section 1: CUTLASS Kernels - The
          Foundation" of the same page: e2m1 x e2m1, ue4m3 scale per 16 K,
          f32 accumulate), then the per-tensor scales.
swiglu    h = silu(gate) * up on the gate_up output, re-quantised to NVFP4.
combine   out[t] = sum_j w[t, j] * y[row of assignment (t, j)]: the weighted
          reduction back to token order (the "finalize" epilogue of "The
          Critical Search: Uncovering SM120 CUTLASS Collective Implementations",
          section "Context: The Optimization Journey").

Readings where the pages say nothing (the pages hold no equations):
* ties between equal logits go to the lower expert id; the k ids of a token are
  listed by descending logit;
* rows inside one expert keep ascending assignment index t*k + j (stable);
* gate_up rows [0, I) are the gate, [I, 2I) the up projection;
* the intermediate h is re-quantised with a caller-supplied per-tensor scale;
* routing weights are applied in the combine, after the down GEMM.
"""
from __future__ import annotations

import numpy as np

from .formats import round_to_bf16
from .quant import dequantize_unscaled, quantize


# --------------------------------------------------------------------------- route
def route(logits: np.ndarray, k: int):
    """logits float32 [T, E] -> (topk_ids int32 [T, k], topk_w float32 [T, k]).

    ids: the k largest logits of each token, by descending logit, ties to the
    lower expert id (a stable sort of -logit).  Weights: softmax over all E
    experts renormalised over the chosen k, which is
    exp(l_j - l_max) / sum_{i in top-k} exp(l_i - l_max); float64, rounded to
    float32 once."""
    l = np.asarray(logits, dtype=np.float64)
    T, E = l.shape
    assert 1 <= k <= E
    ids = np.argsort(-l, axis=1, kind="stable")[:, :k]
    sel = np.take_along_axis(l, ids, axis=1)
    ex = np.exp(sel - sel[:, :1])
    w = ex / ex.sum(axis=1, keepdims=True)
    return ids.astype(np.int32), w.astype(np.float32)


# ------------------------------------------------------------------------- permute
def permute(topk_ids: np.ndarray, topk_w: np.ndarray, E: int):
    """Counting sort of the T*k assignments by expert, stable in the flat
    assignment index f = t*k + j.

    Returns counts int32[E], offsets int32[E+1] (exclusive prefix sum of counts),
    perm_src_token int32[T*k] (token of permuted row p), perm_of_assignment
    int32[T*k] (permuted row of assignment f), perm_weight float32[T*k] (routing
    weight of permuted row p)."""
    T, k = topk_ids.shape
    flat = topk_ids.reshape(-1).astype(np.int64)
    order = np.argsort(flat, kind="stable")
    counts = np.bincount(flat, minlength=E).astype(np.int64)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    perm_src_token = order // k
    perm_of_assignment = np.empty(T * k, dtype=np.int64)
    perm_of_assignment[order] = np.arange(T * k)
    perm_weight = np.asarray(topk_w, dtype=np.float32).reshape(-1)[order]
    return (counts.astype(np.int32), offsets.astype(np.int32),
            perm_src_token.astype(np.int32), perm_of_assignment.astype(np.int32),
            perm_weight.astype(np.float32))


# ---------------------------------------------------------------------------- gemm
def grouped_gemm(a_codes, a_scales, a_g, b_codes, b_scales, b_g, offsets,
                 a_rows=None, want_absdot=True):
    """Grouped NVFP4 GEMM.

    For expert e and permuted row p in [offsets[e], offsets[e+1]) with A row
    r = a_rows[p] (or p):
        y[p, n] = g_a * g_b[e] * sum_kb s_a[r, kb] * s_b[e, n, kb]
                                 * sum_{i<16} q_a[r, 16kb+i] * q_b[e, n, 16kb+i]
    The inner products of E2M1(q)*E4M3(s) values are exact in float64; the sum
    runs in float64 (numpy matmul as the summation primitive) and is rounded to
    float32 once after the per-tensor scales.  Also returns
    absdot[p, n] = sum_k |a^_k * b^_k| with the per-tensor scales, the scale of
    the error bound.
    a_*: codes [rows_a, K/2], scales [rows_a, K/16], g float.  b_*: codes
    [E, N, K/2], scales [E, N, K/16], g [E]."""
    E, N, K2 = b_codes.shape
    offsets = np.asarray(offsets, dtype=np.int64)
    M = int(offsets[-1])
    y = np.zeros((M, N), dtype=np.float32)
    absdot = np.zeros((M, N), dtype=np.float64) if want_absdot else None
    ga = np.float64(np.float32(a_g))
    for e in range(E):
        p0, p1 = int(offsets[e]), int(offsets[e + 1])
        if p1 == p0:
            continue
        rows = np.arange(p0, p1) if a_rows is None else np.asarray(a_rows)[p0:p1]
        a_hat = dequantize_unscaled(a_codes[rows], a_scales[rows])     # [Me, K]
        b_hat = dequantize_unscaled(b_codes[e], b_scales[e])           # [N, K]
        gab = ga * np.float64(np.float32(b_g[e]))
        s = a_hat @ b_hat.T
        y[p0:p1] = (s * gab).astype(np.float32)
        if want_absdot:
            absdot[p0:p1] = (np.abs(a_hat) @ np.abs(b_hat).T) * gab
    return y, absdot


def grouped_gemm_blockwise(a_codes, a_scales, a_g, b_codes, b_scales, b_g, offsets,
                           a_rows=None):
    """The same GEMM written block by block (per-16-block partial dot products
    of E2M1 values, scaled by the two E4M3 block scales, summed over blocks).
    Slow; used on small shapes to check ``grouped_gemm`` term by term."""
    from .formats import e2m1_decode, e4m3_decode
    from .quant import unpack_codes
    E, N, K2 = b_codes.shape
    K = 2 * K2
    KB = K // 16
    offsets = np.asarray(offsets, dtype=np.int64)
    M = int(offsets[-1])
    y = np.zeros((M, N), dtype=np.float64)
    for e in range(E):
        for p in range(int(offsets[e]), int(offsets[e + 1])):
            r = p if a_rows is None else int(a_rows[p])
            qa = e2m1_decode(unpack_codes(a_codes[r])).reshape(KB, 16)
            sa = e4m3_decode(a_scales[r])
            for n in range(N):
                qb = e2m1_decode(unpack_codes(b_codes[e, n])).reshape(KB, 16)
                sb = e4m3_decode(b_scales[e, n])
                acc = 0.0
                for kb in range(KB):
                    acc += sa[kb] * sb[kb] * float(np.dot(qa[kb], qb[kb]))
                y[p, n] = acc * float(np.float32(a_g)) * float(np.float32(b_g[e]))
    return y


# -------------------------------------------------------------------------- swiglu
def silu(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def swiglu(y1: np.ndarray) -> np.ndarray:
    """h = silu(gate) * up, gate = y1[:, :I], up = y1[:, I:], float64."""
    y1 = np.asarray(y1, dtype=np.float64)
    I = y1.shape[1] // 2
    return silu(y1[:, :I]) * y1[:, I:]


def swiglu_quantize(y1: np.ndarray, g_h: float | None):
    """SwiGLU, rounded to float32, then NVFP4 with the per-tensor scale g_h
    (None: computed from amax).  Returns (codes, scales, g_h, h64)."""
    h64 = swiglu(y1)
    codes, scales, g = quantize(h64.astype(np.float32), g=g_h)
    return codes, scales, g, h64


# ------------------------------------------------------------------------- combine
def combine(y2: np.ndarray, perm_of_assignment: np.ndarray, topk_w: np.ndarray):
    """out[t, :] = sum_j w[t, j] * y2[perm_of_assignment[t*k + j], :] in float64;
    returns (out64, out_bf16_as_float32)."""
    T, k = topk_w.shape
    y2 = np.asarray(y2, dtype=np.float64)
    idx = np.asarray(perm_of_assignment, dtype=np.int64).reshape(T, k)
    w = np.asarray(topk_w, dtype=np.float64)
    out = np.einsum("tj,tjh->th", w, y2[idx])
    return out, round_to_bf16(out)


# --------------------------------------------------------------------- whole layer
def quantize_experts(weights):
    """Quantise a list of per-expert float32 matrices, one per-tensor scale each."""
    cs, ss, gs = [], [], []
    for w in weights:
        c, s, g = quantize(w)
        cs.append(c), ss.append(s), gs.append(g)
    return np.stack(cs), np.stack(ss), np.asarray(gs, dtype=np.float32)


def moe_layer(logits, x, wgu_q, wdn_q, k, g_h=None):
    """Full layer: route, permute, quantise x, gate_up GEMM on gathered rows,
    SwiGLU + requantise, down GEMM, weighted combine.  wgu_q / wdn_q are
    (codes, scales, g[E]) of the quantised expert weights."""
    T, E = logits.shape
    ids, w = route(logits, k)
    counts, offsets, src_tok, perm_of_asg, perm_w = permute(ids, w, E)
    xc, xs, xg = quantize(x)
    y1, absdot1 = grouped_gemm(xc, xs, xg, *wgu_q, offsets, a_rows=src_tok)
    hc, hs, hg, h64 = swiglu_quantize(y1, g_h)
    y2, absdot2 = grouped_gemm(hc, hs, hg, *wdn_q, offsets)
    out64, out_bf16 = combine(y2, perm_of_asg, w)
    return dict(topk_ids=ids, topk_w=w, counts=counts, offsets=offsets,
                perm_src_token=src_tok, perm_of_assignment=perm_of_asg,
                perm_weight=perm_w, x_codes=xc, x_scales=xs, x_g=xg,
                y1=y1, absdot1=absdot1, h64=h64, h_codes=hc, h_scales=hs, h_g=hg,
                y2=y2, absdot2=absdot2, out64=out64, out=out_bf16)
