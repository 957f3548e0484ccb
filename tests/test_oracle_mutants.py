"""Planted mistakes in the oracle (on the CPU) must be caught by its pins.

Each case swaps one oracle function for a plausible wrong variant (a dropped
term, a wrong sign or index, a transposed operand, a different rounding) and
runs a pin that must then fail."""
import numpy as np
import pytest

import oracle.formats as F
import oracle.moe as M
import oracle.quant as Q
import tests.test_oracle_formats as TF
import tests.test_oracle_gemm as TG
import tests.test_oracle_moe as TM
import tests.test_oracle_quant as TQ


def _fails(fn, *a, **kw):
    try:
        fn(*a, **kw)
    except AssertionError:
        return True
    return False


def test_mutant_e2m1_ties_away(monkeypatch):
    def bad(v):
        v = np.minimum(np.asarray(v, np.float64), 6.0)
        d = np.abs(v[..., None] - F.E2M1_MAGNITUDES)
        return (7 - np.argmin(d[..., ::-1], axis=-1)).astype(np.uint8)   # ties -> larger
    monkeypatch.setattr(Q, "e2m1_encode_magnitude", bad)
    assert _fails(TQ.test_worked_example_by_hand)


def test_mutant_scale_not_divided_by_six(monkeypatch):
    orig = Q.block_scale_codes

    def bad(x32, g):
        return orig(x32 * np.float32(6.0), g)   # forgets the /6
    monkeypatch.setattr(Q, "block_scale_codes", bad)
    assert _fails(TQ.test_worked_example_by_hand)


def test_mutant_global_scale_wrong_constant(monkeypatch):
    monkeypatch.setattr(Q, "F32_2688", np.float32(448.0))
    assert _fails(TQ.test_global_scale_is_float32_amax_over_2688)


def test_mutant_nibble_order_swapped(monkeypatch):
    def bad_pack(codes):
        codes = np.asarray(codes, np.uint8)
        return (codes[:, 1::2] | (codes[:, 0::2] << 4)).astype(np.uint8)
    monkeypatch.setattr(Q, "pack_codes", bad_pack)
    assert _fails(TQ.test_worked_example_by_hand)


def test_mutant_gemm_transposed_b(monkeypatch):
    orig = Q.dequantize_unscaled

    def bad(codes, scales):
        v = orig(codes, scales)
        return v[::-1] if v.ndim == 2 and v.shape[0] == 5 else v    # rows of B reversed
    monkeypatch.setattr(M, "dequantize_unscaled", bad)
    assert _fails(TG.test_grouped_gemm_equals_exact_rational, 0)


def test_mutant_gemm_drops_b_global_scale(monkeypatch):
    def bad(a_codes, a_scales, a_g, b_codes, b_scales, b_g, offsets, a_rows=None, want_absdot=True):
        return ORIG_GEMM(a_codes, a_scales, a_g, b_codes, b_scales, np.ones_like(b_g), offsets,
                         a_rows=a_rows, want_absdot=want_absdot)
    monkeypatch.setattr(TG, "grouped_gemm", bad)
    assert _fails(TG.test_grouped_gemm_equals_exact_rational, 1)


def test_mutant_gemm_ignores_row_gather(monkeypatch):
    def bad(a_codes, a_scales, a_g, b_codes, b_scales, b_g, offsets, a_rows=None, want_absdot=True):
        return ORIG_GEMM(a_codes, a_scales, a_g, b_codes, b_scales, b_g, offsets,
                         a_rows=None, want_absdot=want_absdot)
    monkeypatch.setattr(TG, "grouped_gemm", bad)
    assert _fails(TG.test_grouped_gemm_equals_exact_rational, 2)


def test_mutant_route_softmax_not_renormalised(monkeypatch):
    def bad(logits, k):
        ids, _ = ORIG_ROUTE(logits, k)
        l = np.asarray(logits, np.float64)
        p = np.exp(l - l.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        return ids, np.take_along_axis(p, ids.astype(np.int64), axis=1).astype(np.float32)
    monkeypatch.setattr(TM.M, "route", bad)
    assert _fails(TM.test_route_weights_are_renormalised_softmax)


def test_mutant_route_ties_to_higher_id(monkeypatch):
    def bad(logits, k):
        l = np.asarray(logits, np.float64)
        E = l.shape[1]
        ids = (E - 1 - np.argsort(-l[:, ::-1], axis=1, kind="stable"))[:, :k]
        sel = np.take_along_axis(l, ids, axis=1)
        ex = np.exp(sel - sel[:, :1])
        return ids.astype(np.int32), (ex / ex.sum(axis=1, keepdims=True)).astype(np.float32)
    monkeypatch.setattr(TM.M, "route", bad)
    assert _fails(TM.test_route_ties_go_to_lower_id)


def test_mutant_permute_unstable(monkeypatch):
    def bad(topk_ids, topk_w, E):
        T, k = topk_ids.shape
        flat = topk_ids.reshape(-1).astype(np.int64)
        order = np.lexsort((-np.arange(T * k), flat))          # descending inside an expert
        counts = np.bincount(flat, minlength=E)
        offsets = np.concatenate([[0], np.cumsum(counts)])
        perm_of = np.empty(T * k, np.int64)
        perm_of[order] = np.arange(T * k)
        return (counts.astype(np.int32), offsets.astype(np.int32), (order // k).astype(np.int32),
                perm_of.astype(np.int32), topk_w.reshape(-1)[order])
    monkeypatch.setattr(TM.M, "permute", bad)
    assert _fails(TM.test_permute_brute_force_and_invariants, 40, 16, 3)


def test_mutant_swiglu_halves_swapped(monkeypatch):
    def bad(y1):
        y1 = np.asarray(y1, np.float64)
        I = y1.shape[1] // 2
        return M.silu(y1[:, I:]) * y1[:, :I]
    monkeypatch.setattr(TM.M, "swiglu", bad)
    assert _fails(TM.test_swiglu_gate_then_up)


def test_mutant_combine_weights_of_wrong_slot(monkeypatch):
    def bad(y2, perm_of_assignment, topk_w):
        return ORIG_COMBINE(y2, perm_of_assignment, np.asarray(topk_w)[:, ::-1])
    monkeypatch.setattr(TM.M, "combine", bad)
    assert _fails(TM.test_combine_equal_rows_and_brute_force)


def test_mutant_e4m3_truncating_encoder(monkeypatch):
    def bad(t):
        t = np.minimum(np.asarray(t, np.float64), 448.0)
        return (np.searchsorted(F.E4M3_POS, t, side="right") - 1).astype(np.uint8)
    monkeypatch.setattr(F, "e4m3_encode_satfinite", bad)
    assert _fails(TF.test_e4m3_encode_matches_torch_rne)


def test_mutant_absdot_doubled(monkeypatch):
    # a looser error-bound scale would widen every GEMM tolerance unnoticed
    def bad(*a, **kw):
        y, absdot = ORIG_GEMM(*a, **kw)
        return y, absdot * 2
    monkeypatch.setattr(TG, "grouped_gemm", bad)
    assert _fails(TG.test_grouped_gemm_equals_exact_rational, 0)


def test_mutant_absdot_per_tensor_scales_twice(monkeypatch):
    def bad(a_codes, a_scales, a_g, b_codes, b_scales, b_g, offsets, a_rows=None, want_absdot=True):
        y, absdot = ORIG_GEMM(a_codes, a_scales, a_g, b_codes, b_scales, b_g, offsets, a_rows=a_rows,
                              want_absdot=want_absdot)
        gb = np.repeat(np.asarray(b_g, np.float64), np.diff(np.asarray(offsets, np.int64)))
        return y, absdot * float(np.float32(a_g)) * gb[:, None]
    monkeypatch.setattr(TG, "grouped_gemm", bad)
    assert _fails(TG.test_grouped_gemm_equals_exact_rational, 1)


def test_mutant_layer_swaps_permutation_maps(monkeypatch):
    # the gather of gate_up and the combine read the two maps of the
    # permutation; handing each the other's map must break the routed pin
    def bad(topk_ids, topk_w, E):
        counts, offsets, src, perm_of, pw = ORIG_PERMUTE(topk_ids, topk_w, E)
        return counts, offsets, perm_of // topk_ids.shape[1], src * topk_ids.shape[1], pw
    monkeypatch.setattr(M, "permute", bad)
    assert _fails(TM.test_layer_routed_matches_token_by_token_definition)


def test_mutant_layer_gathers_assignment_not_token(monkeypatch):
    # perm_src_token holding the flat assignment index instead of its token
    def bad(topk_ids, topk_w, E):
        T, k = topk_ids.shape
        counts, offsets, src, perm_of, pw = ORIG_PERMUTE(topk_ids, topk_w, E)
        order = np.argsort(topk_ids.reshape(-1), kind="stable")
        return counts, offsets, (order % T).astype(np.int32), perm_of, pw
    monkeypatch.setattr(M, "permute", bad)
    assert _fails(TM.test_layer_routed_matches_token_by_token_definition)


def test_mutant_layer_combine_ignores_permutation(monkeypatch):
    def bad(y2, perm_of_assignment, topk_w):
        return ORIG_COMBINE(y2, np.arange(len(perm_of_assignment), dtype=np.int32), topk_w)
    monkeypatch.setattr(M, "combine", bad)
    assert _fails(TM.test_layer_routed_matches_token_by_token_definition)


ORIG_GEMM = M.grouped_gemm
ORIG_ROUTE = M.route
ORIG_COMBINE = M.combine
ORIG_PERMUTE = M.permute


# ------------------------------------------------------------------ MXFP4 oracle
import oracle.mx as MXO
import tests.test_oracle_mx as TMX


def test_mutant_mx_exponent_off_by_one(monkeypatch):
    orig = MXO.mx_shared_exponent
    monkeypatch.setattr(MXO, "mx_shared_exponent", lambda a: np.clip(orig(a) + 1, -127, 127))
    assert _fails(TMX.test_worked_block_by_hand)


def test_mutant_mx_e8m0_bias(monkeypatch):
    monkeypatch.setattr(MXO, "E8M0_BIAS", 128)
    assert _fails(TMX.test_e8m0_closed_form_and_library)


def test_mutant_mx_ties_away_from_zero(monkeypatch):
    def bad(v):
        v = np.minimum(np.asarray(v, np.float64), 6.0)
        d = np.abs(v[..., None] - F.E2M1_MAGNITUDES)
        return (7 - np.argmin(d[..., ::-1], axis=-1)).astype(np.uint8)
    monkeypatch.setattr(MXO, "e2m1_encode_magnitude", bad)
    assert _fails(TMX.test_worked_block_by_hand)


def test_mutant_mx_gemm_drops_b_block_scale(monkeypatch):
    orig = MXO.mx_dequantize

    def bad(codes, scales):
        return orig(codes, np.full_like(scales, 127) if codes.ndim == 2 and codes.shape[0] == 5 else scales)
    monkeypatch.setattr(MXO, "mx_dequantize", bad)
    assert _fails(TMX.test_mx_gemm_equals_exact_rational, 0)


def test_mutant_mx_zero_block_keeps_sign(monkeypatch):
    orig = MXO.mx_quantize

    def bad(x):
        codes, scales = orig(x)
        q = Q.unpack_codes(codes)
        q[np.signbit(np.asarray(x, np.float32)) & (np.asarray(x) == 0)] |= 8
        return Q.pack_codes(q), scales
    monkeypatch.setattr(MXO, "mx_quantize", bad)
    assert _fails(TMX.test_quantiser_invariants)


# ------------------------------------------------------------------ FP8 block-scaled oracle
import oracle.fp8 as P8
import tests.test_oracle_fp8 as TP8


def test_mutant_fp8_scale_constant(monkeypatch):
    monkeypatch.setattr(P8, "F32_448", np.float32(240.0))       # the E4M3 max of another FP8 variant
    assert _fails(TP8.test_worked_block_by_hand)


def test_mutant_fp8_truncating_encoder(monkeypatch):
    def bad(t):
        t = np.minimum(np.asarray(t, np.float64), 448.0)
        return (np.searchsorted(F.E4M3_POS, t, side="right") - 1).astype(np.uint8)
    monkeypatch.setattr(P8, "e4m3_encode_satfinite", bad)
    assert _fails(TP8.test_encoder_matches_torch_float8_cast)


def test_mutant_fp8_weight_scale_per_row(monkeypatch):
    # the weight scale indexed by output row instead of by its 128-row block
    orig = P8.fp8_row_scales

    def bad(scales, block_rows, rows):
        if block_rows != 128:
            return orig(scales, block_rows, rows)
        sc = np.asarray(scales)
        idx = np.minimum(np.arange(rows), sc.shape[-2] - 1)
        return orig(sc[..., idx, :], 1, rows)
    monkeypatch.setattr(P8, "fp8_row_scales", bad)
    assert _fails(TP8.test_fp8_gemm_equals_exact_rational)


def test_mutant_fp8_gemm_drops_activation_scale(monkeypatch):
    orig = P8.fp8_row_scales

    def bad(scales, block_rows, rows):
        return orig(np.ones_like(scales) if block_rows == 1 else scales, block_rows, rows)
    monkeypatch.setattr(P8, "fp8_row_scales", bad)
    assert _fails(TP8.test_fp8_gemm_equals_exact_rational)


def test_mutant_fp8_gemm_scales_dequantised_operands(monkeypatch):
    # products of the dequantised values (E4M3 x float32 scale on each side)
    # instead of scaled exact block sums: rounding where the code products cancel
    def bad(a_codes, a_scales, b_codes, b_scales, offsets, a_rows=None, want_absdot=True):
        E, N, K = b_codes.shape
        offsets = np.asarray(offsets, np.int64)
        y = np.zeros((int(offsets[-1]), N), np.float32)
        for e in range(E):
            p0, p1 = int(offsets[e]), int(offsets[e + 1])
            rows = np.arange(p0, p1) if a_rows is None else np.asarray(a_rows)[p0:p1]
            y[p0:p1] = (P8.fp8_dequantize(a_codes[rows], a_scales[rows], 1)
                        @ P8.fp8_dequantize(b_codes[e], b_scales[e], 128).T).astype(np.float32)
        return y, np.zeros_like(y, np.float64)
    monkeypatch.setattr(P8, "fp8_grouped_gemm", bad)
    assert _fails(TP8.test_fp8_gemm_single_block_terms_correctly_rounded)
