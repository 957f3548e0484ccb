"""GPU parity of routing/permutation and NVFP4 quantisation: bit-exact against
the oracle on the same seeded inputs."""
import numpy as np
import pytest
import torch

import block_scaled_fp4_permute_amd as m
import workloads
from oracle import moe as OM
from oracle import quant as OQ
from tests.gpu_common import DEV, bf16_up, down, up

pytestmark = pytest.mark.gpu


def _route_case(logits, k):
    T, E = logits.shape
    print(f"route case T={T} E={E} k={k}", flush=True)
    r = m.moe_route_permute(up(logits), k)
    torch.cuda.synchronize()
    ids, w = OM.route(logits, k)
    counts, offsets, src, perm_of, pw = OM.permute(ids, w, E)
    assert np.array_equal(down(r.topk_ids), ids)
    gw = down(r.topk_w)
    assert np.all(np.abs(gw.astype(np.float64) - w) <= 2.0 ** -20 * np.abs(w)), "routing weights"
    assert np.array_equal(down(r.counts), counts)
    assert np.array_equal(down(r.offsets), offsets)
    assert np.array_equal(down(r.perm_src_token), src)
    assert np.array_equal(down(r.perm_of_assignment), perm_of)
    # the permuted weights are the GPU's own topk_w moved by the permutation
    assert np.array_equal(down(r.perm_weight), gw.reshape(-1)[np.argsort(ids.reshape(-1), kind="stable")])
    return r


@pytest.mark.parametrize("cfg", [0, 1, 2, 3])
def test_route_permute_configs(cfg):
    c = workloads.CONFIGS[cfg]
    _route_case(workloads.logits(c), c.k)


@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (1, 256, 8), (5, 7, 7), (129, 64, 3), (1000, 256, 8),
                                   (3, 4096, 32), (70000, 128, 8), (2048, 300, 1)])
def test_route_permute_shapes(T, E, k):
    rng = np.random.default_rng(T * 7 + E)
    _route_case(rng.standard_normal((T, E)).astype(np.float32), k)


def test_route_permute_ties_and_repeat_determinism():
    rng = np.random.default_rng(9)
    logits = rng.integers(-2, 3, (777, 96)).astype(np.float32)    # many exact ties
    logits[5] = 0.0
    logits[6, :] = -0.0
    r1 = _route_case(logits, 6)
    r2 = m.moe_route_permute(up(logits), 6)
    torch.cuda.synchronize()
    for a in ("topk_ids", "topk_w", "counts", "offsets", "perm_src_token", "perm_of_assignment", "perm_weight"):
        assert torch.equal(getattr(r1, a), getattr(r2, a)), a


def test_route_permute_skewed_single_expert():
    logits = np.zeros((4096, 64), np.float32)
    logits[:, 17] = 5.0
    _route_case(logits, 2)


# --------------------------------------------------------------------- quantise
def _quant_case(x32, dtype, g=None):
    rows, cols = x32.shape
    print(f"quant case rows={rows} cols={cols} dtype={dtype} g={g}", flush=True)
    xt = bf16_up(x32) if dtype == torch.bfloat16 else up(x32)
    gt = None if g is None else up(np.array([g], np.float32))
    q = m.nvfp4_quantize(xt, g=gt)
    torch.cuda.synchronize()
    c, s, gg = OQ.quantize(x32, g=g)
    assert down(q.g)[0] == gg
    assert np.array_equal(down(q.scales), s)
    assert np.array_equal(down(q.codes), c)


@pytest.mark.parametrize("rows,cols", [(1, 32), (7, 96), (33, 256), (8, 6144), (513, 160)])
@pytest.mark.parametrize("kind", ["normal", "heavy", "small"])
def test_quantize_bf16_shapes(rows, cols, kind):
    rng = np.random.default_rng(rows * cols)
    x = rng.standard_normal((rows, cols))
    if kind == "heavy":
        x = x * np.exp(rng.uniform(-8, 8, x.shape))
    elif kind == "small":
        x = x * 1e-3
    _quant_case(workloads.to_bf16_values(x.astype(np.float32)), torch.bfloat16)


@pytest.mark.parametrize("rows,cols", [(5, 64), (64, 512)])
def test_quantize_f32_and_given_scale(rows, cols):
    rng = np.random.default_rng(rows + cols)
    x = (rng.standard_normal((rows, cols)) * 3).astype(np.float32)
    _quant_case(x, torch.float32)
    _quant_case(x, torch.float32, g=0.001)        # static scale: saturating blocks
    _quant_case(x, torch.float32, g=0.5)          # static scale: many tiny/zero scales


def test_quantize_zero_rows_and_signed_zeros():
    x = np.zeros((9, 64), np.float32)
    x[3, 5] = 1.5
    x[4, :] = -0.0
    x[7, 16:32] = np.linspace(-1, 1, 16)
    _quant_case(x, torch.float32)
    _quant_case(np.zeros((4, 32), np.float32), torch.bfloat16)


def test_quantize_e4m3_and_e2m1_decision_points():
    # values placed exactly on E2M1 midpoints (after scaling) and block maxima on
    # E4M3 midpoints: every tie rule is exercised on the GPU
    from oracle import formats as F
    mids = (F.E2M1_MAGNITUDES[:-1] + F.E2M1_MAGNITUDES[1:]) / 2
    rows = []
    for s in (1.0, 1.125, 1.875, 2.0 ** -7, 96.0):
        r = np.zeros(16)
        r[0] = 6 * s
        r[1:8] = mids * s
        r[8:15] = -mids * s
        rows.append(r)
    e4 = (F.E4M3_POS[:-1] + F.E4M3_POS[1:]) / 2
    for t in e4[::9]:
        r = np.linspace(-1, 1, 16) * t * 6
        r[3] = t * 6
        rows.append(r)
    x = np.array(rows, np.float32)
    x = np.concatenate([x, x], axis=1)
    _quant_case(x, torch.float32, g=1.0)


def test_quantize_quotients_next_to_e2m1_boundaries():
    # a non-power-of-two per-tensor scale, so x / (s * g) is a rounded float32
    # quotient; elements a few ulp either side of boundary * (s * g) make every
    # E2M1 decision hang on the last bit of that quotient
    from oracle import formats as F
    g = np.float32(0.0371)
    mids = (F.E2M1_MAGNITUDES[:-1] + F.E2M1_MAGNITUDES[1:]) / 2
    rows = []
    for sc in (8, 9, 30, 55, 56, 77, 100, 119, 126):          # E4M3 codes
        sv = np.float32(F.e4m3_decode(np.array([sc], np.uint8))[0])
        b = np.float32(sv * g)
        for shift in (-2, -1, 1, 2):
            r = np.zeros(16, np.float32)
            r[0] = np.float32(np.float32(6.0) * b)               # block maximum: scale code sc
            for i, mval in enumerate(mids):
                v = np.float32(np.float32(mval) * b)
                for _ in range(abs(shift)):
                    v = np.nextafter(v, np.float32(np.inf if shift > 0 else 0), dtype=np.float32)
                r[1 + 2 * i] = v
                r[2 + 2 * i] = -np.nextafter(v, np.float32(0), dtype=np.float32)
            rows.append(r)
    x = np.array(rows, np.float32)
    x = np.concatenate([x, x[::-1]], axis=1)
    c, sc_codes, _ = OQ.quantize(x, g=g)
    assert len(np.unique(OQ.unpack_codes(c))) >= 12          # the cases reach most codes
    _quant_case(x, torch.float32, g=float(g))


def test_quantize_config_activations_and_weights():
    c = workloads.CONFIGS[2]
    _quant_case(workloads.activations(c), torch.bfloat16)
    _quant_case(workloads.gate_up_weight(c, 3), torch.float32)
    _quant_case(workloads.down_weight(c, 200), torch.float32)


# ------------------------------------------------------------------ route + quantise in one call
def _route_quantize_case(logits, x, k, dtype, g=None):
    T, E = logits.shape
    print(f"route+quantise case T={T} E={E} k={k} cols={x.shape[1]} {dtype} g={g}", flush=True)
    xt = (bf16_up(x) if dtype == torch.bfloat16 else up(x.astype(np.float32)))
    gt = None if g is None else up(np.array([g], np.float32))
    r, xq = m.moe_route_quantize(up(logits), k, xt, g=gt)
    torch.cuda.synchronize()
    # the separate calls, themselves checked against the oracle
    r2 = _route_case(logits, k)
    xq2 = m.nvfp4_quantize(xt, g=gt)
    torch.cuda.synchronize()
    for name in ("topk_ids", "topk_w", "counts", "offsets", "perm_src_token", "perm_of_assignment", "perm_weight"):
        assert np.array_equal(down(getattr(r, name)).view(np.uint32), down(getattr(r2, name)).view(np.uint32)), name
    assert np.array_equal(down(xq.codes), down(xq2.codes))
    assert np.array_equal(down(xq.scales), down(xq2.scales))
    assert down(xq.g)[0] == down(xq2.g)[0]
    # and the oracle's quantisation of the same values (a sample of rows for
    # the large configs, with the oracle's per-tensor scale of the whole tensor)
    x32 = x.astype(np.float32)
    gg = OQ.global_scale(x32) if g is None else np.float32(g)
    rows = np.arange(T) if T <= 2048 else np.unique(np.random.default_rng(T).integers(0, T, 256))
    c, s, gq = OQ.quantize(x32[rows], g=gg)
    assert down(xq.g)[0] == gg == gq
    assert np.array_equal(down(xq.scales)[rows], s)
    assert np.array_equal(down(xq.codes)[rows], c)


@pytest.mark.parametrize("cfg", [0, 1, 2, 3])
def test_route_quantize_configs(cfg):
    c = workloads.CONFIGS[cfg]
    _route_quantize_case(workloads.logits(c), workloads.activations(c), c.k, torch.bfloat16)


@pytest.mark.parametrize("T,E,k,cols,dt,g", [(1, 1, 1, 32, "bf16", None), (5, 7, 7, 96, "f32", None),
                                             (129, 64, 3, 256, "bf16", 0.01), (3, 4096, 32, 64, "bf16", None),
                                             (1000, 300, 1, 160, "f32", 0.5)])
def test_route_quantize_shapes(T, E, k, cols, dt, g):
    rng = np.random.default_rng(T * 3 + E + cols)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    x = rng.standard_normal((T, cols)) * 2
    x = workloads.to_bf16_values(x.astype(np.float32)) if dt == "bf16" else x.astype(np.float32)
    _route_quantize_case(logits, x, k, torch.bfloat16 if dt == "bf16" else torch.float32, g)
