"""The one-call expert FFN (moe_expert_ffn: gate_up + SwiGLU requant + down,
one persistent launch from 48 rows per expert) against the two grouped-GEMM
calls it replaces.  Both run the same task bodies with the same summation
order, so h (codes and scales) and the bf16 down rows must agree bit for bit;
the two-call path itself is checked against the oracle stage by stage
(test_gpu_gemm.py, test_gpu_whole_decode.py), and the layer built on the one
call end to end (test_gpu_full.py, the smoke check).  The launch's error word
(a down task that stopped waiting for its h rows) must stay 0."""
import numpy as np
import pytest
import torch

import block_scaled_fp4_permute_amd as m
import workloads
from block_scaled_fp4_permute_amd.layer import quantize_expert_weights
from tests.gpu_common import DEV, up

pytestmark = pytest.mark.gpu


def _two_launch(xq, src, offsets, w, g_h, H, I, M, hint):
    hq = m.nvfp4_grouped_gemm(xq, w["gu_c"], w["gu_s"], w["gu_g"], offsets, m_total=M, a_rows=src,
                              epilogue=m.EPI_SWIGLU_NVFP4, out_g=g_h, b_packed=w["gu_p"],
                              max_rows_per_expert_hint=hint)
    y = m.nvfp4_grouped_gemm(hq, w["dn_c"], w["dn_s"], w["dn_g"], offsets, m_total=M, epilogue=m.EPI_BF16,
                             b_packed=w["dn_p"], max_rows_per_expert_hint=hint)
    return hq, y


def _compare(xq, src, offsets, w, g_h, H, I, M, hint=0, what=""):
    ws = m.moe_expert_ffn_workspace(offsets.numel() - 1, M, H, I, DEV)
    ws.fill_(0xA5)                     # the call must not rely on a cleared workspace
    h1, y1 = m.moe_expert_ffn(xq, src, offsets, w["gu_p"], w["gu_g"], w["dn_p"], w["dn_g"], g_h, H=H, I=I,
                              m_total=M, workspace=ws, max_rows_per_expert_hint=hint)
    # a second call on the same workspace (its counters and lists rewritten)
    h1b, y1b = m.moe_expert_ffn(xq, src, offsets, w["gu_p"], w["gu_g"], w["dn_p"], w["dn_g"], g_h, H=H, I=I,
                                m_total=M, workspace=ws, max_rows_per_expert_hint=hint)
    h2, y2 = _two_launch(xq, src, offsets, w, g_h, H, I, M, hint)
    torch.cuda.synchronize()
    E = offsets.numel() - 1
    if (hint if hint > 0 else M // E) >= 48:    # the one persistent launch ran
        err_word = int(ws[:256].view(torch.int32)[8].item())
        assert err_word == 0, f"{what}: a down task gave up waiting"
    for a, b, name in ((h1.codes, h2.codes, "h codes"), (h1.scales, h2.scales, "h scales"), (y1, y2, "y"),
                       (h1b.codes, h2.codes, "h codes (2nd call)"), (y1b, y2, "y (2nd call)")):
        if not torch.equal(a, b):
            bad = (a != b).nonzero()
            raise AssertionError(f"{what}: {name} differ at {bad.shape[0]} places, first {bad[0].tolist()}")


def _layer_inputs(cfg):
    logits = torch.from_numpy(workloads.logits(cfg)).to(DEV)
    x = torch.from_numpy(workloads.activations(cfg)).to(DEV).to(torch.bfloat16)
    r, xq = m.moe_route_quantize(logits, cfg.k, x)
    w_gu, w_dn = workloads.torch_expert_weights(cfg, DEV)
    wq = quantize_expert_weights(w_gu, w_dn).pack()
    del w_gu, w_dn
    w = dict(gu_c=wq.gu_codes, gu_s=wq.gu_scales, gu_g=wq.gu_g, gu_p=wq.gu_packed,
             dn_c=wq.dn_codes, dn_s=wq.dn_scales, dn_g=wq.dn_g, dn_p=wq.dn_packed)
    g_h = up(np.array([np.float32(workloads.H_CALIBRATION_AMAX[cfg.index]) / np.float32(2688.0)], np.float32))
    return r, xq, w, g_h


@pytest.mark.parametrize("cfg_index", [0, 1, 2, 3])
def test_expert_ffn_equals_two_calls_on_workloads(cfg_index):
    cfg = workloads.CONFIGS[cfg_index]
    print(f"expert ffn cfg={cfg_index} T={cfg.T} E={cfg.E} k={cfg.k}", flush=True)
    r, xq, w, g_h = _layer_inputs(cfg)
    _compare(xq, r.perm_src_token, r.offsets, w, g_h, cfg.H, cfg.I, cfg.T * cfg.k, what=f"config {cfg_index}")


def _random_weights(rng, E, H, I):
    gu_c = up(rng.integers(0, 256, (E, 2 * I, H // 2), dtype=np.uint8))
    gu_s = up(rng.integers(0x28, 0x48, (E, 2 * I, H // 16), dtype=np.uint8))
    dn_c = up(rng.integers(0, 256, (E, H, I // 2), dtype=np.uint8))
    dn_s = up(rng.integers(0x28, 0x48, (E, H, I // 16), dtype=np.uint8))
    return dict(gu_c=gu_c, gu_s=gu_s, gu_g=up(rng.uniform(0.001, 0.01, E).astype(np.float32)),
                gu_p=m.nvfp4_weight_repack(gu_c, gu_s), dn_c=dn_c, dn_s=dn_s,
                dn_g=up(rng.uniform(0.001, 0.01, E).astype(np.float32)), dn_p=m.nvfp4_weight_repack(dn_c, dn_s))


CASES = [
    # E, H, I, counts (None: random), x rows, hint
    (1500, 256, 128, None, 300, 48),          # more experts and chunks than a planner tile (1024), many empty
    (1, 512, 256, [1], 1, 48),                # a single row
    (3, 1024, 64, [0, 700, 5], 50, 64),       # one expert with many chunks (cached weight loads)
    (8, 512, 256, [64, 65, 63, 1, 0, 128, 16, 17], 100, 0),   # chunk-boundary sizes
    (5, 512, 256, [200, 300, 150, 0, 400], 90, 128),           # the MFMA-bound sizes: still one launch
    (16, 512, 256, [8] * 16, 40, 0),          # the few-rows bucket: two launches
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_expert_ffn_equals_two_calls_edge_cases(case):
    E, H, I, counts, rows_x, hint = CASES[case]
    rng = np.random.default_rng(900 + case)
    if counts is None:
        counts = rng.integers(0, 60, E) * (rng.random(E) < 0.8)
        counts[rng.choice(E, 3, replace=False)] = [90, 130, 1]
    counts = np.asarray(counts, np.int64)
    M = int(counts.sum())
    print(f"expert ffn edge case {case}: E={E} H={H} I={I} M={M} hint={hint}", flush=True)
    offsets = up(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32))
    src = up(rng.integers(0, rows_x, max(M, 1)).astype(np.int32))
    xq = m.NVFP4Tensor(up(rng.integers(0, 256, (rows_x, H // 2), dtype=np.uint8)),
                       up(rng.integers(0x28, 0x48, (rows_x, H // 16), dtype=np.uint8)),
                       up(np.array([0.02], np.float32)))
    w = _random_weights(rng, E, H, I)
    g_h = up(np.array([0.05], np.float32))
    _compare(xq, src, offsets, w, g_h, H, I, M, hint=hint, what=f"edge case {case}")


def _fused_combine_check(xq, r, w, g_h, H, I, k, hint=0, what=""):
    """moe_expert_ffn with the combine fused (in the one-launch regime: inside
    the persistent launch) against the same call without it followed by
    moe_unpermute_combine: h, y and the combined output equal bit for bit, on
    two calls in a row over one workspace (its counters cleared by the call)."""
    M = r.perm_src_token.numel()
    T = M // k
    E = r.offsets.numel() - 1
    ws = m.moe_expert_ffn_workspace(E, M, H, I, DEV)
    ws.fill_(0x5A)
    h0, y0 = m.moe_expert_ffn(xq, r.perm_src_token, r.offsets, w["gu_p"], w["gu_g"], w["dn_p"], w["dn_g"], g_h,
                              H=H, I=I, m_total=M, max_rows_per_expert_hint=hint)
    ref = m.moe_unpermute_combine(y0, r.perm_of_assignment, r.topk_w, T, k)
    for call in range(2):
        h1, y1, out = m.moe_expert_ffn(xq, r.perm_src_token, r.offsets, w["gu_p"], w["gu_g"], w["dn_p"], w["dn_g"],
                                       g_h, H=H, I=I, m_total=M, workspace=ws, max_rows_per_expert_hint=hint,
                                       perm_of_assignment=r.perm_of_assignment, topk_w=r.topk_w, k=k)
        torch.cuda.synchronize()
        if (hint if hint > 0 else M // E) >= 48:
            assert int(ws[:256].view(torch.int32)[8].item()) == 0, f"{what}: a down task gave up waiting"
        for a, b, name in ((h1.codes, h0.codes, "h codes"), (y1, y0, "y"), (out, ref, "combined out")):
            if not torch.equal(a, b):
                bad = (a != b).nonzero()
                raise AssertionError(f"{what} call {call}: {name} differ at {bad.shape[0]} places, "
                                     f"first {bad[0].tolist()}")


@pytest.mark.parametrize("cfg_index,hint", [(0, 0), (1, 0), (1, 64), (2, 0), (3, 0)])
def test_expert_ffn_fused_combine_on_workloads(cfg_index, hint):
    cfg = workloads.CONFIGS[cfg_index]
    print(f"fused combine cfg={cfg_index} hint={hint}", flush=True)
    r, xq, w, g_h = _layer_inputs(cfg)
    _fused_combine_check(xq, r, w, g_h, cfg.H, cfg.I, cfg.k, hint=hint, what=f"config {cfg_index} hint {hint}")


@pytest.mark.parametrize("T,E,k,H,I,hint", [(300, 16, 4, 512, 256, 0), (40, 8, 8, 512, 128, 48),
                                            (5, 4, 2, 256, 64, 48), (200, 32, 10, 512, 256, 0),
                                            (500, 64, 1, 1024, 256, 48), (64, 8, 3, 1600, 96, 0)])
def test_expert_ffn_fused_combine_routings(T, E, k, H, I, hint):
    # routed by the library on random logits (k = E: every token at every
    # expert; k = 1; k = 10 past one batch of 8 rows; H = 1600 leaves the last
    # down column group partial)
    rng = np.random.default_rng(T * 7 + E + k)
    print(f"fused combine T={T} E={E} k={k} H={H} I={I} hint={hint}", flush=True)
    logits = up(rng.standard_normal((T, E)).astype(np.float32))
    x = up(rng.standard_normal((T, H)).astype(np.float32)).to(torch.bfloat16)
    r, xq = m.moe_route_quantize(logits, k, x)
    w = _random_weights(rng, E, H, I)
    g_h = up(np.array([0.05], np.float32))
    _fused_combine_check(xq, r, w, g_h, H, I, k, hint=hint, what=f"T={T} E={E} k={k}")
