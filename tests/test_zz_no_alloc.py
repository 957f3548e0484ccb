"""The no-allocation route + quantise entry point against the one with a
caller workspace: same kernels, so every output must agree bit for bit.  Two
calls in a row on one GPU, the second smaller, so the second runs on scratch
that still holds the first call's contents."""
import numpy as np
import pytest
import torch

import block_scaled_fp4_permute_amd as m
import workloads
from tests.gpu_common import DEV

pytestmark = pytest.mark.gpu


def _outputs(T, E, k, cols):
    i32 = dict(dtype=torch.int32, device=DEV)
    r = m.Routing(torch.full((T, k), -7, **i32), torch.full((T, k), -7.0, device=DEV), torch.full((E,), -7, **i32),
                  torch.full((E + 1,), -7, **i32), torch.full((T * k,), -7, **i32), torch.full((T * k,), -7, **i32),
                  torch.full((T * k,), -7.0, device=DEV))
    xq = m.NVFP4Tensor(torch.full((T, cols // 2), 0xEE, dtype=torch.uint8, device=DEV),
                       torch.full((T, cols // 16), 0xEE, dtype=torch.uint8, device=DEV),
                       torch.full((1,), -7.0, device=DEV))
    return r, xq


def _same(a, b, what):
    assert torch.equal(a, b), what


@pytest.mark.parametrize("order", ["large_then_small"])
def test_route_quantize_noalloc_matches_workspace_call(order):
    cases = [(workloads.CONFIGS[2], 2048, 6144), (workloads.small_variant(workloads.CONFIGS[1], E=64, k=4, index=1),
                                                  100, 512)]
    for cfg, T, cols in cases:
        print(f"noalloc route+quantize T={T} E={cfg.E} k={cfg.k} cols={cols}", flush=True)
        logits = torch.from_numpy(workloads.logits(cfg, T=T)).to(DEV)
        x = torch.from_numpy(np.ascontiguousarray(workloads.activations(cfg, T=T)[:, :cols])).to(DEV).to(torch.bfloat16)
        r1, q1 = _outputs(T, cfg.E, cfg.k, cols)
        r2, q2 = _outputs(T, cfg.E, cfg.k, cols)
        m.moe_route_quantize(logits, cfg.k, x, out=r1, xq=q1)
        m.moe_route_quantize_noalloc(logits, cfg.k, x, out=r2, xq=q2)
        torch.cuda.synchronize()
        for f in ("topk_ids", "topk_w", "counts", "offsets", "perm_src_token", "perm_of_assignment", "perm_weight"):
            _same(getattr(r1, f), getattr(r2, f), f"{f} T={T}")
        _same(q1.codes, q2.codes, "codes")
        _same(q1.scales, q2.scales, "scales")
        _same(q1.g, q2.g, "g")
        assert int(r2.counts.sum()) == T * cfg.k
