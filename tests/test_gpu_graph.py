"""A layer step recorded into a HIP graph (the launch mode bench.py times)
replays the eager step's kernels: every replay's outputs equal the eager
step's bit for bit, with eager steps on other inputs in between, for the
one-launch FFN (Zipf decode, 64 rows per expert) and the two-launch path
(T=256, 8 rows per expert)."""
import numpy as np
import pytest
import torch

import workloads
from block_scaled_fp4_permute_amd.layer import MoELayer, capture_step, quantize_expert_weights
from tests.gpu_common import DEV, up

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cfg_index", [2, 1])
def test_graph_replay_equals_eager(cfg_index):
    c = workloads.CONFIGS[cfg_index]
    print(f"graph replay cfg={cfg_index}", flush=True)
    logits, x = up(workloads.logits(c)), up(workloads.activations(c)).to(torch.bfloat16)
    # other inputs for the eager steps in between: the same shapes, new draws
    logits2, x2 = logits.flip(0).contiguous(), (x * 0.5).flip(0).contiguous()
    w_gu, w_dn = workloads.torch_expert_weights(c, DEV)
    wq = quantize_expert_weights(w_gu, w_dn).pack()
    del w_gu, w_dn
    g_h = torch.tensor([workloads.H_CALIBRATION_AMAX[c.index] / 2688.0], dtype=torch.float32, device=DEV)
    layer = MoELayer(c.T, c.H, c.I, c.E, c.k, DEV)
    layer.forward(logits, x, wq, g_h)
    torch.cuda.synchronize()
    ref = {"out": layer.out.clone(), "h": layer.hq.codes.clone(), "hs": layer.hq.scales.clone(),
           "src": layer.routing.perm_src_token.clone(), "w": layer.routing.topk_w.clone()}
    graph = capture_step(layer, logits, x, wq, g_h)
    torch.cuda.synchronize()
    for rep in range(3):
        layer.forward(logits2, x2, wq, g_h)          # eager work on other inputs in between
        torch.cuda.synchronize()
        assert not torch.equal(layer.out, ref["out"])
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(layer.out, ref["out"]), f"replay {rep}: output"
        assert torch.equal(layer.hq.codes, ref["h"]) and torch.equal(layer.hq.scales, ref["hs"]), f"replay {rep}: h"
        assert torch.equal(layer.routing.perm_src_token, ref["src"]) and torch.equal(layer.routing.topk_w, ref["w"])
        if (c.T * c.k) // c.E >= 48:               # the one persistent launch ran: its error word
            assert int(layer.ffn_ws.view(torch.int32)[8].item()) == 0, "a down task stopped waiting for its h rows"
