"""The whole layer forward captured in one HIP graph and replayed: every
library call must be capturable (no allocation, no memset nodes, one stream)
and every replay must equal the eager forward bit for bit, also with other
eager work and synchronisations between the replays."""

import pytest
import torch

import expert_token_routing_router_amd as moe
from expert_token_routing_router_amd import layer
import moe_workloads as W

from gpu_util import to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["switch", "deepseek"])
def test_graph_replays_match_eager(name):
    cfg = W.small(name)
    print(f"[graph {name}] N={cfg['N']} E={cfg['E']} k={cfg['k']}", flush=True)
    inp = moe.prepare_weights(cfg, to_dev(W.make_inputs(cfg)))
    buf = moe.MoeBuffers(cfg)
    outs = ["logits", "topk_idx", "topk_w", "counts", "row_of_slot", "token_of_row",
            "expert_offsets", "x_perm", "y_perm", "y"]

    def snapshot():
        return {k: getattr(buf, k).detach().clone() for k in outs}

    moe.moe_forward(buf, inp)
    torch.cuda.synchronize()
    eager = snapshot()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the capture stream
        moe.moe_forward(buf, inp)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        moe.moe_forward(buf, inp)
    torch.cuda.synchronize()

    for replay in range(4):
        for k in outs:  # clobber every output so a skipped node cannot pass
            getattr(buf, k).view(torch.uint8).fill_(0xA5)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = snapshot()
        M = int(eager["expert_offsets"][-1].item())
        for k in outs:
            a, b = got[k], eager[k]
            if k in ("x_perm", "y_perm"):  # rows >= M (admitted rows) are never written
                a, b = a[:M], b[:M]
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {replay}: {k}"
        # unrelated eager work between replays
        _ = (torch.randn(4096, device="cuda") * 3).sum().item()
