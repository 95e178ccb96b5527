"""GPU parity of the router's backward and the auxiliary load-balancing loss
(moe_router_backward) against the oracle on the same inputs: the oracle's own
logits and selection, a seeded gradient at the combine weights with the
dropped slots' entries zero (as moe_combine_backward leaves them), and a
seeded input gradient the router's term is added to.  Tolerances: dz, dW_r,
db and the loss per-tensor max relative error 1e-4 (fp32 arithmetic against
the oracle's fp64), dx the layer tolerance of its dtype."""

import numpy as np
import pytest
import torch

import expert_token_routing_router_amd as moe
import moe_workloads as W
import oracle

from gpu_util import TOL, as_tensor, n, rel_err, threads

pytestmark = pytest.mark.gpu

CASES = {
    "toy-small": W.small("toy"),
    "switch-small": W.small("switch"),
    "mixtral-small": W.small("mixtral"),
    "deepseek-small": W.small("deepseek"),
    "zipf-small-cf1.0": W.with_(W.small("zipf"), cf=1.0),
    "deepseek-full": W.full("deepseek"),
    "switch-full": W.full("switch"),
}


def _run(cfg, coef, seed=3):
    N, d, E, k = cfg["N"], cfg["d"], cfg["E"], cfg["k"]
    dt = cfg["dtype"]
    tdt = torch.float32 if dt == "fp32" else torch.bfloat16
    inp = W.make_inputs(cfg, weights=False)
    oracle.set_threads(threads())
    r = oracle.route(cfg, n(inp["x"]), n(inp["w_router"]), n(inp["router_bias"]),
                     n(inp["sel_bias"]))
    dsp = oracle.dispatch(cfg, r["topk_idx"])
    g = torch.Generator().manual_seed(seed)
    dtw = torch.randn(N, k, generator=g).numpy().astype(np.float32)
    dtw[dsp["row_of_slot"] < 0] = 0.0  # dropped slots pass no gradient
    dx_in = torch.randn(N, d, generator=g).to(tdt)
    ref = oracle.router_backward(cfg, n(inp["x"]), n(inp["w_router"]), r["logits"],
                                 r["topk_idx"], dtw, r["counts"], coef, dx_in=n(dx_in))
    desc = moe.desc_from_workload(cfg)
    dev = "cuda"
    dl = torch.full((N, E), 9.0, device=dev)
    dw = torch.full((E, d), 9.0, device=dev)
    db = torch.full((E,), 9.0, device=dev)
    dx = dx_in.to(dev)
    loss = torch.full((1,), 9.0, device=dev)
    ws = moe.workspace(moe.moe_router_backward_workspace_size(desc), dev)
    moe.moe_router_backward(desc, inp["x"].to(dev), inp["w_router"].to(dev),
                            torch.from_numpy(r["logits"]).to(dev),
                            torch.from_numpy(r["topk_idx"]).to(dev), torch.from_numpy(dtw).to(dev),
                            torch.from_numpy(r["counts"]).to(dev), coef, dl, dw, db, dx, True, loss,
                            ws)
    torch.cuda.synchronize()
    return ref, {"dz": dl.cpu(), "dw_router": dw.cpu(), "db": db.cpu(), "dx": dx.cpu(),
                 "aux_loss": float(loss.item())}


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("coef", [0.0, 0.01])
def test_router_backward_matches_oracle(name, coef):
    cfg = CASES[name]
    if name.endswith("full") and coef == 0.0:
        pytest.skip("full sizes run once, with the auxiliary loss")
    print(f"[router backward {name}] N={cfg['N']} d={cfg['d']} E={cfg['E']} k={cfg['k']} "
          f"{cfg['score']} coef={coef}", flush=True)
    ref, got = _run(cfg, coef)
    for key in ("dz", "dw_router", "db"):
        err = rel_err(got[key], torch.from_numpy(ref[key]))
        assert err <= 1e-4, f"{key} max rel err {err:.3e}"
    err = rel_err(got["dx"].float(), as_tensor(ref["dx"], cfg["dtype"]).float())
    assert err <= TOL[cfg["dtype"]], f"dx max rel err {err:.3e}"
    if coef:
        assert abs(got["aux_loss"] - ref["aux_loss"]) <= 1e-5 * abs(ref["aux_loss"])
    else:
        assert got["aux_loss"] == 0.0


def test_router_backward_empty_batch():
    """No tokens: zero weight and bias gradients, zero loss, nothing else read."""
    cfg = W.with_(W.small("deepseek"), N=0)
    desc = moe.desc_from_workload(cfg)
    E, d = cfg["E"], cfg["d"]
    dw = torch.full((E, d), 9.0, device="cuda")
    db = torch.full((E,), 9.0, device="cuda")
    loss = torch.full((1,), 9.0, device="cuda")
    counts = torch.zeros(E, dtype=torch.int32, device="cuda")
    moe.moe_router_backward(desc, None, None, None, None, None, counts, 0.01, None, dw, db, None,
                            False, loss, None)
    torch.cuda.synchronize()
    assert bool((dw == 0).all()) and bool((db == 0).all()) and float(loss.item()) == 0.0
