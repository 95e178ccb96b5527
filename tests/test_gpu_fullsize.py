"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times: routing and the dispatch layout against the oracle run on
every token (bit-exact), the certified-logit bound over every (token, expert)
pair, and the expert FFN and combine on sampled rows / tokens the oracle
computes one by one."""

import concurrent.futures as cf

import numpy as np
import pytest
import torch

import expert_token_routing_router_amd as moe
from expert_token_routing_router_amd import layer
import moe_workloads as W
import oracle

from gpu_util import TOL, TOPK_W_TOL, as_tensor, bits, n, rel_err, threads

pytestmark = pytest.mark.gpu

CASES = {name: W.full(name) for name in W.ORDER}
CASES["zipf-cf1.0"] = W.with_(W.full("zipf"), cf=1.0)
CASES["zipf-cf2.0"] = W.with_(W.full("zipf"), cf=2.0)


def bits_t(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def inputs_on_device(cfg):
    if cfg["name"] == "toy":
        src = W.make_inputs(cfg)
        return {k: (tuple(None if t is None else t.cuda() for t in v) if isinstance(v, tuple)
                    else (v.cuda() if isinstance(v, torch.Tensor) else v)) for k, v in src.items()}
    return W.make_inputs(cfg, device="cuda")


@pytest.mark.parametrize("name", list(CASES))
def test_fullsize(name):
    cfg = CASES[name]
    print(f"[fullsize {name}] N={cfg['N']} d={cfg['d']} h={cfg['h']} E={cfg['E']} k={cfg['k']}",
          flush=True)
    inp = inputs_on_device(cfg)
    buf = moe.MoeBuffers(cfg)
    moe.moe_forward(buf, moe.prepare_weights(cfg, inp))
    torch.cuda.synchronize()
    dt = cfg["dtype"]

    # Routing: the oracle on every token.
    x_h, wr_h = inp["x"].cpu(), inp["w_router"].cpu()
    rb = None if inp.get("router_bias") is None else inp["router_bias"].cpu()
    sb = None if inp.get("sel_bias") is None else inp["sel_bias"].cpu()
    oracle.set_threads(threads())
    r = oracle.route(cfg, n(x_h), n(wr_h), n(rb), n(sb))
    assert np.array_equal(buf.topk_idx.cpu().numpy(), r["topk_idx"])
    assert np.array_equal(buf.counts.cpu().numpy(), r["counts"])
    assert np.abs(buf.topk_w.cpu().numpy() - r["topk_w"]).max() <= TOPK_W_TOL
    zr = torch.from_numpy(r["logits"])
    sel = torch.from_numpy(r["topk_idx"]).long()
    zg = buf.logits.cpu()
    assert torch.equal(bits_t(zg.gather(1, sel)), bits_t(zr.gather(1, sel)))
    if dt == "bf16":
        m = (2.0 ** -16 * x_h.double().norm(dim=1)[:, None] * wr_h.double().norm(dim=1)[None, :]
             + 2.0 ** -22 * zr.double().abs() + 1e-27)
        assert bool(((zg.double() - zr.double()).abs() <= m).all()), "certified bound violated"

    # Layout: the oracle's dispatch of the oracle's routing.
    dsp = oracle.dispatch(cfg, r["topk_idx"])
    for key in ["row_of_slot", "token_of_row", "slot_of_row", "expert_offsets", "admitted",
                "rank_offsets", "rank_counts"]:
        assert np.array_equal(getattr(buf, key).cpu().numpy(), dsp[key]), key
    M = dsp["num_rows"]
    tor = buf.token_of_row[:M].long()
    assert torch.equal(bits_t(buf.x_perm[:M]), bits_t(inp["x"][tor]))

    # Expert FFN on sampled rows: first and last row of some experts + random.
    rng = np.random.default_rng(7)
    off = dsp["expert_offsets"]
    rows = set(rng.choice(M, size=min(M, 16), replace=False).tolist()) if M else set()
    for e in rng.choice(cfg["E"], size=min(cfg["E"], 4), replace=False):
        if off[e + 1] > off[e]:
            rows.update([int(off[e]), int(off[e + 1] - 1)])
    rows = sorted(rows)
    expert_of = np.searchsorted(off, np.array(rows), side="right") - 1
    xp = buf.x_perm.cpu()
    w3 = inp.get("w3")

    def ffn_one(i):
        e = int(expert_of[i])
        return oracle.ffn_row(dt, cfg["act"], n(xp[rows[i]]), n(inp["w1"][e].cpu()),
                              None if w3 is None else n(w3[e].cpu()), n(inp["w2"][e].cpu()))

    with cf.ThreadPoolExecutor(threads()) as ex:
        ref_rows = list(ex.map(ffn_one, range(len(rows))))
    if rows:
        got = buf.y_perm[torch.tensor(rows, device="cuda")].cpu()
        ref = torch.stack([as_tensor(v, dt) for v in ref_rows])
        err = rel_err(got, ref)
        assert err <= TOL[dt], f"sampled y_perm max rel err {err:.3e}"

    # Combine on sampled tokens from the GPU's expert rows (checked above).
    toks = sorted(rng.choice(cfg["N"], size=32, replace=False).tolist())
    ros = buf.row_of_slot.cpu().numpy()[toks]
    used = sorted(set(int(v) for v in ros.ravel() if v >= 0))
    remap = {v: i for i, v in enumerate(used)}
    yp_rows = buf.y_perm[torch.tensor(used, device="cuda").long()].cpu() if used else None
    ros_local = np.vectorize(lambda v: remap.get(int(v), -1))(ros).astype(np.int32)
    shared = None if buf.shared_out is None else n(buf.shared_out.cpu()[toks])
    y_ref = oracle.combine(dt, n(yp_rows) if used else None, ros_local,
                           buf.topk_w.cpu().numpy()[toks], n(x_h[toks]), shared)
    err = rel_err(buf.y.cpu()[toks], as_tensor(y_ref, dt))
    assert err <= TOL[dt], f"sampled y max rel err {err:.3e}"
    full_drop = np.all(ros < 0, axis=1)
    if full_drop.any() and buf.shared_out is None:
        idx = [t for t, f in zip(toks, full_drop) if f]
        assert torch.equal(buf.y.cpu()[idx], x_h[idx])

    # Shared expert (DeepSeek-like) on sampled tokens.
    if buf.shared_out is not None:
        sw1, sw3, sw2 = (None if t is None else n(t[0].cpu()) for t in inp["shared"])
        with cf.ThreadPoolExecutor(threads()) as ex:
            ref_sh = list(ex.map(lambda t: oracle.ffn_row(dt, cfg["act"], n(x_h[t]), sw1, sw3, sw2),
                                 toks[:8]))
        got = buf.shared_out.cpu()[toks[:8]]
        err = rel_err(got, torch.stack([as_tensor(v, dt) for v in ref_sh]))
        assert err <= TOL[dt], f"sampled shared_out max rel err {err:.3e}"


def test_fullsize_zipf_bias_update_reroute():
    """Zipf workload: route, one bias update, route again -- bit-exact."""
    cfg = W.full("zipf")
    inp = W.make_inputs(cfg, device="cuda", weights=False)
    buf = moe.MoeBuffers(cfg)
    layer.route(buf, inp)
    sel = inp["sel_bias"].clone()
    layer.bias_update(buf, sel, cfg["bias_step"])
    layer.route(buf, inp, sel_bias=sel)
    torch.cuda.synchronize()
    oracle.set_threads(threads())
    x_h, wr_h, rb = inp["x"].cpu(), inp["w_router"].cpu(), inp["router_bias"].cpu()
    r1 = oracle.route(cfg, n(x_h), n(wr_h), n(rb), n(inp["sel_bias"].cpu()))
    b = oracle.bias_update(cfg["N"], cfg["k"], r1["counts"], n(inp["sel_bias"].cpu()),
                           cfg["bias_step"])
    assert np.array_equal(bits(sel.cpu()), b.view(np.int32))
    r2 = oracle.select(cfg, r1["logits"], b)
    assert np.array_equal(buf.topk_idx.cpu().numpy(), r2["topk_idx"])
