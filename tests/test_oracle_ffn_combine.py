"""Pins of the oracle's expert FFN, combine and whole-layer forward.  CPU only."""

import numpy as np
import pytest
import torch

import oracle
import moe_workloads as W


def _bf16(a):
    return torch.from_numpy(np.asarray(a, np.float32)).bfloat16()


def _torch_ffn(x, w1, w3, w2, act, dtype):
    """Library reference: torch fp64 matmuls and activations, with H and O
    rounded to the dtype at the same two points."""
    xd = x.double()
    u = xd @ w1.double().T
    if act == "relu":
        hdn = torch.relu(u)
    elif act == "gelu":
        hdn = torch.nn.functional.gelu(u)  # exact erf form
    else:
        hdn = torch.nn.functional.silu(u) * (xd @ w3.double().T)
    tdt = torch.float32 if dtype == "fp32" else torch.bfloat16
    hdn = hdn.to(tdt).double()
    return (hdn @ w2.double().T).to(tdt)


@pytest.mark.parametrize("act,dtype", [("relu", "fp32"), ("gelu", "bf16"), ("swiglu", "bf16"),
                                       ("relu", "bf16"), ("swiglu", "fp32")])
def test_ffn_rows_match_library(act, dtype):
    torch.manual_seed(30)
    E, d, h = 3, 64, 96
    tdt = torch.float32 if dtype == "fp32" else torch.bfloat16
    x = torch.randn(40, d).to(tdt)
    w1 = (torch.randn(E, h, d) * 0.1).to(tdt)
    w3 = (torch.randn(E, h, d) * 0.1).to(tdt) if act == "swiglu" else None
    w2 = (torch.randn(E, d, h) * 0.1).to(tdt)
    off = np.array([0, 7, 7, 40], np.int32)  # one empty expert
    y = oracle.expert_ffn(dtype, act, W.to_numpy(x), off, W.to_numpy(w1),
                          W.to_numpy(w3), W.to_numpy(w2))
    for e in range(E):
        lo, hi = off[e], off[e + 1]
        if hi == lo:
            continue
        ref = _torch_ffn(x[lo:hi], w1[e], None if w3 is None else w3[e], w2[e], act, dtype)
        got = torch.from_numpy(y[lo:hi]) if dtype == "fp32" else W.from_numpy_bf16(y[lo:hi])
        err = (got.double() - ref.double()).abs().max() / ref.double().abs().max()
        # H is rounded on both sides from nearly equal fp64 sums; a rare one-ulp
        # difference in H is the only source of disagreement.
        assert err < (1e-6 if dtype == "fp32" else 1e-2), (e, float(err))
        same = (got.double() == ref.double()).float().mean()
        assert same > (0.99 if dtype == "fp32" else 0.9)


def test_bf16_rounding_is_round_to_nearest_even():
    """The combine's single rounding to bf16 of an exact fp64 value equals
    torch's fp32->bf16 cast (round-to-nearest-even), ties included."""
    rng = np.random.default_rng(31)
    base = _bf16(rng.standard_normal(2000)).float().numpy()
    # exact midpoints between neighbouring bf16 values, plus random values
    nxt = np.nextafter(base, np.float32(np.inf))
    up = torch.from_numpy(nxt).bfloat16().float().numpy()
    up = np.where(up == base, torch.from_numpy((base * (1 + 2 ** -7)).astype(np.float32))
                  .bfloat16().float().numpy(), up)
    mids = ((base.astype(np.float64) + up.astype(np.float64)) / 2).astype(np.float32)
    vals = np.concatenate([mids, rng.standard_normal(2000).astype(np.float32)])
    n = vals.size
    ones = W.to_numpy(_bf16(np.ones((1, 1))))
    y = oracle.combine("bf16", ones, np.zeros((n, 1), np.int32), vals[:, None])
    ref = torch.from_numpy(vals).bfloat16()
    assert np.array_equal(y[:, 0], W.to_numpy(ref))


def test_dropped_rows_leave_layer_unchanged():
    """A token with every slot dropped returns its input bit for bit."""
    rng = np.random.default_rng(32)
    N, d, k = 20, 16, 2
    x = W.to_numpy(_bf16(rng.standard_normal((N, d))))
    y_perm = W.to_numpy(_bf16(rng.standard_normal((5, d))))
    ros = -np.ones((N, k), np.int32)
    ros[3, 1] = 2
    w = rng.uniform(0, 1, (N, k)).astype(np.float32)
    y = oracle.combine("bf16", y_perm, ros, w, residual=x)
    keep = np.ones(N, bool)
    keep[3] = False
    assert np.array_equal(y[keep], x[keep])
    assert not np.array_equal(y[3], x[3])


def test_combine_matches_library_weighted_sum():
    rng = np.random.default_rng(33)
    N, d, k, M = 50, 24, 3, 120
    x = rng.standard_normal((N, d)).astype(np.float32)
    sh = rng.standard_normal((N, d)).astype(np.float32)
    yp = rng.standard_normal((M, d)).astype(np.float32)
    ros = rng.integers(-1, M, (N, k)).astype(np.int32)
    w = rng.uniform(0, 1, (N, k)).astype(np.float32)
    y = oracle.combine("fp32", yp, ros, w, residual=x, shared_out=sh)
    gathered = torch.from_numpy(yp).double()[torch.from_numpy(np.maximum(ros, 0)).long()]
    mask = torch.from_numpy((ros >= 0).astype(np.float64))[..., None]
    ref = (torch.from_numpy(x).double() + torch.from_numpy(sh).double()
           + (gathered * mask * torch.from_numpy(w).double()[..., None]).sum(1)).float()
    assert np.abs(y - ref.numpy()).max() <= 1e-6 * np.abs(ref.numpy()).max()


def test_dense_equivalence_small():
    """No capacity, no groups, no bias, E=4, k=2: the sparse layer equals the
    dense mixture x + sum_e g_e(x) FFN_e(x) with g the softmax over the two
    largest logits and zero elsewhere (torch, fp64, every expert on every token)."""
    torch.manual_seed(34)
    cfg = dict(name="dense", N=64, d=32, h=48, E=4, k=2, R=2, cf=0.0, G=1, kg=1,
               score="softmax_topk", act="gelu", dtype="fp32")
    x = torch.randn(64, 32)
    wr = torch.randn(4, 32) * 0.3
    w1 = torch.randn(4, 48, 32) * 0.1
    w2 = torch.randn(4, 32, 48) * 0.1
    out = oracle.forward(cfg, x.numpy(), wr.numpy(), None, None, w1.numpy(), None, w2.numpy())
    z = x.double() @ wr.double().T
    top = z.topk(2, -1)
    g = torch.zeros_like(z).scatter(1, top.indices, torch.softmax(top.values, -1))
    ref = x.double().clone()
    for e in range(4):
        ref += g[:, e:e + 1] * _torch_ffn(x, w1[e], None, w2[e], "gelu", "fp32").double()
    assert np.abs(out["y"] - ref.float().numpy()).max() < 1e-5


def test_single_expert_closed_form():
    """E = 1, k = 1, no cap: every token goes to the one expert with weight 1,
    so y = x + FFN(x)."""
    torch.manual_seed(35)
    cfg = dict(name="e1", N=33, d=64, h=64, E=1, k=1, R=1, cf=0.0, G=1, kg=1,
               score="softmax_topk", act="swiglu", dtype="bf16")
    x = torch.randn(33, 64).bfloat16()
    wr = (torch.randn(1, 64) * 0.1).bfloat16()
    w1 = (torch.randn(1, 64, 64) * 0.1).bfloat16()
    w3 = (torch.randn(1, 64, 64) * 0.1).bfloat16()
    w2 = (torch.randn(1, 64, 64) * 0.1).bfloat16()
    out = oracle.forward(cfg, W.to_numpy(x), W.to_numpy(wr), None, None,
                         W.to_numpy(w1), W.to_numpy(w3), W.to_numpy(w2))
    assert np.all(out["topk_w"] == 1.0)
    f = _torch_ffn(x, w1[0], w3[0], w2[0], "swiglu", "bf16")
    ref = (x.double() + f.double()).bfloat16()
    got = W.from_numpy_bf16(out["y"])
    assert (got.double() - ref.double()).abs().max() <= 2 ** -7 * ref.double().abs().max()


def test_forward_small_workloads_consistent():
    """Every small workload runs end to end; dropped tokens keep x bitwise;
    per-rank counts add up to the rows."""
    for name in W.ORDER:
        cfg = W.small(name)
        inp = W.make_inputs(cfg)
        x = W.to_numpy(inp["x"])
        out = oracle.forward(cfg, x, W.to_numpy(inp["w_router"]), W.to_numpy(inp["router_bias"]),
                             W.to_numpy(inp["sel_bias"]), W.to_numpy(inp["w1"]),
                             W.to_numpy(inp["w3"]), W.to_numpy(inp["w2"]),
                             shared=None if inp["shared"] is None else tuple(W.to_numpy(t[0]) if t is not None else None for t in inp["shared"]))
        assert out["rank_counts"].sum() == out["num_rows"]
        full_drop = np.all(out["row_of_slot"] < 0, axis=1)
        if full_drop.any() and inp["shared"] is None:
            assert np.array_equal(out["y"][full_drop], x[full_drop])
