"""Pins of the oracle's routing step (logits, selection, weights, counts) to
what the pages and mathematics fix.  CPU only.

Each test states the independent fact it checks; none re-types the oracle's
formula.
"""

import itertools
import os

import numpy as np
import pytest
import torch

import oracle
import moe_workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split()
                out[k] = int(v)
    return out


def _cfg(**kw):
    base = dict(name="t", N=0, d=1, h=1, E=8, k=2, R=1, cf=0.0, G=1, kg=1,
                score="softmax_topk", act="relu", dtype="fp32")
    base.update(kw)
    return base


# ------------------------------------------------------------------ the page --

def test_page_worked_example_counts():
    """The glossary snippet's printed ranges: per-expert 948..1087 (mean 1024),
    per-GPU 1968..2139 of 8192, with 8 experts on 4 GPUs (gpu = e // 2)."""
    g = _golden("glossary_routing_snippet.txt")
    cfg = W.full("toy")
    inp = W.make_inputs(cfg, weights=False)
    r = oracle.route(cfg, W.to_numpy(inp["x"]), W.to_numpy(inp["w_router"]),
                     W.to_numpy(inp["router_bias"]))
    counts = r["counts"]
    assert counts.sum() == g["total"]
    assert counts.min() == g["expert_min"] and counts.max() == g["expert_max"]
    assert counts.sum() // cfg["E"] == g["expert_mean"]
    gpu = np.bincount((r["topk_idx"] // (cfg["E"] // cfg["R"])).ravel(), minlength=cfg["R"])
    assert gpu.min() == g["gpu_min"] and gpu.max() == g["gpu_max"]
    # Per-rank counts from the dispatch layout agree with the per-GPU bincount.
    dsp = oracle.dispatch(cfg, r["topk_idx"])
    assert dsp["rank_counts"].tolist() == gpu.tolist()


def test_page_snippet_library_reduction():
    """Running the snippet itself (torch fp32 Linear + topk + bincount) gives the
    same selected sets and histograms as the oracle on the same tensors."""
    cfg = W.full("toy")
    inp = W.make_inputs(cfg, weights=False)
    with torch.no_grad():
        z = torch.nn.functional.linear(inp["x"], inp["w_router"], inp["router_bias"])
        _, ex = z.topk(cfg["k"], dim=-1)
    r = oracle.route(cfg, W.to_numpy(inp["x"]), W.to_numpy(inp["w_router"]),
                     W.to_numpy(inp["router_bias"]))
    assert np.array_equal(np.sort(ex.numpy(), 1), np.sort(r["topk_idx"], 1))
    assert torch.bincount(ex.flatten(), minlength=8).tolist() == r["counts"].tolist()


# ---------------------------------------------------------------- logits ----

def test_logit_left_to_right_fp64_order():
    """Summation order is fixed left to right in fp64: with products 2^53, 1,
    -2^53 the running sum is 2^53 (2^53+1 rounds to even), then 0; the exact
    value 1 (or any order adding 1 last) would differ.  Bias is added after."""
    cfg = _cfg(N=1, d=3, E=1, k=1)
    x = np.array([[2.0 ** 26, 1.0, -(2.0 ** 26)]], np.float32)
    w = np.array([[2.0 ** 27, 1.0, 2.0 ** 27]], np.float32)
    assert oracle.logits(cfg, x, w)[0, 0] == 0.0
    assert oracle.logits(cfg, x, w, np.array([0.5], np.float32))[0, 0] == 0.5
    # Reversed hidden order puts the 1 first: 1 - 2^53 is exact, then + 2^53 = 1.
    assert oracle.logits(cfg, x[:, ::-1].copy(), w[:, ::-1].copy())[0, 0] == 1.0


def test_logits_match_fp64_library_matmul():
    """Against torch's fp64 matmul (another summation order) the fp32-rounded
    logits agree to within one fp32 ulp, and are equal almost always."""
    rng = np.random.default_rng(1)
    N, d, E = 300, 384, 16
    x = rng.standard_normal((N, d)).astype(np.float32)
    w = (rng.uniform(-1, 1, (E, d)) / np.sqrt(d)).astype(np.float32)
    b = rng.uniform(-0.1, 0.1, E).astype(np.float32)
    z = oracle.logits(_cfg(N=N, d=d, E=E), x, w, b)
    ref = (torch.from_numpy(x).double() @ torch.from_numpy(w).double().T
           + torch.from_numpy(b).double()).float().numpy()
    ulp = np.spacing(np.abs(ref).astype(np.float32))
    assert np.all(np.abs(z - ref) <= ulp)
    assert (z == ref).mean() > 0.99


def test_logits_bf16_inputs_are_decoded_exactly():
    """bf16 bit patterns decode to the fp32 value with the same top 16 bits."""
    rng = np.random.default_rng(2)
    N, d, E = 50, 64, 4
    xt = torch.from_numpy(rng.standard_normal((N, d)).astype(np.float32)).bfloat16()
    wt = torch.from_numpy(rng.standard_normal((E, d)).astype(np.float32) / 8).bfloat16()
    z = oracle.logits(_cfg(N=N, d=d, E=E, dtype="bf16"), W.to_numpy(xt), W.to_numpy(wt))
    ref = (xt.double() @ wt.double().T).float().numpy()
    assert np.all(np.abs(z - ref) <= np.spacing(np.abs(ref).astype(np.float32)))


# ------------------------------------------------------------- selection ----

def test_tie_free_selection_equals_torch_topk():
    """With continuous random scores (no ties) the chosen experts, in order,
    equal torch.topk's."""
    rng = np.random.default_rng(3)
    for E, k in [(8, 1), (8, 2), (64, 1), (128, 2), (256, 8)]:
        z = rng.standard_normal((200, E)).astype(np.float32)
        r = oracle.select(_cfg(E=E, k=k), z)
        ref = torch.from_numpy(z).topk(k, dim=-1).indices.numpy()
        assert np.array_equal(r["topk_idx"], ref), (E, k)


def _dominant_subset(scores, items, size):
    """All size-subsets S of items such that every member is ranked before every
    non-member under (score desc, index asc); returns the list of such S."""
    out = []
    for S in itertools.combinations(items, size):
        rest = [i for i in items if i not in S]
        ok = all(scores[a] > scores[b] or (scores[a] == scores[b] and a < b)
                 for a in S for b in rest)
        if ok:
            out.append(S)
    return out


@pytest.mark.parametrize("score", ["softmax_topk", "sigmoid_norm"])
def test_brute_force_selection_with_ties(score):
    """Tiny inputs with integer-valued logits and biases (so ties abound):
    enumerate every k-subset (and every kg-subset of groups); exactly one is
    dominant, and it is the oracle's choice, in (score desc, index asc) order."""
    rng = np.random.default_rng(4)
    for trial in range(60):
        E = int(rng.choice([2, 4, 6, 8]))
        G = int(rng.choice([g for g in (1, 2, 4) if E % g == 0]))
        kg = int(rng.integers(1, G + 1))
        per = E // G
        k = int(rng.integers(1, min(3, kg * per) + 1))
        N = int(rng.integers(1, 65))
        z = rng.integers(-2, 3, (N, E)).astype(np.float32)
        bias = rng.integers(-1, 2, E).astype(np.float32) if trial % 2 else None
        cfg = _cfg(N=N, E=E, k=k, G=G, kg=kg, score=score)
        r = oracle.select(cfg, z, bias)
        for t in range(N):
            a = 1.0 / (1.0 + np.exp(-z[t].astype(np.float64))) if score == "sigmoid_norm" else z[t]
            s = a.astype(np.float32) + (bias if bias is not None else 0)
            s = {e: float(s[e]) for e in range(E)}
            eligible = list(range(E))
            if G > 1:
                gs = {g: max(s[e] for e in range(g * per, (g + 1) * per)) for g in range(G)}
                keep = _dominant_subset(gs, list(range(G)), kg)
                assert len(keep) == 1
                eligible = [e for e in range(E) if e // per in keep[0]]
            sel = _dominant_subset(s, eligible, k)
            assert len(sel) == 1
            expect = sorted(sel[0], key=lambda e: (-s[e], e))
            assert r["topk_idx"][t].tolist() == expect, (trial, t)


def test_counts_sum_to_n_times_k():
    rng = np.random.default_rng(5)
    for E, k in [(8, 2), (64, 1), (256, 8)]:
        z = rng.standard_normal((333, E)).astype(np.float32)
        r = oracle.select(_cfg(E=E, k=k), z)
        assert r["counts"].sum() == 333 * k
        assert np.array_equal(r["counts"], np.bincount(r["topk_idx"].ravel(), minlength=E))


def test_selected_experts_are_distinct():
    rng = np.random.default_rng(6)
    z = rng.integers(-1, 2, (500, 16)).astype(np.float32)  # heavy ties
    r = oracle.select(_cfg(E=16, k=5), z)
    for row in r["topk_idx"]:
        assert len(set(row.tolist())) == 5


# --------------------------------------------------------------- weights ----

def test_softmax_topk_weights_library_reduction():
    """Softmax over the k selected logits: equals torch.softmax in fp64 over the
    selected set, and sums to 1."""
    rng = np.random.default_rng(7)
    z = rng.standard_normal((400, 8)).astype(np.float32) * 2
    r = oracle.select(_cfg(E=8, k=2), z)
    zs = np.take_along_axis(z, r["topk_idx"], 1)
    ref = torch.softmax(torch.from_numpy(zs).double(), -1).numpy()
    assert np.abs(r["topk_w"] - ref).max() < 1e-7
    assert np.abs(r["topk_w"].astype(np.float64).sum(1) - 1).max() < 1e-6


def test_softmax_all_top1_weight_is_max_probability():
    """Top-1 with softmax over all experts: the weight is the largest softmax
    probability of the token (torch.softmax in fp64)."""
    rng = np.random.default_rng(8)
    z = rng.standard_normal((400, 64)).astype(np.float32)
    r = oracle.select(_cfg(E=64, k=1, score="softmax_all"), z)
    p = torch.softmax(torch.from_numpy(z).double(), -1)
    assert np.abs(r["topk_w"][:, 0] - p.max(-1).values.numpy()).max() < 1e-7
    assert np.array_equal(r["topk_idx"][:, 0], p.argmax(-1).numpy())


def test_sigmoid_norm_weights_sum_to_one_and_follow_logistic():
    rng = np.random.default_rng(9)
    z = rng.standard_normal((300, 256)).astype(np.float32)
    cfg = _cfg(E=256, k=8, G=8, kg=4, score="sigmoid_norm")
    r = oracle.select(cfg, z)
    assert np.abs(r["topk_w"].astype(np.float64).sum(1) - 1).max() < 1e-6
    a = torch.sigmoid(torch.from_numpy(z).double()).numpy()
    assert np.abs(r["affinity"] - a).max() < 1e-7
    sel = np.take_along_axis(a, r["topk_idx"], 1)
    assert np.abs(r["topk_w"] - sel / sel.sum(1, keepdims=True)).max() < 1e-6
    # Group limit: the chosen experts lie in at most kg groups.
    for row in r["topk_idx"]:
        assert len(set((row // 32).tolist())) <= 4


@pytest.mark.parametrize("score", ["softmax_topk", "softmax_all", "sigmoid_norm"])
def test_bias_changes_selection_not_weights(score):
    """The per-expert bias only affects which experts are chosen: tokens whose
    selection does not change keep bitwise-equal weights, and some selections
    do change."""
    rng = np.random.default_rng(10)
    E, k = 64, (1 if score == "softmax_all" else 4)
    z = rng.standard_normal((1000, E)).astype(np.float32)
    scale = 0.01 if score == "sigmoid_norm" else 0.3
    bias = (rng.standard_normal(E) * scale).astype(np.float32)
    G, kg = (8, 4) if score == "sigmoid_norm" else (1, 1)
    cfg = _cfg(E=E, k=k, G=G, kg=kg, score=score)
    a = oracle.select(cfg, z)
    b = oracle.select(cfg, z, bias)
    same = np.all(a["topk_idx"] == b["topk_idx"], axis=1)
    assert same.any() and (~same).any()
    assert np.array_equal(a["topk_w"][same].view(np.uint32), b["topk_w"][same].view(np.uint32))
    assert np.array_equal(a["affinity"], b["affinity"])


def test_bias_can_force_every_token_to_one_expert():
    """A huge bias on one expert puts every token on it (all-to-one load)."""
    rng = np.random.default_rng(11)
    z = rng.standard_normal((257, 16)).astype(np.float32)
    bias = np.zeros(16, np.float32)
    bias[5] = 1e6
    r = oracle.select(_cfg(E=16, k=2), z, bias)
    assert np.all(r["topk_idx"][:, 0] == 5)
    assert r["counts"][5] == 257
