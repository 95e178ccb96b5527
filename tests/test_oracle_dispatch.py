"""Pins of the oracle's dispatch step (capacity, token-order and first-choice-
first admission, expert/rank-contiguous layout, permute) and the selection-bias
update.  CPU only.
"""

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle


def _cfg(**kw):
    base = dict(name="t", N=0, d=4, h=4, E=8, k=2, R=1, cf=0.0, G=1, kg=1,
                score="softmax_topk", act="relu", dtype="fp32")
    base.update(kw)
    return base


def _random_topk(rng, N, E, k, skew=0.0):
    """k distinct experts per token, optionally skewed toward low indices."""
    p = np.arange(1, E + 1, dtype=np.float64) ** (-skew)
    p /= p.sum()
    out = np.empty((N, k), np.int32)
    for t in range(N):
        out[t] = rng.choice(E, size=k, replace=False, p=p)
    return out


def _check_invariants(cfg, idx, dsp, admission="token"):
    N, k, E, R = idx.shape[0], cfg["k"], cfg["E"], cfg["R"]
    cap = oracle.capacity(cfg)
    counts = np.bincount(idx.ravel(), minlength=E)
    adm = dsp["admitted"]
    assert np.array_equal(adm, np.minimum(counts, cap))
    M = dsp["num_rows"]
    ros = dsp["row_of_slot"]
    dropped = (ros < 0).sum()
    assert adm.sum() == N * k - dropped == M
    off = dsp["expert_offsets"]
    assert off[0] == 0 and np.array_equal(np.diff(off), adm)
    # Bijection: admitted slots <-> rows [0, M)
    t_idx, j_idx = np.nonzero(ros >= 0)
    rows = ros[t_idx, j_idx]
    assert np.array_equal(np.sort(rows), np.arange(M))
    assert np.array_equal(dsp["token_of_row"][rows], t_idx)
    assert np.array_equal(dsp["slot_of_row"][rows], j_idx)
    # Each row sits in its expert's segment; inside a segment tokens increase
    # (token order) or (slot, token) pairs increase (first choice first).
    e_of_row = np.repeat(np.arange(E), adm)
    assert np.array_equal(idx[t_idx, j_idx], e_of_row[rows])
    tor = dsp["token_of_row"][:M].astype(np.int64)
    sor = dsp["slot_of_row"][:M].astype(np.int64)
    key = tor if admission == "token" else sor * (N + 1) + tor
    for e in range(E):
        seg = key[off[e]:off[e + 1]]
        assert np.all(np.diff(seg) > 0)
    # Ranks: blocks of E/R experts, counts are sums over the block.
    per = E // R
    assert np.array_equal(dsp["rank_counts"], adm.reshape(R, per).sum(1))
    assert np.array_equal(dsp["rank_offsets"], off[::per])
    return counts


def test_no_capacity_equals_stable_argsort():
    """Without a capacity limit the rows are the flattened (token, slot) list
    stably sorted by expert: numpy.argsort(kind='stable')."""
    rng = np.random.default_rng(20)
    for N, E, k in [(1000, 8, 2), (777, 64, 1), (300, 256, 8)]:
        idx = _random_topk(rng, N, E, k)
        dsp = oracle.dispatch(_cfg(N=N, E=E, k=k, R=E // 4 if E >= 4 else 1), idx)
        order = np.argsort(idx.ravel(), kind="stable")
        assert np.array_equal(dsp["token_of_row"], order // k)
        assert np.array_equal(dsp["slot_of_row"], (order % k).astype(np.int8))
        assert dsp["num_rows"] == N * k


def test_capacity_fifo_brute_force():
    """Capacity admission equals an explicit per-expert FIFO filled in token
    order that turns away arrivals once it holds `cap` entries."""
    rng = np.random.default_rng(21)
    for trial in range(40):
        E = int(rng.choice([2, 4, 8, 16]))
        k = int(rng.integers(1, min(3, E) + 1))
        N = int(rng.integers(1, 200))
        cf = float(rng.choice([0.25, 0.5, 1.0, 1.25, 2.0]))
        idx = _random_topk(rng, N, E, k, skew=float(rng.choice([0.0, 1.5])))
        cfg = _cfg(N=N, E=E, k=k, cf=cf)
        dsp = oracle.dispatch(cfg, idx)
        cap = int(np.ceil(np.float64(np.float32(cf)) * N * k / E))
        assert oracle.capacity(cfg) == cap
        queues = {e: [] for e in range(E)}
        for t in range(N):
            for j in range(k):
                e = idx[t, j]
                if len(queues[e]) < cap:
                    queues[e].append((t, j))
        expect_rows = [ts for e in range(E) for ts in queues[e]]
        M = dsp["num_rows"]
        assert M == len(expect_rows)
        got = list(zip(dsp["token_of_row"][:M].tolist(), dsp["slot_of_row"][:M].tolist()))
        assert got == expect_rows
        _check_invariants(cfg, idx, dsp)


def test_capacity_one_admits_first_token_per_expert():
    rng = np.random.default_rng(22)
    N, E, k = 64, 8, 2
    idx = _random_topk(rng, N, E, k)
    cfg = _cfg(N=N, E=E, k=k, cf=E / (N * k))  # cap = ceil(1) = 1
    assert oracle.capacity(cfg) == 1
    dsp = oracle.dispatch(cfg, idx)
    for e in range(E):
        first = np.argwhere(idx == e)
        if len(first):
            t, j = first[0]
            assert dsp["row_of_slot"][t, j] == dsp["expert_offsets"][e]
    assert np.array_equal(dsp["admitted"], (np.bincount(idx.ravel(), minlength=E) > 0).astype(int))


def test_uniform_routing_no_drops_at_cf_one():
    """Forced round-robin routing gives every expert exactly N*k/E slots, so a
    capacity factor of 1 drops nothing."""
    N, E, k = 512, 16, 2
    idx = np.stack([(np.arange(N) * k + j) % E for j in range(k)], 1).astype(np.int32)
    cfg = _cfg(N=N, E=E, k=k, cf=1.0, R=4)
    dsp = oracle.dispatch(cfg, idx)
    assert np.all(dsp["admitted"] == N * k // E)
    assert np.all(dsp["row_of_slot"] >= 0)


def test_tiny_capacity_drops_nearly_everything():
    rng = np.random.default_rng(23)
    N, E, k = 1000, 8, 2
    idx = _random_topk(rng, N, E, k)
    cfg = _cfg(N=N, E=E, k=k, cf=1e-6)
    dsp = oracle.dispatch(cfg, idx)
    assert dsp["num_rows"] == E  # cap rounds up to 1
    _check_invariants(cfg, idx, dsp)


def test_empty_batch():
    cfg = _cfg(N=0, E=8, k=2, R=4, cf=1.25)
    dsp = oracle.dispatch(cfg, np.zeros((0, 2), np.int32))
    assert dsp["num_rows"] == 0
    assert np.all(dsp["expert_offsets"] == 0) and np.all(dsp["rank_counts"] == 0)


def test_out_of_range_expert_rejected():
    with pytest.raises(ValueError):
        oracle.dispatch(_cfg(N=1, E=4, k=1), np.array([[4]], np.int32))


@settings(max_examples=60, deadline=None)
@given(N=st.integers(0, 300), E_pow=st.integers(0, 8), k=st.integers(1, 8),
       R_pow=st.integers(0, 6), cf=st.sampled_from([0.0, 0.5, 1.0, 1.25, 2.0]),
       skew=st.sampled_from([0.0, 1.1, 3.0]), seed=st.integers(0, 2 ** 31 - 1))
def test_dispatch_invariants_property(N, E_pow, k, R_pow, cf, skew, seed):
    E = 2 ** E_pow
    k = min(k, E)
    R = 2 ** min(R_pow, E_pow)
    rng = np.random.default_rng(seed)
    idx = _random_topk(rng, N, E, k, skew)
    cfg = _cfg(N=N, E=E, k=k, R=R, cf=cf)
    dsp = oracle.dispatch(cfg, idx)
    _check_invariants(cfg, idx, dsp)


# ---- first choice first (GShard's top-2 router; admission = "first_choice") --


def test_first_choice_equals_token_order_for_top1():
    """With one slot per token both admission orders are the same walk."""
    rng = np.random.default_rng(30)
    for N, E, cf in [(500, 8, 1.0), (777, 64, 1.25), (64, 4, 0.25)]:
        idx = _random_topk(rng, N, E, 1, skew=1.5)
        cfg = _cfg(N=N, E=E, k=1, cf=cf, R=2)
        a, b = oracle.dispatch(cfg, idx, "token"), oracle.dispatch(cfg, idx, "first_choice")
        for key in a:
            assert np.array_equal(np.asarray(a[key]), np.asarray(b[key])), key


def _lexsort_rows(idx):
    """(t, j) of every slot, sorted by (expert, slot, token) with numpy.lexsort."""
    N, k = idx.shape
    t = np.repeat(np.arange(N), k)
    j = np.tile(np.arange(k), N)
    e = idx.ravel()
    order = np.lexsort((t, j, e))
    return e[order], t[order], j[order]


def test_first_choice_no_capacity_is_lexsort():
    """Without a capacity limit the rows are every slot sorted by (expert,
    slot, token): numpy.lexsort."""
    rng = np.random.default_rng(31)
    for N, E, k in [(1000, 8, 2), (300, 256, 8), (129, 16, 3)]:
        idx = _random_topk(rng, N, E, k, skew=1.1)
        cfg = _cfg(N=N, E=E, k=k, R=E // 4)
        dsp = oracle.dispatch(cfg, idx, "first_choice")
        _, t, j = _lexsort_rows(idx)
        assert np.array_equal(dsp["token_of_row"], t)
        assert np.array_equal(dsp["slot_of_row"], j.astype(np.int8))
        _check_invariants(cfg, idx, dsp, "first_choice")


def test_first_choice_capacity_is_lexsort_prefix():
    """With a capacity, each expert keeps the first cap entries of its
    (slot, token)-sorted list (numpy.lexsort, then a per-expert prefix)."""
    rng = np.random.default_rng(32)
    for trial in range(40):
        E = int(rng.choice([2, 4, 8, 16]))
        k = int(rng.integers(1, min(4, E) + 1))
        N = int(rng.integers(1, 300))
        cf = float(rng.choice([0.25, 0.5, 1.0, 1.25, 2.0]))
        idx = _random_topk(rng, N, E, k, skew=float(rng.choice([0.0, 1.5, 3.0])))
        cfg = _cfg(N=N, E=E, k=k, cf=cf)
        cap = oracle.capacity(cfg)
        dsp = oracle.dispatch(cfg, idx, "first_choice")
        e, t, j = _lexsort_rows(idx)
        first = np.searchsorted(e, np.arange(E))  # start of each expert's run
        keep = np.arange(e.size) - first[e] < cap
        M = dsp["num_rows"]
        assert M == int(keep.sum())
        assert np.array_equal(dsp["token_of_row"][:M], t[keep])
        assert np.array_equal(dsp["slot_of_row"][:M], j[keep].astype(np.int8))
        _check_invariants(cfg, idx, dsp, "first_choice")


def test_first_choice_priority_over_token_order():
    """No expert admits a later choice while turning away an earlier one, and
    no admission order admits more first choices."""
    rng = np.random.default_rng(33)
    for trial in range(30):
        E, k = 8, int(rng.integers(2, 5))
        N = int(rng.integers(50, 400))
        idx = _random_topk(rng, N, E, k, skew=2.0)
        cfg = _cfg(N=N, E=E, k=k, cf=float(rng.choice([0.5, 1.0])))
        fc = oracle.dispatch(cfg, idx, "first_choice")["row_of_slot"]
        to = oracle.dispatch(cfg, idx, "token")["row_of_slot"]
        for ex in range(E):
            for j in range(1, k):
                if np.any(fc[:, j][idx[:, j] == ex] >= 0):
                    for jj in range(j):
                        assert np.all(fc[:, jj][idx[:, jj] == ex] >= 0)
        assert (fc[:, 0] >= 0).sum() >= (to[:, 0] >= 0).sum()
        # the same number of rows either way: min(count, cap) per expert
        assert (fc >= 0).sum() == (to >= 0).sum()


def test_unknown_admission_rejected():
    with pytest.raises(KeyError):
        oracle.dispatch(_cfg(N=1, E=4, k=1), np.array([[0]], np.int32), "slot")


@settings(max_examples=40, deadline=None)
@given(N=st.integers(0, 300), E_pow=st.integers(0, 8), k=st.integers(1, 8),
       R_pow=st.integers(0, 6), cf=st.sampled_from([0.0, 0.5, 1.0, 1.25, 2.0]),
       skew=st.sampled_from([0.0, 1.1, 3.0]), seed=st.integers(0, 2 ** 31 - 1))
def test_first_choice_invariants_property(N, E_pow, k, R_pow, cf, skew, seed):
    E = 2 ** E_pow
    k = min(k, E)
    R = 2 ** min(R_pow, E_pow)
    rng = np.random.default_rng(seed)
    idx = _random_topk(rng, N, E, k, skew)
    cfg = _cfg(N=N, E=E, k=k, R=R, cf=cf)
    dsp = oracle.dispatch(cfg, idx, "first_choice")
    _check_invariants(cfg, idx, dsp, "first_choice")


# ---- padded layout (GShard-style fixed buffers of cap rows per expert) ----


def test_padded_layout_relocates_the_compact_rows():
    """Expert e's admitted rows move from the compact offset to row e*cap, in
    the same order; the rows after them up to (e+1)*cap are padding; offsets
    and per-rank counts become multiples of cap.  Both admission orders."""
    rng = np.random.default_rng(34)
    for trial in range(30):
        E = int(rng.choice([2, 4, 8, 16]))
        k = int(rng.integers(1, min(3, E) + 1))
        N = int(rng.integers(1, 250))
        R = int(rng.choice([r for r in (1, 2, 4) if E % r == 0]))
        cf = float(rng.choice([0.25, 0.5, 1.0, 1.25, 2.0]))
        idx = _random_topk(rng, N, E, k, skew=float(rng.choice([0.0, 1.5])))
        for adm in ("token", "first_choice"):
            cfg = _cfg(N=N, E=E, k=k, R=R, cf=cf, admission=adm)
            cap = oracle.capacity(cfg)
            com = oracle.dispatch(cfg, idx)
            pad = oracle.dispatch(dict(cfg, layout="padded"), idx)
            assert np.array_equal(pad["admitted"], com["admitted"])
            assert np.array_equal(pad["expert_offsets"], np.arange(E + 1) * cap)
            assert np.array_equal(pad["rank_counts"], np.full(R, E // R * cap))
            assert pad["num_rows"] == E * cap
            ros_c, ros_p = com["row_of_slot"], pad["row_of_slot"]
            assert np.array_equal(ros_c < 0, ros_p < 0)
            e_of = idx[ros_c >= 0]
            off = com["expert_offsets"]
            assert np.array_equal(ros_p[ros_c >= 0], e_of * cap + ros_c[ros_c >= 0] - off[e_of])
            for e in range(E):
                a = com["admitted"][e]
                seg = slice(e * cap, e * cap + a)
                assert np.array_equal(pad["token_of_row"][seg], com["token_of_row"][off[e]:off[e] + a])
                assert np.array_equal(pad["slot_of_row"][seg], com["slot_of_row"][off[e]:off[e] + a])
                assert np.all(pad["token_of_row"][e * cap + a:(e + 1) * cap] == -1)
                assert np.all(pad["slot_of_row"][e * cap + a:(e + 1) * cap] == -1)


def test_padded_layout_needs_a_capacity():
    with pytest.raises(ValueError):
        oracle.dispatch(_cfg(N=8, E=4, k=1, cf=0.0, layout="padded"),
                        np.zeros((8, 1), np.int32))


def test_padding_rows_permute_to_zero():
    x = np.arange(4 * 8, dtype=np.float32).reshape(4, 8) + 1
    tor = np.array([2, -1, 0, -1, 3], np.int32)
    out = oracle.permute("fp32", x, tor, 5)
    assert np.array_equal(out[[0, 2, 4]], x[[2, 0, 3]])
    assert np.all(out[[1, 3]] == 0)


def test_padded_layer_output_equals_compact():
    """Each FFN row depends on its input row only and padding rows are zero,
    so the padded layout changes no output bit (Switch and Zipf, small)."""
    import moe_workloads as W
    for name, cf in (("switch", None), ("zipf", 1.0)):
        cfg = W.small(name) if cf is None else W.with_(W.small(name), cf=cf)
        inp = W.make_inputs(cfg)
        n = W.to_numpy
        args = (n(inp["x"]), n(inp["w_router"]), n(inp["router_bias"]), n(inp["sel_bias"]),
                n(inp["w1"]), n(inp["w3"]), n(inp["w2"]))
        com = oracle.forward(cfg, *args)
        pad = oracle.forward(dict(cfg, layout="padded"), *args)
        assert np.array_equal(com["y"], pad["y"]), name
        live = pad["token_of_row"][:pad["num_rows"]] >= 0
        assert np.all(pad["y_perm"][~live] == 0)


def test_permute_is_bitwise_row_copy():
    rng = np.random.default_rng(24)
    N, d, E, k = 100, 32, 4, 2
    idx = _random_topk(rng, N, E, k)
    dsp = oracle.dispatch(_cfg(N=N, E=E, k=k, d=d), idx)
    x = rng.integers(0, 65535, (N, d)).astype(np.uint16)  # arbitrary bit patterns
    xp = oracle.permute("bf16", x, dsp["token_of_row"], dsp["num_rows"])
    assert np.array_equal(xp, x[dsp["token_of_row"][:dsp["num_rows"]]])


# ----------------------------------------------------------- bias update ----

def test_bias_update_closed_form():
    """Mean load N*k/E = 4: load 5 lowers the bias by the step, 3 raises it,
    4 leaves it bitwise unchanged."""
    counts = np.array([5, 3, 4, 4, 0, 8], np.int32)  # N*k = 24, E = 6
    b0 = np.array([0.0, 0.0, 0.25, -1.5, 1.0, 1e-3], np.float32)
    b = oracle.bias_update(12, 2, counts, b0, 1e-3)
    step = np.float32(1e-3)
    expect = np.array([b0[0] - step, b0[1] + step, b0[2], b0[3], b0[4] + step, b0[5] - step],
                      np.float32)
    assert np.array_equal(b.view(np.uint32), expect.view(np.uint32))
    assert b[5] == 0.0


def test_bias_update_non_integer_mean():
    """Mean 7/3 is not an integer: loads 2 and 3 fall strictly below/above."""
    counts = np.array([2, 3, 2], np.int32)  # N*k = 7
    b = oracle.bias_update(7, 1, counts, np.zeros(3, np.float32), 0.5)
    assert b.tolist() == [0.5, -0.5, 0.5]
