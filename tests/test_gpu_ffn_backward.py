"""GPU parity of the expert-FFN backward (moe_expert_ffn_backward) against the
oracle: input gradients and fp32 weight gradients within the bf16 layer
tolerance (max |gpu - ref| / max |ref| per tensor), on

- seeded ragged segments (an empty expert, a segment of one row, rows after
  the last segment that must stay untouched) at the reduced shapes of every
  activation, including an h that is not a multiple of the 128-column tile;
- the layer's backward chained through the data path (combine backward ->
  FFN backward -> permute backward) on the oracle forward's own layout;
- the full Switch shape (16384 rows, d 1024, h 4096, 64 experts), sampled:
  input gradients of rows across the batch and both weight gradients of one
  whole expert, each from the oracle's per-row backward.
"""

import numpy as np
import pytest
import torch

import expert_token_routing_router_amd as moe
import moe_workloads as W
import oracle

from gpu_util import TOL, as_tensor, n, oracle_reference, rel_err, threads

pytestmark = pytest.mark.gpu

BF16 = torch.bfloat16
SHAPES = {
    # name: (workload for d, h, act; experts; rows)
    "switch-small-gelu": (W.small("switch"), 16, 700),
    "mixtral-small-swiglu": (W.small("mixtral"), 8, 611),       # h 448: a 64-column tail
    "deepseek-small-swiglu": (W.small("deepseek"), 24, 523),    # h 192, d 384
    "toy-small-relu": (W.with_(W.small("toy"), dtype="bf16"), 8, 300),
}


def _segments(E, rows, seed):
    """Ragged, monotone offsets over the first rows - 37 rows: expert 1 empty,
    expert 2 a single row; the last 37 rows lie outside every segment."""
    g = np.random.default_rng(seed)
    used = rows - 37
    cuts = np.sort(g.integers(0, used + 1, size=E - 1))
    off = np.concatenate([[0], cuts, [used]]).astype(np.int32)
    off[2] = off[1]
    off[3] = min(off[2] + 1, off[4]) if E > 3 else off[3]
    return off


def _weights(E, d, h, act, seed, scale=0.05):
    g = torch.Generator().manual_seed(seed)
    w1 = (torch.randn(E, h, d, generator=g) * scale).to(BF16)
    w3 = (torch.randn(E, h, d, generator=g) * scale).to(BF16) if act == "swiglu" else None
    w2 = (torch.randn(E, d, h, generator=g) * scale).to(BF16)
    return w1, w3, w2


def _backward_call(path, E, rows, d, h, act, x, off, group_rows, w1, w3, w2, dy, dx, dw1, dw3,
                   dw2):
    """One FFN backward on device tensors: ``plain`` (moe_expert_ffn_backward,
    row-major weights) or ``packed`` (moe_expert_ffn_backward_packed on the
    forward's grouped GEMM, weights from prepare_backward_weights)."""
    if path == "plain":
        ws = moe.workspace(moe.moe_expert_ffn_backward_workspace_size(E, rows, d, h, act, "bf16"))
        moe.moe_expert_ffn_backward(E, rows, d, h, act, "bf16", x, off, group_rows, w1, w3, w2,
                                    dy, dx, dw1, dw3, dw2, ws)
    else:
        pw = moe.prepare_backward_weights({"dtype": "bf16", "d": d, "h": h},
                                          {"w1": w1, "w3": w3, "w2": w2})
        ws = moe.workspace(moe.moe_expert_ffn_backward_packed_workspace_size(E, rows, d, h, act,
                                                                              "bf16"))
        moe.moe_expert_ffn_backward_packed(E, rows, d, h, act, "bf16", x, off, group_rows,
                                           pw["w1"], pw["w3"], pw["w2t"], pw["w13t"], dy, dx,
                                           dw1, dw3, dw2, ws)


def _gpu_backward(E, rows, d, h, act, x, off, w1, w3, w2, dy, sentinel=3.0, path="plain"):
    dev = lambda t: None if t is None else t.cuda()  # noqa: E731
    sw = act == "swiglu"
    dx = torch.full((max(rows, 1), d), sentinel, dtype=BF16, device="cuda")
    dw1 = torch.full((E, h, d), 9.0, device="cuda")
    dw3 = torch.full((E, h, d), 9.0, device="cuda") if sw else None
    dw2 = torch.full((E, d, h), 9.0, device="cuda")
    _backward_call(path, E, rows, d, h, act, dev(x), dev(off), None, dev(w1), dev(w3), dev(w2),
                   dev(dy), dx, dw1, dw3, dw2)
    torch.cuda.synchronize()
    return dx.cpu(), dw1.cpu(), None if dw3 is None else dw3.cpu(), dw2.cpu()


PATHS = ["plain", "packed"]


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("name", list(SHAPES))
def test_ffn_backward_ragged_segments(name, path):
    cfg, E, rows = SHAPES[name]
    d, h, act = cfg["d"], cfg["h"], cfg["act"]
    print(f"[ffn backward {name} {path}] E={E} rows={rows} d={d} h={h} {act}", flush=True)
    off = _segments(E, rows, seed=rows)
    g = torch.Generator().manual_seed(d + h)
    x = torch.randn(rows, d, generator=g).to(BF16)
    dy = (torch.randn(rows, d, generator=g) * 0.5).to(BF16)
    w1, w3, w2 = _weights(E, d, h, act, seed=E + d)
    dx, dw1, dw3, dw2 = _gpu_backward(E, rows, d, h, act, x, torch.from_numpy(off), w1, w3, w2,
                                      dy, path=path)
    oracle.set_threads(threads())
    r_dx, r_dw1, r_dw3, r_dw2 = oracle.expert_ffn_backward("bf16", act, n(x), off, n(w1), n(w3),
                                                           n(w2), n(dy))
    used = int(off[-1])
    err = rel_err(dx[:used].float(), as_tensor(r_dx[:used], "bf16").float())
    assert err <= TOL["bf16"], f"dx max rel err {err:.3e}"
    assert bool((dx[used:] == 3.0).all()), "rows outside every segment must stay untouched"
    for got, ref, key in ((dw1, r_dw1, "dw1"), (dw3, r_dw3, "dw3"), (dw2, r_dw2, "dw2")):
        if ref is None:
            continue
        err = rel_err(got, torch.from_numpy(ref))
        assert err <= TOL["bf16"], f"{key} max rel err {err:.3e}"
        assert bool((got[1] == 0).all()), f"{key}: an expert with no rows gets zeros"


@pytest.mark.parametrize("name", ["switch", "mixtral"])
def test_layer_backward_chain(name):
    """combine backward -> FFN backward -> permute backward on the oracle
    forward's layout, expert outputs and weights (compact layout, drops
    included), against the same chain of oracle calls."""
    cfg = W.small(name)
    dt, act = cfg["dtype"], cfg["act"]
    N, d, h, E, k = cfg["N"], cfg["d"], cfg["h"], cfg["E"], cfg["k"]
    print(f"[layer backward {name}] N={N} d={d} h={h} E={E} k={k}", flush=True)
    inp_cpu = W.make_inputs(cfg)
    ref = oracle_reference(cfg, inp_cpu)
    M = ref["num_rows"]
    buf = moe.MoeBuffers(cfg)
    rows = buf.rows
    g = torch.Generator().manual_seed(N)
    dy = torch.randn(N, d, generator=g).to(BF16)

    def padded(a):
        t = torch.zeros(max(rows, 1), d, dtype=BF16)
        t[:M] = as_tensor(a[:M], dt)
        return t.cuda()

    x_perm, y_perm = padded(ref["x_perm"]), padded(ref["y_perm"])
    ros = torch.from_numpy(ref["row_of_slot"]).cuda()
    tw = torch.from_numpy(ref["topk_w"]).cuda()
    off = torch.from_numpy(ref["expert_offsets"]).cuda()
    dy_perm = torch.zeros(max(rows, 1), d, dtype=BF16, device="cuda")
    dtw = torch.empty(N, k, device="cuda")
    moe.moe_combine_backward(buf.desc, dy.cuda(), y_perm, ros, tw, dy_perm, dtw, num_rows=rows)
    w1, w3, w2 = inp_cpu["w1"], inp_cpu["w3"], inp_cpu["w2"]
    dev = lambda t: None if t is None else t.cuda()  # noqa: E731
    dx_perm = torch.zeros(max(rows, 1), d, dtype=BF16, device="cuda")
    dw1 = torch.empty(E, h, d, device="cuda")
    dw3 = torch.empty(E, h, d, device="cuda") if act == "swiglu" else None
    dw2 = torch.empty(E, d, h, device="cuda")
    ws = moe.workspace(moe.moe_expert_ffn_backward_workspace_size(E, rows, d, h, act, dt))
    moe.moe_expert_ffn_backward(E, rows, d, h, act, dt, x_perm, off, None, dev(w1), dev(w3),
                                dev(w2), dy_perm, dx_perm, dw1, dw3, dw2, ws)
    dx = torch.empty(N, d, dtype=BF16, device="cuda")
    moe.moe_permute_backward(buf.desc, dx_perm, ros, dx, num_rows=rows)
    torch.cuda.synchronize()

    oracle.set_threads(threads())
    r_dyp, r_dtw = oracle.combine_backward(dt, n(dy), ref["y_perm"][:M], ref["row_of_slot"],
                                           ref["topk_w"], M)
    r_dxp, r_dw1, r_dw3, r_dw2 = oracle.expert_ffn_backward(
        dt, act, ref["x_perm"][:M], ref["expert_offsets"], n(w1), n(w3), n(w2), r_dyp)
    r_dx = oracle.permute_backward(dt, r_dxp, ref["row_of_slot"])
    assert rel_err(dtw.cpu(), torch.from_numpy(r_dtw)) <= 1e-5
    err = rel_err(dx.cpu().float(), as_tensor(r_dx, dt).float())
    assert err <= TOL[dt], f"dx max rel err {err:.3e}"
    for got, r, key in ((dw1, r_dw1, "dw1"), (dw3, r_dw3, "dw3"), (dw2, r_dw2, "dw2")):
        if r is None:
            continue
        err = rel_err(got.cpu(), torch.from_numpy(r))
        assert err <= TOL[dt], f"{key} max rel err {err:.3e}"


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("name,kw", [("zipf", dict(cf=1.0)), ("switch", {})])
def test_ffn_backward_padded_layout_equals_compact(name, kw, path):
    """The layer's backward on the capacity-padded layout, with NaN planted in
    every padding row of x_perm and dy_perm (rows no call is obliged to write):
    with group_rows = admitted the FFN backward leaves them out, so the weight
    gradients and every admitted row's dx equal the compact layout's bit for
    bit (each expert's rows, and their order, are the same in both layouts)."""
    cfg = W.with_(W.small(name), **kw)
    print(f"[ffn backward padded vs compact] {name} {kw} {path}", flush=True)
    dev = lambda t: None if t is None else t.cuda()  # noqa: E731
    inp_cpu = W.make_inputs(cfg)
    inp = moe.prepare_weights(cfg, {k: (dev(v) if isinstance(v, torch.Tensor) else v)
                                    for k, v in inp_cpu.items() if k != "shared"})
    N, d, h, E, act = cfg["N"], cfg["d"], cfg["h"], cfg["E"], cfg["act"]
    sw = act == "swiglu"
    g = torch.Generator().manual_seed(11)
    dy = torch.randn(N, d, generator=g).to(BF16).cuda()
    out = {}
    for layout in ("compact", "padded"):
        c = W.with_(cfg, layout=layout)
        buf = moe.MoeBuffers(c)
        moe.moe_forward(buf, inp)
        rows = buf.rows
        dy_perm = torch.full((rows, d), float("nan"), dtype=BF16, device="cuda")
        if layout == "padded":
            pad = buf.token_of_row[:rows] < 0
            buf.x_perm[:rows][pad] = float("nan")
        moe.moe_combine_backward(buf.desc, dy, buf.y_perm, buf.row_of_slot, buf.topk_w, dy_perm,
                                 torch.empty(N, cfg["k"], device="cuda"), num_rows=rows)
        dx_perm = torch.full((rows, d), 5.0, dtype=BF16, device="cuda")
        dw1 = torch.empty(E, h, d, device="cuda")
        dw3 = torch.empty(E, h, d, device="cuda") if sw else None
        dw2 = torch.empty(E, d, h, device="cuda")
        _backward_call(path, E, rows, d, h, act, buf.x_perm, buf.expert_offsets,
                       buf.admitted if layout == "padded" else None, inp_cpu["w1"].cuda(),
                       dev(inp_cpu["w3"]), inp_cpu["w2"].cuda(), dy_perm, dx_perm, dw1, dw3,
                       dw2)
        dx = torch.empty(N, d, dtype=BF16, device="cuda")
        moe.moe_permute_backward(buf.desc, dx_perm, buf.row_of_slot, dx, num_rows=rows)
        torch.cuda.synchronize()
        out[layout] = (dx.cpu(), dw1.cpu(), None if dw3 is None else dw3.cpu(), dw2.cpu(),
                       int(buf.admitted.sum()))
    (cdx, c1, c3, c2, cm), (pdx, p1, p3, p2, pm) = out["compact"], out["padded"]
    assert cm == pm  # same admitted rows in both layouts
    for a, b, key in ((c1, p1, "dw1"), (c3, p3, "dw3"), (c2, p2, "dw2")):
        if a is None:
            continue
        assert bool(torch.isfinite(b).all()), f"{key}: padding rows leaked into the gradient"
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), f"{key} differs"
    assert torch.equal(cdx.view(torch.int16), pdx.view(torch.int16))


@pytest.mark.parametrize("path", PATHS)
def test_ffn_backward_full_switch_sampled(path):
    """The full Switch shape in the launch configuration the benchmark's
    backward pass uses: input gradients of 8 rows spread over the batch, and
    dw1 / dw2 of one whole expert, from the oracle's per-row backward."""
    cfg = W.full("switch")
    N, d, h, E, act = cfg["N"], cfg["d"], cfg["h"], cfg["E"], cfg["act"]
    print(f"[ffn backward full switch {path}] rows={N} d={d} h={h} E={E}", flush=True)
    inp = W.make_inputs(cfg)
    x, w1, w2 = inp["x"], inp["w1"], inp["w2"]
    g = torch.Generator().manual_seed(7)
    dy = (torch.randn(N, d, generator=g) * 0.5).to(BF16)
    counts = np.bincount(np.random.default_rng(3).integers(0, E, N), minlength=E)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    dx, dw1, _, dw2 = _gpu_backward(E, N, d, h, act, x, torch.from_numpy(off), w1, None, w2, dy,
                                    path=path)
    xn, dyn, w1n, w2n = n(x), n(dy), n(w1), n(w2)
    expert_of = np.searchsorted(off, np.arange(N), side="right") - 1
    for r in np.linspace(0, N - 1, 8).astype(int):
        e = expert_of[r]
        r_dx, _, _, _ = oracle.ffn_backward_row("bf16", act, xn[r], w1n[e], None, w2n[e], dyn[r])
        err = rel_err(dx[r].float(), as_tensor(r_dx, "bf16").float())
        assert err <= TOL["bf16"], f"dx row {r} max rel err {err:.3e}"
    e = 5
    lo, hi = int(off[e]), int(off[e + 1])
    Hs, dus = [], []
    for r in range(lo, hi):
        _, H, du, _ = oracle.ffn_backward_row("bf16", act, xn[r], w1n[e], None, w2n[e], dyn[r])
        Hs.append(H)
        dus.append(du)
    xe = as_tensor(xn[lo:hi], "bf16").double().numpy()
    dye = as_tensor(dyn[lo:hi], "bf16").double().numpy()
    r_dw1 = np.array(dus).T @ xe      # sum over the expert's rows of du x^T
    r_dw2 = dye.T @ np.array(Hs)      # sum over the expert's rows of dy H^T
    err = rel_err(dw1[e], torch.from_numpy(r_dw1))
    assert err <= TOL["bf16"], f"dw1[{e}] max rel err {err:.3e}"
    err = rel_err(dw2[e], torch.from_numpy(r_dw2))
    assert err <= TOL["bf16"], f"dw2[{e}] max rel err {err:.3e}"


# The packed backward on 192-row tiles: h = 2048 takes the wide recompute and
# g GEMMs (256 columns per tile; SwiGLU 256 of W1 and of W3), d = 1024 the
# 256-column dx GEMM; experts on the fragment edges of a 192-row tile, one
# past it (split in two), 37 rows outside every segment.
WIDE_COUNTS = [0, 1, 31, 32, 33, 63, 64, 65, 96, 127, 128, 129, 160, 191, 192, 193]


@pytest.mark.parametrize("act", ["swiglu", "gelu"])
def test_ffn_backward_packed_wide_tiles(act):
    E, d, h = len(WIDE_COUNTS), 1024, 2048
    used = sum(WIDE_COUNTS)
    rows = used + 37
    assert 32 * E < rows <= 128 * E, "must take the 192-row tiles"
    print(f"[ffn backward packed wide] E={E} rows={rows} d={d} h={h} {act}", flush=True)
    off = np.concatenate([[0], np.cumsum(WIDE_COUNTS)]).astype(np.int32)
    g = torch.Generator().manual_seed(h + E)
    x = torch.randn(rows, d, generator=g).to(BF16)
    dy = (torch.randn(rows, d, generator=g) * 0.5).to(BF16)
    w1, w3, w2 = _weights(E, d, h, act, seed=d, scale=0.03)
    dx, dw1, dw3, dw2 = _gpu_backward(E, rows, d, h, act, x, torch.from_numpy(off), w1, w3, w2,
                                      dy, path="packed")
    oracle.set_threads(threads())
    r_dx, r_dw1, r_dw3, r_dw2 = oracle.expert_ffn_backward("bf16", act, n(x), off, n(w1), n(w3),
                                                           n(w2), n(dy))
    err = rel_err(dx[:used].float(), as_tensor(r_dx[:used], "bf16").float())
    assert err <= TOL["bf16"], f"dx max rel err {err:.3e}"
    assert bool((dx[used:] == 3.0).all()), "rows outside every segment must stay untouched"
    for e in range(E):
        a, b = int(off[e]), int(off[e + 1])
        if b > a:
            ee = rel_err(dx[a:b].float(), as_tensor(r_dx[a:b], "bf16").float())
            assert ee <= TOL["bf16"], f"dx of expert {e} ({b - a} rows): {ee:.3e}"
    for got, ref, key in ((dw1, r_dw1, "dw1"), (dw3, r_dw3, "dw3"), (dw2, r_dw2, "dw2")):
        if ref is None:
            continue
        err = rel_err(got, torch.from_numpy(ref))
        assert err <= TOL["bf16"], f"{key} max rel err {err:.3e}"
        assert bool((got[0] == 0).all()), f"{key}: an expert with no rows gets zeros"


# The packed backward on 320-row tiles (more than 128 rows per expert on
# average) with h = 2048: the wide recompute and the activation-gradient
# epilogue (branch-free loads and stores) at their largest tile, experts on
# the fragment edges of a 320-row tile and one past it (split in two).
TALL_COUNTS = [0, 1, 33, 64, 95, 160, 255, 319, 320, 321]


@pytest.mark.parametrize("act", ["swiglu", "relu"])
def test_ffn_backward_packed_tall_tiles(act):
    E, d, h = len(TALL_COUNTS), 256, 2048
    used = sum(TALL_COUNTS)
    rows = used + 37
    assert rows > 128 * E, "must take the 320-row tiles"
    print(f"[ffn backward packed tall] E={E} rows={rows} d={d} h={h} {act}", flush=True)
    off = np.concatenate([[0], np.cumsum(TALL_COUNTS)]).astype(np.int32)
    g = torch.Generator().manual_seed(h + E + 1)
    x = torch.randn(rows, d, generator=g).to(BF16)
    dy = (torch.randn(rows, d, generator=g) * 0.5).to(BF16)
    w1, w3, w2 = _weights(E, d, h, act, seed=d + 1, scale=0.05)
    dx, dw1, dw3, dw2 = _gpu_backward(E, rows, d, h, act, x, torch.from_numpy(off), w1, w3, w2,
                                      dy, path="packed")
    oracle.set_threads(threads())
    r_dx, r_dw1, r_dw3, r_dw2 = oracle.expert_ffn_backward("bf16", act, n(x), off, n(w1), n(w3),
                                                           n(w2), n(dy))
    assert bool((dx[used:] == 3.0).all()), "rows outside every segment must stay untouched"
    for e in range(E):
        a, b = int(off[e]), int(off[e + 1])
        if b > a:
            ee = rel_err(dx[a:b].float(), as_tensor(r_dx[a:b], "bf16").float())
            assert ee <= TOL["bf16"], f"dx of expert {e} ({b - a} rows): {ee:.3e}"
    for got, ref, key in ((dw1, r_dw1, "dw1"), (dw3, r_dw3, "dw3"), (dw2, r_dw2, "dw2")):
        if ref is None:
            continue
        for e in range(E):
            ee = rel_err(got[e], torch.from_numpy(ref[e])) if TALL_COUNTS[e] else 0.0
            assert ee <= TOL["bf16"], f"{key}[{e}] ({TALL_COUNTS[e]} rows) max rel err {ee:.3e}"
        assert bool((got[0] == 0).all()), f"{key}: an expert with no rows gets zeros"


# The packed backward on large-expert batches (at least 1024 rows per expert on
# average and 8192 in all) takes the 192-row tiles too: every expert with rows
# spans several of them with a shorter last one, in the grouped block order;
# h = 2048 with SwiGLU takes the wide recompute, h = 1024 with GELU the narrow.
LARGE_COUNTS = [2100, 0, 2500, 1999, 1600]


@pytest.mark.parametrize("h,act", [(2048, "swiglu"), (1024, "gelu")])
def test_ffn_backward_packed_large_expert_tiles(h, act):
    E, d = len(LARGE_COUNTS), 256
    used = sum(LARGE_COUNTS)
    rows = used + 7
    assert rows >= 1024 * E and rows >= 8192, "must take the large-expert 192-row tiles"
    print(f"[ffn backward packed large] E={E} rows={rows} d={d} h={h} {act}", flush=True)
    off = np.concatenate([[0], np.cumsum(LARGE_COUNTS)]).astype(np.int32)
    g = torch.Generator().manual_seed(h + E + 2)
    x = torch.randn(rows, d, generator=g).to(BF16)
    dy = (torch.randn(rows, d, generator=g) * 0.5).to(BF16)
    w1, w3, w2 = _weights(E, d, h, act, seed=d + 2, scale=0.05)
    dx, dw1, dw3, dw2 = _gpu_backward(E, rows, d, h, act, x, torch.from_numpy(off), w1, w3, w2,
                                      dy, path="packed")
    oracle.set_threads(threads())
    r_dx, r_dw1, r_dw3, r_dw2 = oracle.expert_ffn_backward("bf16", act, n(x), off, n(w1), n(w3),
                                                           n(w2), n(dy))
    assert bool((dx[used:] == 3.0).all()), "rows outside every segment must stay untouched"
    for e in range(E):
        a, b = int(off[e]), int(off[e + 1])
        if b > a:
            ee = rel_err(dx[a:b].float(), as_tensor(r_dx[a:b], "bf16").float())
            assert ee <= TOL["bf16"], f"dx of expert {e} ({b - a} rows): {ee:.3e}"
    for got, ref, key in ((dw1, r_dw1, "dw1"), (dw3, r_dw3, "dw3"), (dw2, r_dw2, "dw2")):
        if ref is None:
            continue
        for e in range(E):
            ee = rel_err(got[e], torch.from_numpy(ref[e])) if LARGE_COUNTS[e] else 0.0
            assert ee <= TOL["bf16"], f"{key}[{e}] ({LARGE_COUNTS[e]} rows) max rel err {ee:.3e}"
        assert bool((got[1] == 0).all()), f"{key}: an expert with no rows gets zeros"


@pytest.mark.parametrize("act", ["swiglu", "gelu"])
def test_ffn_backward_packed_empty_batch(act):
    """No rows: every weight gradient is written as zeros, nothing else read
    (no workspace, no activations)."""
    E, d, h = 3, 64, 128
    sw = act == "swiglu"
    w1, w3, w2 = _weights(E, d, h, act, seed=5)
    pw = moe.prepare_backward_weights({"dtype": "bf16", "d": d, "h": h},
                                      {"w1": w1.cuda(), "w3": None if w3 is None else w3.cuda(),
                                       "w2": w2.cuda()})
    off = torch.zeros(E + 1, dtype=torch.int32, device="cuda")
    dw1 = torch.full((E, h, d), 9.0, device="cuda")
    dw3 = torch.full((E, h, d), 9.0, device="cuda") if sw else None
    dw2 = torch.full((E, d, h), 9.0, device="cuda")
    moe.moe_expert_ffn_backward_packed(E, 0, d, h, act, "bf16", None, off, None, pw["w1"],
                                       pw["w3"], pw["w2t"], pw["w13t"], None, None, dw1, dw3, dw2,
                                       None)
    torch.cuda.synchronize()
    for t in (dw1, dw3, dw2):
        if t is not None:
            assert bool((t == 0).all())
