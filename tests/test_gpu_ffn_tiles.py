"""GPU parity of the expert FFN at the edges of its row tiles, and the bf16
weight packing as an exact permutation.

Row tiles hold up to 320 rows in 32-row fragments, experts longer than that
are split into equal tiles, and fragments without rows are skipped: the
per-expert row counts below sit on every one of those edges (0, 1, 31/32/33,
160/161, 319/320/321, 641), with output widths that are and are not a
multiple of the column tile.  Experts of many row tiles take the grouped
block order (4 row tiles walk their column tiles together), with a short last
group; decode-sized batches take 128-row tiles with wider column tiles, and
batches of at most 128 rows per expert on average 192-row tiles, as do
batches of at least 1024 rows per expert on average and 8192 in all.
Reference: the oracle's grouped FFN on the same
rows (glossary "Expert Parallelism", step 3), per-tensor max relative error
within 2e-2 (bf16) / 1e-4 (fp32).
"""

import numpy as np
import pytest
import torch

import expert_token_routing_router_amd as moe
import moe_workloads as W
import oracle

from gpu_util import TOL, as_tensor, n, rel_err, threads

pytestmark = pytest.mark.gpu

COUNTS = [0, 1, 31, 32, 33, 160, 161, 200, 319, 320, 321, 641, 5, 0, 96, 257]


def packed_reference(w: np.ndarray) -> np.ndarray:
    """The layout include/moe.h states for moe_expert_ffn_pack_weights, in
    numpy, read backwards: packed element p comes from row es*S + 16g + L/4,
    column 32t + 8((L%4) ^ sw(L/4)) + u of W viewed as [E*rows, cols]."""
    E, R, C = w.shape
    S = 256 if R % 256 == 0 else 64
    p = np.arange(E * R * C, dtype=np.int64)
    blk, within = p // 512, p % 512
    L, u = within // 8, within % 8
    g, st = blk % (S // 16), blk // (S // 16)
    t, es = st % (C // 32), st // (C // 32)
    r = L // 4
    sw = ((r >> 1) ^ (r >> 2)) & 3
    src = (es * S + 16 * g + r) * C + 32 * t + 8 * ((L % 4) ^ sw) + u
    assert np.unique(src).size == src.size  # a permutation
    return w.reshape(-1)[src].reshape(w.shape)


@pytest.mark.parametrize("E,R,C", [(1, 64, 64), (3, 192, 128), (2, 1024, 320), (2, 512, 64)])
def test_pack_weights_is_the_documented_permutation(E, R, C):
    g = torch.Generator().manual_seed(E * 1000 + R + C)
    w = torch.randn(E, R, C, generator=g).bfloat16()
    wd = w.cuda()
    wp = torch.empty_like(wd)
    moe.moe_expert_ffn_pack_weights(E, R, C, "bf16", wd, wp)
    torch.cuda.synchronize()
    got = wp.cpu().view(torch.int16).numpy()
    want = packed_reference(w.view(torch.int16).numpy())
    assert np.array_equal(got, want)
    assert torch.equal(wd.cpu().view(torch.int16), w.view(torch.int16))  # source untouched


def _inputs(d, h, act, dtype, seed, counts=COUNTS, spare=7):
    g = torch.Generator().manual_seed(seed)
    E, M = len(counts), sum(counts)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    x = torch.randn(M + spare, d, generator=g).to(tdt)
    w1 = (torch.randn(E, h, d, generator=g) / d ** 0.5).to(tdt)
    w3 = (torch.randn(E, h, d, generator=g) / d ** 0.5).to(tdt) if act == "swiglu" else None
    w2 = (torch.randn(E, d, h, generator=g) / h ** 0.5).to(tdt)
    offs = torch.tensor(np.concatenate([[0], np.cumsum(counts)]), dtype=torch.int32)
    return x, w1, w3, w2, offs


@pytest.mark.parametrize("d,h,act,dtype", [
    (128, 256, "gelu", "bf16"),     # 128-column tiles in both GEMMs
    (128, 256, "swiglu", "bf16"),   # gate and up in one tile
    (128, 192, "relu", "bf16"),     # h not a multiple of the column tile
    (1024, 2048, "gelu", "bf16"),   # 256-column tiles in both GEMMs
    (128, 256, "gelu", "fp32"),
])
def test_ffn_row_tile_edges(d, h, act, dtype):
    _check_ffn(d, h, act, dtype, COUNTS, seed=d + h)


# Experts of several row tiles each (5, 0, 3 and 7 tiles: 15 in all): the bf16
# GEMMs then walk groups of 4 row tiles column tile by column tile, and the
# last group holds 3.  Several column tiles in both GEMMs.
@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_ffn_grouped_row_tiles(act):
    _check_ffn(512, 1024, act, "bf16", [1500, 0, 700, 2100], seed=77)


# At least 1024 rows per expert on average and 8192 in all: the 192-row tiles
# (the wide form where h >= 2048), every expert split into several of them
# with a shorter last tile, in the grouped block order; every row checked.
LARGE_COUNTS = [2100, 0, 2500, 1999, 3001]


@pytest.mark.parametrize("d,h,act", [(256, 2048, "swiglu"), (512, 1024, "gelu")])
def test_ffn_large_expert_row_tiles(d, h, act):
    M = sum(LARGE_COUNTS) + 7
    assert M >= 1024 * len(LARGE_COUNTS) and M >= 8192, "must take the 192-row tiles"
    _check_ffn(d, h, act, "bf16", LARGE_COUNTS, seed=d + 11 * h)


# Decode-sized batches (at most 32 rows per expert on average) take 128-row
# tiles with twice the columns per tile: experts of 0, 1, 31/32/33, 64, 127,
# 128, 129 (split in two) and 300 (split in three) rows among many small ones,
# with output widths that are and are not a multiple of the wider column tile.
SMALL_COUNTS = [0, 1, 31, 32, 33, 64, 127, 128, 129, 300] + [3, 0, 7, 1] * 24


@pytest.mark.parametrize("d,h,act", [(512, 1024, "swiglu"), (512, 2048, "gelu"),
                                     (2048, 640, "swiglu"), (384, 512, "relu")])
def test_ffn_small_row_tiles(d, h, act):
    assert sum(SMALL_COUNTS) + 7 <= 32 * len(SMALL_COUNTS), "must take the 128-row tiles"
    _check_ffn(d, h, act, "bf16", SMALL_COUNTS, seed=d + 3 * h)


# Batches of at most 128 rows per expert on average (the DeepSeek-like layer)
# take 192-row tiles: experts on the fragment edges of such a tile (0, 1,
# 31/32/33, 63/64/65, 96, 127/128/129, 160, 191/192), one just past it (193,
# split in two) and one of three tiles (385), among experts of 100 rows.
MID_COUNTS = [0, 1, 31, 32, 33, 63, 64, 65, 96, 127, 128, 129, 160, 191, 192, 193, 385] + [100] * 15


@pytest.mark.parametrize("d,h,act", [(512, 1024, "swiglu"), (384, 2048, "gelu"),
                                     (1024, 640, "swiglu"), (256, 512, "relu")])
def test_ffn_mid_row_tiles(d, h, act):
    M = sum(MID_COUNTS) + 7
    assert 32 * len(MID_COUNTS) < M <= 128 * len(MID_COUNTS), "must take the 192-row tiles"
    _check_ffn(d, h, act, "bf16", MID_COUNTS, seed=d + 5 * h)


# Wide 192-row tiles (SwiGLU up: 256 columns of each of W1 and W3; down: 512
# columns when d >= 4096; one register set per wave): the fragment edges of
# MID_COUNTS without the fillers, at widths that are multiples of the column
# tile and at widths that are not (partial last column tile, 64-row weight
# slabs).
WIDE_COUNTS = MID_COUNTS[:17]


@pytest.mark.parametrize("d,h,act", [(4096, 2048, "swiglu"), (4160, 2112, "swiglu"),
                                     (4096, 2048, "gelu")])
def test_ffn_wide_row_tiles(d, h, act):
    M = sum(WIDE_COUNTS) + 7
    assert 32 * len(WIDE_COUNTS) < M <= 128 * len(WIDE_COUNTS), "must take the 192-row tiles"
    _check_ffn(d, h, act, "bf16", WIDE_COUNTS, seed=d + 7 * h)


# A bound far above the rows the batch holds (a capacity-bound layer whose hot
# experts dropped most of their slots): the bound alone asks for 320-row
# tiles, the plan sees at most 128 rows per expert and picks the 192-row ones,
# and both GEMMs follow its choice.  The same experts at a bound that keeps
# 320-row tiles give the same outputs to the tolerance.
@pytest.mark.parametrize("d,h,act", [(512, 1024, "swiglu"), (384, 2048, "gelu"),
                                     (4096, 2048, "swiglu"), (256, 512, "relu")])
def test_ffn_plan_picks_the_row_tile_height(d, h, act):
    counts = WIDE_COUNTS if d >= 4096 else MID_COUNTS  # d >= 4096: 512-column down tiles
    spare = 3 * sum(counts)
    M = sum(counts) + spare
    assert M > 128 * len(counts) >= sum(counts), "bound: 320 rows; batch: 192"
    _check_ffn(d, h, act, "bf16", counts, seed=d + 11 * h, spare=spare)


def _check_ffn(d, h, act, dtype, counts, seed, spare=7):
    print(f"[ffn tiles] d={d} h={h} act={act} dtype={dtype} counts={counts} spare={spare}",
          flush=True)
    x, w1, w3, w2, offs = _inputs(d, h, act, dtype, seed=seed, counts=counts, spare=spare)
    E, M = len(counts), x.shape[0]
    cfg = {"dtype": dtype, "d": d, "h": h}
    wts = moe.prepare_weights(cfg, {"w1": w1.cuda(), "w3": None if w3 is None else w3.cuda(),
                                    "w2": w2.cuda()})
    y = torch.full((M, d), 7.0, dtype=x.dtype, device="cuda")
    ws = moe.workspace(moe.moe_expert_ffn_workspace_size(E, M, d, h, act, dtype))
    moe.moe_expert_ffn(E, M, d, h, act, dtype, x.cuda(), offs.cuda(), wts["w1"], wts["w3"],
                       wts["w2"], y, None, ws)
    torch.cuda.synchronize()
    oracle.set_threads(threads())
    ref = oracle.expert_ffn(dtype, act, n(x), n(offs), n(w1), n(w3), n(w2))
    used = int(offs[-1])
    err = rel_err(y[:used].float(), as_tensor(ref[:used], dtype).float())
    assert err <= TOL[dtype], f"max rel err {err:.3e}"
    # Each expert's rows on their own: no tile edge may hide behind a larger one.
    for e in range(E):
        a, b = int(offs[e]), int(offs[e + 1])
        if b > a:
            ee = rel_err(y[a:b].float(), as_tensor(ref[a:b], dtype).float())
            assert ee <= TOL[dtype], f"expert {e} ({b - a} rows): {ee:.3e}"
    assert bool((y[used:].float() == 7.0).all()), "rows past offsets[E] were written"
