"""Pins of the oracle's backward data path (the combine's expert terms and the
permute, read backwards).  CPU only.  Each pin is an identity the backward must
satisfy with respect to the forward, not its formula retyped: the adjoint
identities of the two linear maps, finite differences in the weights, and
dropped slots."""

import numpy as np
import torch

import moe_workloads as W
import oracle


def _bf16(a):
    """numpy fp32 -> bf16 bits (round to nearest even), as the oracle takes them."""
    return W.to_numpy(torch.from_numpy(np.asarray(a, np.float32)).bfloat16())


def _layout(rng, N, E, k, cf):
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(N)]).astype(np.int32)
    cfg = dict(name="t", N=N, d=8, h=8, E=E, k=k, R=1, cf=cf, G=1, kg=1,
               score="softmax_topk", act="relu", dtype="fp32")
    return cfg, oracle.dispatch(cfg, idx)


def test_combine_backward_is_the_adjoint_of_the_combine():
    """L(v) = sum_t <dy[t], sum_j w_tj v[r_tj]> is linear in the expert rows v,
    so L(v) = sum_r <dy_perm[r], v[r]> for every v; with drops (cf 0.5)."""
    rng = np.random.default_rng(50)
    N, E, k, d = 300, 8, 2, 48
    cfg, dsp = _layout(rng, N, E, k, 0.5)
    M = dsp["num_rows"]
    w = rng.random((N, k)).astype(np.float32)
    dy = rng.standard_normal((N, d)).astype(np.float32)
    y_perm = rng.standard_normal((M, d)).astype(np.float32)
    dy_perm, dw = oracle.combine_backward("fp32", dy, y_perm, dsp["row_of_slot"], w, M)
    for trial in range(3):
        v = rng.standard_normal((M, d)).astype(np.float32)
        lhs = (dy.astype(np.float64) * oracle.combine("fp32", v, dsp["row_of_slot"], w)).sum()
        rhs = (dy_perm.astype(np.float64) * v).sum()
        assert abs(lhs - rhs) <= 1e-5 * (np.abs(dy).sum() * np.abs(v).max() + 1)


def test_weight_gradients_by_finite_differences():
    """dL/dw_tj for L = <dy, combine(y_perm, w)>: the combine is linear in each
    weight, so a difference quotient gives it up to rounding."""
    rng = np.random.default_rng(51)
    N, E, k, d = 40, 4, 2, 32
    cfg, dsp = _layout(rng, N, E, k, 0.0)
    M = dsp["num_rows"]
    w = rng.random((N, k)).astype(np.float32)
    dy = rng.standard_normal((N, d)).astype(np.float32)
    y_perm = rng.standard_normal((M, d)).astype(np.float32)
    _, dw = oracle.combine_backward("fp32", dy, y_perm, dsp["row_of_slot"], w, M)

    def loss(ww):
        return (dy.astype(np.float64) * oracle.combine("fp32", y_perm, dsp["row_of_slot"],
                                                       ww).astype(np.float64)).sum()
    base = loss(w)
    for t, j in [(0, 0), (5, 1), (17, 0), (39, 1)]:
        w2 = w.copy()
        w2[t, j] += np.float32(0.5)
        fd = (loss(w2) - base) / 0.5
        assert abs(fd - dw[t, j]) <= 1e-4 * (abs(dw[t, j]) + 1)


def test_dropped_slots_have_zero_weight_gradient():
    rng = np.random.default_rng(52)
    cfg, dsp = _layout(rng, 200, 8, 2, 0.25)
    M = dsp["num_rows"]
    ros = dsp["row_of_slot"]
    assert (ros < 0).any()
    dy = rng.standard_normal((200, 16)).astype(np.float32)
    y_perm = rng.standard_normal((M, 16)).astype(np.float32)
    w = rng.random((200, 2)).astype(np.float32)
    dy_perm, dw = oracle.combine_backward("fp32", dy, y_perm, ros, w, M)
    assert np.all(dw[ros < 0] == 0)
    # every admitted row receives its slot's w * dy
    t, j = np.nonzero(ros >= 0)
    np.testing.assert_allclose(dy_perm[ros[t, j]], w[t, j, None] * dy[t], rtol=1e-6)


def test_permute_backward_is_the_adjoint_of_the_permute():
    """<dx_perm, permute(x)> = <permute_backward(dx_perm), x> (bf16 rows, fp32
    sums), with drops; a token with every slot dropped gets zero."""
    rng = np.random.default_rng(53)
    N, E, k, d = 257, 8, 3, 40
    cfg, dsp = _layout(rng, N, E, k, 0.4)
    M = dsp["num_rows"]
    x = _bf16(rng.standard_normal((N, d)))
    dx_perm = _bf16(rng.standard_normal((M, d)))
    xp = oracle.permute("bf16", x, dsp["token_of_row"], M)
    dx = oracle.permute_backward("bf16", dx_perm, dsp["row_of_slot"])
    f = lambda a: W.from_numpy_bf16(a).double().numpy()
    lhs = (f(dx_perm) * f(xp)).sum()
    rhs = (f(dx) * f(x)).sum()
    assert abs(lhs - rhs) <= 2 ** -7 * (np.abs(f(dx_perm)).sum() * np.abs(f(x)).max())
    none = np.all(dsp["row_of_slot"] < 0, axis=1)
    assert np.all(f(dx)[none] == 0)
