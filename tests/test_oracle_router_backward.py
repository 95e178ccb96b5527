"""Pins of the oracle's router backward and auxiliary load-balancing loss.  CPU
only.  None retypes the oracle's formulas: the gradients are checked against
torch fp64 autograd of the forward definitions (the combine weights of each
score function on a fixed selection, the load-balancing loss, the router's
linear layer), against central differences through the oracle's own forward,
and against identities the exact gradients satisfy (softmax shift invariance;
the sigmoid renormalisation's invariance to scaling the selected affinities;
zero gradient and loss = coefficient at uniform load)."""

import numpy as np
import pytest
import torch

import moe_workloads as W
import oracle

SCORES = ["softmax_topk", "softmax_all", "sigmoid_norm"]


def _cfg(N, d, E, k, score, dtype="fp32", G=1, kg=1):
    return dict(name="rb", N=N, d=d, h=8, E=E, k=k, R=1, cf=0.0, G=G, kg=kg, score=score,
                act="relu", dtype=dtype)


def _case(seed, N, E, k, score, G=1, kg=1, drop=0.2, scale=1.0):
    """Logits, a selection the oracle itself makes (with a selection bias and
    a group limit when G > 1), and dtopk_w with some slots dropped (g = 0)."""
    rng = np.random.default_rng(seed)
    cfg = _cfg(N, 16, E, k, score, G=G, kg=kg)
    z = (rng.standard_normal((N, E)) * scale).astype(np.float32)
    sb = (rng.standard_normal(E) * 0.3).astype(np.float32)
    sel = oracle.select(cfg, z, sb)
    g = rng.standard_normal((N, k)).astype(np.float32)
    g[rng.random((N, k)) < drop] = 0.0
    return cfg, z, sel["topk_idx"], sel["topk_w"], g, sel["counts"]


def _torch_loss(z64, idx, g, counts, coef, score):
    """The forward definition in torch: combine weights of the selected
    experts, weighted by g, plus coef * E * sum_e f_e P_e."""
    N, E = z64.shape
    k = idx.shape[1]
    ii = torch.from_numpy(idx.astype(np.int64))
    gg = torch.from_numpy(g.astype(np.float64))
    if score == "softmax_topk":
        w = torch.softmax(z64.gather(1, ii), dim=1)
        P = torch.softmax(z64, dim=1)
    elif score == "softmax_all":
        P = torch.softmax(z64, dim=1)
        w = P.gather(1, ii)
    else:
        a = torch.sigmoid(z64)
        sa = a.gather(1, ii)
        w = sa / sa.sum(1, keepdim=True)
        P = a / a.sum(1, keepdim=True)
    loss = (w * gg).sum()
    if coef:
        f = torch.from_numpy(counts.astype(np.float64)) / (N * k)
        loss = loss + coef * E * (f * P.mean(0)).sum()
    return loss


@pytest.mark.parametrize("score", SCORES)
@pytest.mark.parametrize("coef", [0.0, 0.01])
def test_dz_equals_autograd_of_the_forward(score, coef):
    G, kg = (4, 2) if score == "sigmoid_norm" else (1, 1)
    cfg, z, idx, _, g, counts = _case(7, 97, 16, 3, score, G=G, kg=kg)
    z64 = torch.tensor(z, dtype=torch.float64, requires_grad=True)
    loss = _torch_loss(z64, idx, g, counts, coef, score)
    loss.backward()
    x = np.zeros((cfg["N"], cfg["d"]), np.float32)
    wr = np.zeros((cfg["E"], cfg["d"]), np.float32)
    out = oracle.router_backward(cfg, x, wr, z, idx, g, counts, coef)
    ref = z64.grad.numpy()
    assert np.abs(out["dz"] - ref).max() <= 1e-6 * np.abs(ref).max() + 1e-12
    if coef:
        # the loss value itself: coef * E * sum f P (the weights part is not in it)
        aux = _torch_loss(torch.tensor(z, dtype=torch.float64), idx, np.zeros_like(g), counts,
                          coef, score).item()
        assert abs(out["aux_loss"] - aux) <= 1e-12 * abs(aux) + 1e-15
    else:
        assert out["aux_loss"] == 0.0


@pytest.mark.parametrize("score", SCORES)
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_router_gradients_equal_autograd_through_the_linear(score, dtype):
    """z = x W_r^T + b; dW_r, db and dx of the same loss by autograd in fp64
    (the oracle takes the logits as fp32 values, autograd keeps them fp64)."""
    rng = np.random.default_rng(11)
    N, d, E, k, coef = 41, 24, 8, 2, 0.02
    cfg = _cfg(N, d, E, k, score, dtype=dtype)
    x = torch.from_numpy(rng.standard_normal((N, d)).astype(np.float32))
    wr = torch.from_numpy((rng.standard_normal((E, d)) * 0.3).astype(np.float32))
    b = torch.from_numpy((rng.standard_normal(E) * 0.1).astype(np.float32))
    if dtype == "bf16":
        x, wr = x.bfloat16(), wr.bfloat16()
    xn, wn = W.to_numpy(x), W.to_numpy(wr)
    z = oracle.logits(cfg, xn, wn, b.numpy())
    sel = oracle.select(cfg, z)
    g = rng.standard_normal((N, k)).astype(np.float32)
    x64 = x.double().requires_grad_(True)
    w64 = wr.double().requires_grad_(True)
    b64 = b.double().requires_grad_(True)
    loss = _torch_loss(x64 @ w64.T + b64, sel["topk_idx"], g, sel["counts"], coef, score)
    loss.backward()
    out = oracle.router_backward(cfg, xn, wn, z, sel["topk_idx"], g, sel["counts"], coef)
    rel = lambda a, r: np.abs(a.astype(np.float64) - r).max() / max(np.abs(r).max(), 1e-30)  # noqa
    assert rel(out["dw_router"], w64.grad.numpy()) <= 1e-5
    assert rel(out["db"], b64.grad.numpy()) <= 1e-5
    dx = out["dx"] if dtype == "fp32" else W.from_numpy_bf16(out["dx"]).double().numpy()
    assert rel(dx, x64.grad.numpy()) <= (1e-5 if dtype == "fp32" else 8e-3)


@pytest.mark.parametrize("score", SCORES)
def test_dz_by_central_differences_through_the_oracle_forward(score):
    """Perturb one logit at a time (the selection has wide margins, so it does
    not change) and difference the oracle's own combine weights (weighted by g)
    plus its own auxiliary loss value."""
    rng = np.random.default_rng(23)
    N, E, k, coef = 6, 8, 2, 0.05
    cfg = _cfg(N, 16, E, k, score)
    z = (rng.standard_normal((N, E)) * 0.3).astype(np.float32)
    for t in range(N):  # experts t % E and (t + 3) % E chosen with a margin of 4
        z[t, t % E] += 4.0
        z[t, (t + 3) % E] += 4.0
    sel = oracle.select(cfg, z)
    idx, counts = sel["topk_idx"], sel["counts"]
    g = rng.standard_normal((N, k)).astype(np.float32)
    x = np.zeros((N, 16), np.float32)
    wr = np.zeros((E, 16), np.float32)
    dz = oracle.router_backward(cfg, x, wr, z, idx, g, counts, coef)["dz"]

    def L(zz):
        s = oracle.select(cfg, zz)
        assert np.array_equal(s["topk_idx"], idx)
        aux = oracle.router_backward(cfg, x, wr, zz, idx, np.zeros_like(g), counts,
                                     coef)["aux_loss"]
        return float((s["topk_w"].astype(np.float64) * g).sum()) + aux

    eps = 1e-2
    for t, e in [(0, 0), (0, 3), (1, 5), (2, 2), (4, 7), (5, 0)]:
        zp, zm = z.copy(), z.copy()
        zp[t, e] += eps
        zm[t, e] -= eps
        fd = (L(zp) - L(zm)) / (2 * eps)
        assert abs(fd - dz[t, e]) <= 2e-3 * max(abs(dz[t, e]), 1e-2), (t, e, fd, dz[t, e])


@pytest.mark.parametrize("score", ["softmax_topk", "softmax_all"])
def test_softmax_gradients_sum_to_zero_per_token(score):
    """Adding a constant to a token's logits changes no softmax, so the exact
    gradient sums to zero over each token's experts (aux loss included)."""
    cfg, z, idx, _, g, counts = _case(31, 200, 32, 4, score, scale=2.0)
    out = oracle.router_backward(cfg, np.zeros((200, 16), np.float32),
                                 np.zeros((32, 16), np.float32), z, idx, g, counts, 0.03)
    s = out["dz"].astype(np.float64).sum(1)
    assert np.abs(s).max() <= 1e-6 * np.abs(out["dz"]).max()


def test_sigmoid_norm_gradient_is_scale_invariant():
    """Scaling all selected affinities by one factor leaves the renormalised
    weights unchanged, so sum over the selected of a * dL/da = 0, i.e.
    sum_j dz_j / (1 - a_j) = 0 per token (no aux loss); unselected get 0."""
    cfg, z, idx, _, g, counts = _case(41, 150, 32, 8, "sigmoid_norm", G=8, kg=4)
    out = oracle.router_backward(cfg, np.zeros((150, 16), np.float32),
                                 np.zeros((32, 16), np.float32), z, idx, g, counts, 0.0)
    dz = out["dz"].astype(np.float64)
    a = 1.0 / (1.0 + np.exp(-z.astype(np.float64)))
    mask = np.zeros_like(dz, bool)
    np.put_along_axis(mask, idx.astype(np.int64), True, axis=1)
    assert (dz[~mask] == 0).all()
    s = (dz / (1.0 - a) * mask).sum(1)
    assert np.abs(s).max() <= 1e-5 * np.abs(dz).max()


@pytest.mark.parametrize("score", SCORES)
def test_aux_loss_at_uniform_load(score):
    """Equal logits in every token and exactly uniform counts: every P_e and f_e
    is 1/E, so the loss is the coefficient itself and its gradient is zero."""
    N, E, k, coef = 64, 8, 2, 0.7
    cfg = _cfg(N, 16, E, k, score)
    z = np.full((N, E), 0.25, np.float32)
    idx = np.stack([[(2 * t) % E, (2 * t + 1) % E] for t in range(N)]).astype(np.int32)
    counts = np.bincount(idx.ravel(), minlength=E).astype(np.int32)
    assert (counts == N * k // E).all()
    out = oracle.router_backward(cfg, np.zeros((N, 16), np.float32),
                                 np.zeros((E, 16), np.float32), z, idx,
                                 np.zeros((N, k), np.float32), counts, coef)
    assert abs(out["aux_loss"] - coef) <= 1e-12
    assert np.abs(out["dz"]).max() <= 1e-12


def test_dx_in_is_added_before_the_rounding():
    """dx with dx_in equals the fp64 sum of dx without it and dx_in, rounded once."""
    cfg, z, idx, _, g, counts = _case(53, 30, 8, 2, "softmax_topk")
    rng = np.random.default_rng(5)
    x = rng.standard_normal((30, 16)).astype(np.float32)
    wr = rng.standard_normal((8, 16)).astype(np.float32)
    dxi = rng.standard_normal((30, 16)).astype(np.float32)
    a = oracle.router_backward(cfg, x, wr, z, idx, g, counts, 0.0)["dx"]
    b = oracle.router_backward(cfg, x, wr, z, idx, g, counts, 0.0, dx_in=dxi)["dx"]
    assert np.abs(b.astype(np.float64) - (a.astype(np.float64) + dxi)).max() <= \
        2e-7 * np.abs(b).max()
