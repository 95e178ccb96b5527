"""Pins of the oracle's expert-FFN backward (the backward of the layer's expert
networks; each expert is an ordinary feed-forward block).

- torch autograd in fp64 on the same per-expert networks (an independent
  implementation of the chain rule): every gradient, each activation, with
  an expert that has no rows;
- central finite differences of <dy, FFN(x)> through the oracle's own forward
  (``oracle.expert_ffn``), in inputs and in every weight tensor;
- the weight gradients add over rows: two experts sharing weights give
  gradients that sum to those of one expert over all their rows;
- bf16: the returned H, du and dv are bf16 values, and the whole backward
  stays within bf16 rounding of the fp32 result.
"""

import numpy as np
import pytest
import torch

import oracle

ACTS = ["relu", "gelu", "swiglu"]


def _net(E, d, h, act, seed, scale=0.3):
    g = np.random.default_rng(seed)
    w1 = (g.standard_normal((E, h, d)) * scale / np.sqrt(d)).astype(np.float32) * 3
    w3 = (g.standard_normal((E, h, d)) * scale / np.sqrt(d)).astype(np.float32) * 3
    w2 = (g.standard_normal((E, d, h)) * scale / np.sqrt(h)).astype(np.float32) * 3
    return w1, (w3 if act == "swiglu" else None), w2


def _rows(n, d, seed):
    g = np.random.default_rng(seed)
    return g.standard_normal((n, d)).astype(np.float32)


def _autograd(act, x, offsets, w1, w3, w2, dy):
    """fp64 autograd of sum <dy, y> with y = act(x W1^T) [* x W3^T] W2^T per segment."""
    X = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    W1 = torch.tensor(w1, dtype=torch.float64, requires_grad=True)
    W2 = torch.tensor(w2, dtype=torch.float64, requires_grad=True)
    W3 = torch.tensor(w3, dtype=torch.float64, requires_grad=True) if w3 is not None else None
    ys = []
    for e in range(w1.shape[0]):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        xe = X[lo:hi]
        u = xe @ W1[e].T
        if act == "relu":
            H = torch.relu(u)
        elif act == "gelu":
            H = torch.nn.functional.gelu(u)  # exact (erf) form
        else:
            H = torch.nn.functional.silu(u) * (xe @ W3[e].T)
        ys.append(H @ W2[e].T)
    y = torch.cat(ys)
    (y * torch.tensor(dy[: y.shape[0]], dtype=torch.float64)).sum().backward()
    g3 = W3.grad.numpy() if W3 is not None else None
    return X.grad.numpy(), W1.grad.numpy(), g3, W2.grad.numpy()


def _close(a, b, tol):
    scale = max(np.abs(b).max(), 1e-30)
    return np.abs(np.asarray(a, np.float64) - b).max() / scale <= tol


@pytest.mark.parametrize("act", ACTS)
def test_matches_fp64_autograd(act):
    E, d, h = 3, 24, 16
    offsets = np.array([0, 5, 5, 12], np.int32)  # expert 1 has no rows
    w1, w3, w2 = _net(E, d, h, act, seed=11)
    x, dy = _rows(12, d, 1), _rows(12, d, 2)
    dx, dw1, dw3, dw2 = oracle.expert_ffn_backward("fp32", act, x, offsets, w1, w3, w2, dy)
    rx, r1, r3, r2 = _autograd(act, x, offsets, w1, w3, w2, dy)
    assert _close(dx, rx, 1e-5)
    assert _close(dw1, r1, 1e-5)
    assert _close(dw2, r2, 1e-5)
    if act == "swiglu":
        assert _close(dw3, r3, 1e-5)
    else:
        assert dw3 is None
    assert not dw1[1].any() and not dw2[1].any(), "an expert with no rows has zero gradients"


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_finite_differences_through_forward(act):
    """d/dtheta <dy, FFN(x)> by central differences of the oracle's forward."""
    E, d, h = 2, 16, 8
    offsets = np.array([0, 3, 7], np.int32)
    w1, w3, w2 = _net(E, d, h, act, seed=5)
    x, dy = _rows(7, d, 3), _rows(7, d, 4)
    dx, dw1, dw3, dw2 = oracle.expert_ffn_backward("fp32", act, x, offsets, w1, w3, w2, dy)

    def loss(x_, w1_, w3_, w2_):
        y = oracle.expert_ffn("fp32", act, x_, offsets, w1_, w3_, w2_)
        return float(np.sum(y.astype(np.float64) * dy))

    eps = 1e-2
    g = np.random.default_rng(9)
    params = [("x", x, dx), ("w1", w1, dw1), ("w2", w2, dw2)]
    if act == "swiglu":
        params.append(("w3", w3, dw3))
    for name, t, grad in params:
        for _ in range(4):
            idx = tuple(int(g.integers(0, s)) for s in t.shape)
            args = {"x": x, "w1": w1, "w3": w3, "w2": w2}
            plus, minus = t.copy(), t.copy()
            plus[idx] += eps
            minus[idx] -= eps
            args_p = dict(args, **{name: plus})
            args_m = dict(args, **{name: minus})
            fd = (loss(args_p["x"], args_p["w1"], args_p["w3"], args_p["w2"]) -
                  loss(args_m["x"], args_m["w1"], args_m["w3"], args_m["w2"])) / (2 * eps)
            assert abs(fd - float(grad[idx])) <= 2e-3 * max(1.0, np.abs(grad).max()), (name, idx)


@pytest.mark.parametrize("act", ACTS)
def test_weight_gradients_add_over_rows(act):
    """Splitting one expert's rows between two experts with the same weights
    splits its weight gradients into two parts that sum to the whole, and
    leaves dx unchanged."""
    d, h, n, m = 32, 24, 10, 4
    w1, w3, w2 = _net(1, d, h, act, seed=21)
    x, dy = _rows(n, d, 6), _rows(n, d, 7)
    one = oracle.expert_ffn_backward("fp32", act, x, np.array([0, n], np.int32), w1, w3, w2, dy)
    dup = lambda w: None if w is None else np.concatenate([w, w])  # noqa: E731
    two = oracle.expert_ffn_backward("fp32", act, x, np.array([0, m, n], np.int32), dup(w1),
                                     dup(w3), dup(w2), dy)
    assert np.array_equal(one[0], two[0])
    for a, b in zip(one[1:], two[1:]):
        if a is None:
            assert b is None
            continue
        assert _close(b[0] + b[1], a[0], 1e-6)
        assert np.abs(b[0]).max() > 0 and np.abs(b[1]).max() > 0


def _bf16(a):
    """Round-to-nearest-even fp32 -> bf16 bit patterns."""
    u = np.ascontiguousarray(a, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _from_bf16(b):
    return (b.astype(np.uint32) << 16).view(np.float32)


@pytest.mark.parametrize("act", ACTS)
def test_bf16_rounding_points(act):
    d, h = 64, 32
    w1, w3, w2 = _net(1, d, h, act, seed=31)
    x, dy = _rows(1, d, 8)[0], _rows(1, d, 9)[0]
    b = lambda a: None if a is None else _bf16(a)  # noqa: E731
    f = lambda a: None if a is None else _from_bf16(a)  # noqa: E731
    w1b, w3b, w2b, xb, dyb = b(w1[0]), b(None if w3 is None else w3[0]), b(w2[0]), b(x), b(dy)
    dx, H, du, dv = oracle.ffn_backward_row("bf16", act, xb, w1b, w3b, w2b, dyb)
    for v in (H, du, dv):  # each is a bf16 value
        assert np.array_equal(_from_bf16(_bf16(v.astype(np.float32))).astype(np.float64), v)
    dx32, H32, du32, dv32 = oracle.ffn_backward_row("fp32", act, f(xb), f(w1b), f(w3b), f(w2b),
                                                    f(dyb))
    assert np.abs(H - H32).max() <= 2.0 ** -8 * np.abs(H32).max()
    assert np.abs(du - du32).max() <= 2.0 ** -8 * np.abs(du32).max()
    assert np.abs(_from_bf16(dx) - dx32).max() <= 2e-2 * np.abs(dx32).max()
