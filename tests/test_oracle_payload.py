"""Pins of the oracle's INT8 dispatch payload (one symmetric scale per token
row; EP notes, "深入推导": INT8-quantised communication halves the exchange
volume).  CPU only.  Each pin is a closed form or an invariant, not the
formula retyped: exact codes for rows on the grid, ties to even at exact
halves, the round-trip bound, symmetry, monotonicity, zero rows."""

import numpy as np
import torch

import oracle


def _bf16(a):
    return torch.from_numpy(np.asarray(a, np.float32)).bfloat16().view(torch.int16).numpy().view(np.uint16)


def test_rows_on_the_grid_give_their_integers():
    """x = k * 2^e with integer |k| <= 127 and max |k| = 127: the scale is 2^e,
    the codes are k and dequantisation is exact (fp32 and bf16)."""
    rng = np.random.default_rng(40)
    for dtype in ("fp32", "bf16"):
        for e in (-20, -3, 0, 5):
            k = rng.integers(-127, 128, size=(6, 96))
            k[:, 7] = 127 * np.sign(rng.standard_normal(6)).astype(np.int64)
            x = (k * 2.0 ** e).astype(np.float32)
            xin = x if dtype == "fp32" else _bf16(x)
            q, s = oracle.quantize_rows_q8(dtype, xin)
            assert np.array_equal(q, k.astype(np.int8))
            assert np.all(s == np.float32(2.0 ** e))
            back = oracle.dequantize_rows_q8(dtype, q, s)
            want = x if dtype == "fp32" else _bf16(x)
            assert np.array_equal(back, want)


def test_exact_halves_round_to_even():
    """With amax = 127 the inverse scale is exactly 1, so x = n + 1/2 rounds
    to the even neighbour, in both directions."""
    x = np.array([[127.0, 0.5, 1.5, 2.5, 3.5, -0.5, -1.5, -2.5, 126.5, -126.5]], np.float32)
    q, s = oracle.quantize_rows_q8("fp32", x)
    assert q.tolist() == [[127, 0, 2, 2, 4, 0, -2, -2, 126, -126]]
    assert s[0] == np.float32(1.0)


def test_round_trip_bound_symmetry_and_order():
    """|x - q s| <= s/2 (plus fp32 rounding), the absmax element maps to +-127,
    q(-x) = -q(x), and codes keep the order of the values."""
    rng = np.random.default_rng(41)
    x = (rng.standard_normal((64, 512)) * rng.lognormal(0, 3, size=(64, 1))).astype(np.float32)
    q, s = oracle.quantize_rows_q8("fp32", x)
    back = oracle.dequantize_rows_q8("fp32", q, s).astype(np.float64)
    err = np.abs(back - x.astype(np.float64))
    assert np.all(err <= s[:, None].astype(np.float64) * (0.5 + 1e-5) + np.abs(x) * 2.0 ** -22)
    i = np.argmax(np.abs(x), axis=1)
    assert np.all(np.abs(q[np.arange(64), i]) == 127)
    assert np.all(np.abs(q.astype(int)) <= 127)
    qn, sn = oracle.quantize_rows_q8("fp32", -x)
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)
    for r in range(8):
        order = np.argsort(x[r], kind="stable")
        assert np.all(np.diff(q[r][order].astype(int)) >= 0)


def test_zero_rows_and_scale_invariance():
    """A zero row gives zero codes and scale 0; scaling a row by a power of two
    scales its scale and keeps its codes."""
    rng = np.random.default_rng(42)
    x = rng.standard_normal((5, 64)).astype(np.float32)
    x[2] = 0.0
    q, s = oracle.quantize_rows_q8("fp32", x)
    assert np.all(q[2] == 0) and s[2] == 0
    q2, s2 = oracle.quantize_rows_q8("fp32", x * np.float32(8.0))
    assert np.array_equal(q2, q) and np.array_equal(s2, s * np.float32(8.0))


def test_int8_payload_forward_matches_native_within_quantisation():
    """The layer with the INT8 payload differs from the native one only through
    the dispatched rows: same routing and layout, y_perm rows equal the FFN of
    the dequantised rows, and y stays close to the native output."""
    import moe_workloads as W
    cfg = W.small("switch")
    inp = W.make_inputs(cfg)
    n = W.to_numpy
    args = (n(inp["x"]), n(inp["w_router"]), n(inp["router_bias"]), n(inp["sel_bias"]),
            n(inp["w1"]), n(inp["w3"]), n(inp["w2"]))
    nat = oracle.forward(cfg, *args)
    q8 = oracle.forward(dict(cfg, payload="int8"), *args)
    for key in ("topk_idx", "row_of_slot", "token_of_row", "expert_offsets"):
        assert np.array_equal(nat[key], q8[key])
    M = nat["num_rows"]
    a = W.from_numpy_bf16(q8["x_perm"][:M]).double()
    b = W.from_numpy_bf16(nat["x_perm"][:M]).double()
    assert (a - b).abs().max() <= b.abs().max() / 127
    ya, yb = W.from_numpy_bf16(q8["y"]).double(), W.from_numpy_bf16(nat["y"]).double()
    assert (ya - yb).abs().max() <= 0.05 * yb.abs().max()
