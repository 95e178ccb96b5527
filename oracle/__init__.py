"""CPU oracle of the MoE-layer forward (route, dispatch, expert FFN, combine,
selection-bias update).

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code
with the HIP library and the HIP library never calls it.

The arithmetic lives in ``oracle.c`` (plain per-token loops, fp64); this module
only marshals numpy arrays through ctypes.  bf16 tensors travel as ``uint16``
arrays of their bit patterns.

Workload dictionaries use the keys ``N d E k R cf G kg score dtype`` (and
``h act`` for the FFN); ``score`` is ``softmax_topk``, ``softmax_all`` or
``sigmoid_norm``; ``act`` is ``relu``, ``gelu`` or ``swiglu``; ``dtype`` is
``fp32`` or ``bf16``.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# ORACLE_LIB names another build of the same C file (e.g. one compiled with
# sanitizers); the default is the in-tree build.
DEFAULT_LIB = os.path.join(_HERE, "liboracle.so")
LIB_PATH = os.environ.get("ORACLE_LIB") or DEFAULT_LIB
SRC_PATH = os.path.join(_HERE, "oracle.c")

SCORE_CODES = {"softmax_topk": 0, "softmax_all": 1, "sigmoid_norm": 2}
ACT_CODES = {"relu": 0, "gelu": 1, "swiglu": 2}
DTYPE_CODES = {"fp32": 0, "bf16": 1}


def build(out: str = DEFAULT_LIB, sanitize: bool = False) -> str:
    """Compile the oracle with gcc (strict IEEE: no contraction, no fast-math)
    into ``out``; with ``sanitize`` under AddressSanitizer and
    UndefinedBehaviorSanitizer (abort on the first report)."""
    san = (["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
            "-fno-omit-frame-pointer"] if sanitize else ["-O2"])
    cmd = [
        "gcc", *san, "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared", "-fopenmp",
        "-ffp-contract=off", "-fno-fast-math", "-o", out, SRC_PATH, "-lm",
    ]
    subprocess.run(cmd, check=True)
    return out


class _Desc(ctypes.Structure):
    _fields_ = [
        ("num_tokens", ctypes.c_int32),
        ("hidden", ctypes.c_int32),
        ("num_experts", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("num_ranks", ctypes.c_int32),
        ("capacity_factor", ctypes.c_float),
        ("num_groups", ctypes.c_int32),
        ("topk_groups", ctypes.c_int32),
        ("score_fn", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
    ]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            if LIB_PATH != DEFAULT_LIB:
                raise RuntimeError(f"{LIB_PATH} (ORACLE_LIB) does not exist")
            build()
        L = ctypes.CDLL(LIB_PATH)
        P, I32, F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
        D = ctypes.POINTER(_Desc)
        sig = {
            "oracle_logits": [D, P, P, P, P],
            "oracle_select": [D, P, P, P, P, P, P],
            "oracle_dispatch": [D, P, P, P, P, P, P, P, P],
            "oracle_dispatch_ex": [D, I32, P, P, P, P, P, P, P, P],
            "oracle_permute": [I32, I32, I32, P, P, P],
            "oracle_quantize_rows_q8": [I32, I32, I32, P, P, P],
            "oracle_dequantize_rows_q8": [I32, I32, I32, P, P, P],
            "oracle_ffn_row": [I32, I32, I32, I32, P, P, P, P, P],
            "oracle_expert_ffn": [I32, I32, I32, I32, I32, P, P, P, P, P, P],
            "oracle_ffn_backward_row": [I32, I32, I32, I32, P, P, P, P, P, P, P, P, P],
            "oracle_expert_ffn_backward": [I32, I32, I32, I32, I32, P, P, P, P, P, P, P, P, P,
                                           P],
            "oracle_combine": [I32, I32, I32, I32, P, P, P, P, P, P],
            "oracle_combine_backward": [I32, I32, I32, I32, P, P, P, P, P, P],
            "oracle_bias_update": [I32, I32, I32, P, F32, P],
            "oracle_router_backward": [D, P, P, P, P, P, P, ctypes.c_double, P, P, P, P, P, P],
        }
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = I32
        L.oracle_capacity.argtypes = [D]
        L.oracle_capacity.restype = ctypes.c_int64
        L.oracle_set_threads.argtypes = [I32]
        L.oracle_set_threads.restype = None
        L.oracle_get_threads.argtypes = []
        L.oracle_get_threads.restype = I32
        _lib = L
    return _lib


def _desc(cfg: dict, N: int | None = None) -> _Desc:
    return _Desc(
        int(cfg["N"] if N is None else N), int(cfg["d"]), int(cfg["E"]), int(cfg["k"]),
        int(cfg.get("R", 1)), float(cfg.get("cf", 0.0) or 0.0), int(cfg.get("G", 1)),
        int(cfg.get("kg", 1)), SCORE_CODES[cfg["score"]], DTYPE_CODES[cfg["dtype"]],
    )


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def _elem_dtype(dtype: str):
    return np.float32 if dtype == "fp32" else np.uint16


def _check(rc: int, name: str):
    if rc != 0:
        raise ValueError(f"{name}: invalid arguments")


def set_threads(n: int) -> None:
    lib().oracle_set_threads(int(n))


def get_threads() -> int:
    return int(lib().oracle_get_threads())


def capacity(cfg: dict) -> int:
    d = _desc(cfg)
    return int(lib().oracle_capacity(ctypes.byref(d)))


def logits(cfg: dict, x, w_router, router_bias=None) -> np.ndarray:
    ed = _elem_dtype(cfg["dtype"])
    x, w_router = _c(x, ed), _c(w_router, ed)
    router_bias = _c(router_bias, np.float32)
    N = x.shape[0]
    z = np.empty((N, cfg["E"]), np.float32)
    d = _desc(cfg, N)
    _check(lib().oracle_logits(ctypes.byref(d), _ptr(x), _ptr(w_router), _ptr(router_bias),
                               _ptr(z)), "oracle_logits")
    return z


def select(cfg: dict, z, sel_bias=None) -> dict:
    z = _c(z, np.float32)
    sel_bias = _c(sel_bias, np.float32)
    N, k, E = z.shape[0], cfg["k"], cfg["E"]
    idx = np.empty((N, k), np.int32)
    w = np.empty((N, k), np.float32)
    counts = np.empty(E, np.int32)
    aff = np.empty((N, E), np.float32)
    d = _desc(cfg, N)
    _check(lib().oracle_select(ctypes.byref(d), _ptr(z), _ptr(sel_bias), _ptr(idx), _ptr(w),
                               _ptr(counts), _ptr(aff)), "oracle_select")
    return {"topk_idx": idx, "topk_w": w, "counts": counts, "affinity": aff}


def route(cfg: dict, x, w_router, router_bias=None, sel_bias=None) -> dict:
    z = logits(cfg, x, w_router, router_bias)
    out = select(cfg, z, sel_bias)
    out["logits"] = z
    return out


ADMISSION = {"token": 0, "first_choice": 1}


def dispatch(cfg: dict, topk_idx, admission: str | None = None) -> dict:
    """Capacity, admission and layout.  admission: "token" (default; token
    order) or "first_choice" (every token's first choice before any second
    choice); defaults to cfg.get("admission", "token").  cfg["layout"] ==
    "padded" asks for GShard-style fixed buffers of cap rows per expert."""
    adm = ADMISSION[admission or cfg.get("admission", "token")]
    padded = cfg.get("layout", "compact") == "padded"
    if padded:
        adm |= 2
    topk_idx = _c(topk_idx, np.int32)
    N, k, E, R = topk_idx.shape[0], cfg["k"], cfg["E"], cfg.get("R", 1)
    S = N * k
    rows = max(S, E * capacity(dict(cfg, N=N))) if padded else S
    out = {
        "row_of_slot": np.empty((N, k), np.int32),
        "token_of_row": np.empty(rows, np.int32),
        "slot_of_row": np.empty(rows, np.int8),
        "expert_offsets": np.empty(E + 1, np.int32),
        "admitted": np.empty(E, np.int32),
        "rank_offsets": np.empty(R + 1, np.int32),
        "rank_counts": np.empty(R, np.int32),
    }
    d = _desc(cfg, N)
    _check(lib().oracle_dispatch_ex(
        ctypes.byref(d), adm, _ptr(topk_idx), _ptr(out["row_of_slot"]), _ptr(out["token_of_row"]),
        _ptr(out["slot_of_row"]), _ptr(out["expert_offsets"]), _ptr(out["admitted"]),
        _ptr(out["rank_offsets"]), _ptr(out["rank_counts"])), "oracle_dispatch_ex")
    out["num_rows"] = int(out["expert_offsets"][E])
    return out


def permute(dtype: str, x, token_of_row, num_rows: int) -> np.ndarray:
    ed = _elem_dtype(dtype)
    x = _c(x, ed)
    token_of_row = _c(token_of_row, np.int32)
    out = np.empty((max(num_rows, 0), x.shape[1]), ed)
    _check(lib().oracle_permute(int(num_rows), int(x.shape[1]), DTYPE_CODES[dtype], _ptr(x),
                                _ptr(token_of_row), _ptr(out)), "oracle_permute")
    return out


def ffn_row(dtype: str, act: str, x_row, w1, w3, w2) -> np.ndarray:
    """One row through one expert: w1/w3 are [h,d], w2 is [d,h]."""
    ed = _elem_dtype(dtype)
    x_row, w1, w2 = _c(x_row, ed), _c(w1, ed), _c(w2, ed)
    w3 = _c(w3, ed)
    h, d = w1.shape
    y = np.empty(d, ed)
    _check(lib().oracle_ffn_row(d, h, ACT_CODES[act], DTYPE_CODES[dtype], _ptr(x_row), _ptr(w1),
                                _ptr(w3), _ptr(w2), _ptr(y)), "oracle_ffn_row")
    return y


def expert_ffn(dtype: str, act: str, x_rows, offsets, w1, w3, w2) -> np.ndarray:
    """Grouped FFN over rows [offsets[e], offsets[e+1]) with expert e's weights."""
    ed = _elem_dtype(dtype)
    x_rows, w1, w2 = _c(x_rows, ed), _c(w1, ed), _c(w2, ed)
    w3 = _c(w3, ed)
    offsets = _c(offsets, np.int32)
    E, h, d = w1.shape
    y = np.zeros((x_rows.shape[0], d), ed)
    _check(lib().oracle_expert_ffn(E, d, h, ACT_CODES[act], DTYPE_CODES[dtype], _ptr(x_rows),
                                   _ptr(offsets), _ptr(w1), _ptr(w3), _ptr(w2), _ptr(y)),
           "oracle_expert_ffn")
    return y


def ffn_backward_row(dtype: str, act: str, x_row, w1, w3, w2, dy_row) -> tuple:
    """Backward of one row through one expert: (dx [d] in the dtype, H, du, dv
    as fp64 arrays [h] holding the values the dtype rounds them to)."""
    ed = _elem_dtype(dtype)
    x_row, dy_row, w1, w2 = _c(x_row, ed), _c(dy_row, ed), _c(w1, ed), _c(w2, ed)
    w3 = _c(w3, ed)
    h, d = w1.shape
    dx = np.empty(d, ed)
    H, du, dv = np.empty(h), np.empty(h), np.empty(h)
    _check(lib().oracle_ffn_backward_row(d, h, ACT_CODES[act], DTYPE_CODES[dtype], _ptr(x_row),
                                         _ptr(w1), _ptr(w3), _ptr(w2), _ptr(dy_row), _ptr(dx),
                                         _ptr(H), _ptr(du), _ptr(dv)), "oracle_ffn_backward_row")
    return dx, H, du, dv


def expert_ffn_backward(dtype: str, act: str, x_rows, offsets, w1, w3, w2, dy_rows) -> tuple:
    """Backward of the grouped FFN: (dx_rows in the dtype, rows outside every
    segment zero; dw1, dw3 [E,h,d] and dw2 [E,d,h] in fp32; dw3 None unless
    SwiGLU).  Weights are plain row-major."""
    ed = _elem_dtype(dtype)
    x_rows, dy_rows, w1, w2 = _c(x_rows, ed), _c(dy_rows, ed), _c(w1, ed), _c(w2, ed)
    w3 = _c(w3, ed)
    offsets = _c(offsets, np.int32)
    E, h, d = w1.shape
    dx = np.zeros((x_rows.shape[0], d), ed)
    dw1 = np.empty((E, h, d), np.float32)
    dw3 = np.empty((E, h, d), np.float32) if act == "swiglu" else None
    dw2 = np.empty((E, d, h), np.float32)
    _check(lib().oracle_expert_ffn_backward(E, d, h, ACT_CODES[act], DTYPE_CODES[dtype],
                                            _ptr(x_rows), _ptr(offsets), _ptr(w1), _ptr(w3),
                                            _ptr(w2), _ptr(dy_rows), _ptr(dx), _ptr(dw1),
                                            _ptr(dw3), _ptr(dw2)), "oracle_expert_ffn_backward")
    return dx, dw1, dw3, dw2


def combine(dtype: str, y_perm, row_of_slot, topk_w, residual=None, shared_out=None):
    ed = _elem_dtype(dtype)
    row_of_slot = _c(row_of_slot, np.int32)
    topk_w = _c(topk_w, np.float32)
    y_perm = _c(y_perm, ed)
    residual, shared_out = _c(residual, ed), _c(shared_out, ed)
    N, k = row_of_slot.shape
    d = (residual if residual is not None else y_perm).shape[1]
    y = np.empty((N, d), ed)
    _check(lib().oracle_combine(N, d, k, DTYPE_CODES[dtype], _ptr(y_perm), _ptr(row_of_slot),
                                _ptr(topk_w), _ptr(residual), _ptr(shared_out), _ptr(y)),
           "oracle_combine")
    return y


def combine_backward(dtype: str, dy, y_perm, row_of_slot, topk_w, num_rows: int) -> tuple:
    """(dy_perm [num_rows, d], dtopk_w [N, k]); rows no slot maps to are zero."""
    ed = _elem_dtype(dtype)
    dy, y_perm = _c(dy, ed), _c(y_perm, ed)
    row_of_slot, topk_w = _c(row_of_slot, np.int32), _c(topk_w, np.float32)
    N, k = row_of_slot.shape
    d = dy.shape[1]
    dy_perm = np.zeros((max(num_rows, 0), d), ed)
    dw = np.empty((N, k), np.float32)
    _check(lib().oracle_combine_backward(N, d, k, DTYPE_CODES[dtype], _ptr(dy), _ptr(y_perm),
                                         _ptr(row_of_slot), _ptr(topk_w), _ptr(dy_perm),
                                         _ptr(dw)), "oracle_combine_backward")
    return dy_perm, dw


def permute_backward(dtype: str, dx_perm, row_of_slot) -> np.ndarray:
    """dx[t] = sum over the token's admitted rows of dx_perm: the combine with
    unit weights and no residual."""
    row_of_slot = _c(row_of_slot, np.int32)
    return combine(dtype, dx_perm, row_of_slot, np.ones(row_of_slot.shape, np.float32))


def router_backward(cfg: dict, x, w_router, z, topk_idx, dtopk_w, counts=None,
                    aux_coef: float = 0.0, dx_in=None) -> dict:
    """Gradients of the router (and of the auxiliary load-balancing loss with
    coefficient aux_coef): dz [N,E] fp32, dw_router [E,d] fp32, db [E] fp32,
    dx [N,d] in the dtype (dx_in added when given), aux_loss (float)."""
    N, d, E, k = cfg["N"], cfg["d"], cfg["E"], cfg["k"]
    et = _elem_dtype(cfg["dtype"])
    desc = _desc(cfg)
    dz = np.zeros((N, E), np.float32)
    dw = np.zeros((E, d), np.float32)
    db = np.zeros(E, np.float32)
    dx = np.zeros((N, d), et)
    loss = ctypes.c_double(0.0)
    cnt = _c(counts, np.int32)
    _check(lib().oracle_router_backward(
        ctypes.byref(desc), _ptr(_c(x, et)), _ptr(_c(w_router, et)), _ptr(_c(z, np.float32)),
        _ptr(_c(topk_idx, np.int32)), _ptr(_c(dtopk_w, np.float32)), _ptr(cnt),
        float(aux_coef), _ptr(_c(dx_in, et)), _ptr(dz), _ptr(dw), _ptr(db), _ptr(dx),
        ctypes.byref(loss)), "oracle_router_backward")
    return {"dz": dz, "dw_router": dw, "db": db, "dx": dx, "aux_loss": loss.value}


def bias_update(num_tokens: int, top_k: int, counts, sel_bias, step: float = 1e-3):
    counts = _c(counts, np.int32)
    b = np.array(sel_bias, dtype=np.float32, copy=True)
    _check(lib().oracle_bias_update(counts.shape[0], int(num_tokens), int(top_k), _ptr(counts),
                                    float(step), _ptr(b)), "oracle_bias_update")
    return b


def quantize_rows_q8(dtype: str, x) -> tuple:
    """Per-row INT8 payload: (q [rows, d] int8, scale [rows] fp32)."""
    ed = _elem_dtype(dtype)
    x = _c(x, ed)
    rows, d = x.shape
    q = np.empty((rows, d), np.int8)
    s = np.empty(rows, np.float32)
    _check(lib().oracle_quantize_rows_q8(int(rows), int(d), DTYPE_CODES[dtype], _ptr(x), _ptr(q),
                                         _ptr(s)), "oracle_quantize_rows_q8")
    return q, s


def dequantize_rows_q8(dtype: str, q, scale) -> np.ndarray:
    q = _c(q, np.int8)
    scale = _c(scale, np.float32)
    rows, d = q.shape
    out = np.empty((rows, d), _elem_dtype(dtype))
    _check(lib().oracle_dequantize_rows_q8(int(rows), int(d), DTYPE_CODES[dtype], _ptr(q),
                                           _ptr(scale), _ptr(out)), "oracle_dequantize_rows_q8")
    return out


def forward(cfg: dict, x, w_router, router_bias, sel_bias, w1, w3, w2,
            shared=None, residual=True) -> dict:
    """The whole layer: route -> dispatch -> permute -> FFN -> combine.
    ``shared`` is an optional (w1, w3, w2) triple of one always-on expert.
    With cfg["payload"] == "int8" the permuted rows travel as the per-token
    INT8 payload (quantised once per token, rows copied, dequantised before
    the FFN); the shared expert and the residual use x itself."""
    r = route(cfg, x, w_router, router_bias, sel_bias)
    dsp = dispatch(cfg, r["topk_idx"])
    M = dsp["num_rows"]
    if cfg.get("payload", "native") == "int8":
        q, sc = quantize_rows_q8(cfg["dtype"], x)
        tor = dsp["token_of_row"][:M]
        live = tor >= 0  # padding rows of the padded layout carry zero codes
        qr = np.zeros((M, q.shape[1]), np.int8)
        sr = np.zeros(M, np.float32)
        qr[live], sr[live] = q[tor[live]], sc[tor[live]]
        x_perm = dequantize_rows_q8(cfg["dtype"], qr, sr)
    else:
        x_perm = permute(cfg["dtype"], x, dsp["token_of_row"], M)
    y_perm = expert_ffn(cfg["dtype"], cfg["act"], x_perm, dsp["expert_offsets"], w1, w3, w2)
    shared_out = None
    if shared is not None:
        sw1, sw3, sw2 = shared
        N = np.asarray(x).shape[0]
        shared_out = expert_ffn(cfg["dtype"], cfg["act"], x, np.array([0, N], np.int32),
                                np.asarray(sw1)[None], None if sw3 is None else np.asarray(sw3)[None],
                                np.asarray(sw2)[None])
    y = combine(cfg["dtype"], y_perm, dsp["row_of_slot"], r["topk_w"],
                np.asarray(x) if residual else None, shared_out)
    out = dict(r)
    out.update(dsp)
    out.update({"x_perm": x_perm, "y_perm": y_perm, "shared_out": shared_out, "y": y})
    return out
