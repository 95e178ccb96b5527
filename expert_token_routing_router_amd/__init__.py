"""Python binding of the MI355X MoE-layer forward library (``include/moe.h``).

Argument marshalling only: every function here checks the torch tensors it is
given (device, dtype, shape, contiguity), passes their device pointers and the
current HIP stream to the C ABI of ``libmoe_mi355x.so``, and raises
``MoeError`` on a non-zero status.  All computation happens in the library's
gfx950 kernels; there is no fallback path.  PyTorch only provides device
memory and streams.

Entry points (same names and argument order as the C ABI):
``moe_route``, ``moe_dispatch``, ``moe_expert_ffn`` (and its stages),
``moe_expert_ffn_pack_weights``, ``moe_combine``, ``moe_bias_update``, plus the
``*_workspace_size`` queries.
"""

from __future__ import annotations

import ctypes
import os

import torch

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
# MOE_MI355X_LIB names another build of the same library (e.g. one whose host
# code is compiled with sanitizers); the default is the in-tree build.
LIB_PATH = os.environ.get("MOE_MI355X_LIB") or os.path.join(PKG_DIR, "libmoe_mi355x.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_HIP, MOE_ERR_WORKSPACE = range(5)
MOE_F32, MOE_BF16 = 0, 1
MOE_SOFTMAX_TOPK, MOE_SOFTMAX_ALL, MOE_SIGMOID_NORM = 0, 1, 2
MOE_RELU, MOE_GELU, MOE_SWIGLU = 0, 1, 2
MOE_ADMIT_TOKEN_ORDER, MOE_ADMIT_FIRST_CHOICE, MOE_LAYOUT_PADDED = 0, 1, 2

SCORE = {"softmax_topk": MOE_SOFTMAX_TOPK, "softmax_all": MOE_SOFTMAX_ALL,
         "sigmoid_norm": MOE_SIGMOID_NORM}
ACT = {"relu": MOE_RELU, "gelu": MOE_GELU, "swiglu": MOE_SWIGLU}
DTYPE = {"fp32": MOE_F32, "bf16": MOE_BF16}
ADMISSION = {"token": MOE_ADMIT_TOKEN_ORDER, "first_choice": MOE_ADMIT_FIRST_CHOICE}
TORCH_DTYPE = {MOE_F32: torch.float32, MOE_BF16: torch.bfloat16}

EXPORTS = [
    "moe_route_workspace_size", "moe_route", "moe_router_logits",
    "moe_dispatch_workspace_size", "moe_dispatch", "moe_dispatch_ex", "moe_dispatch_q8",
    "moe_dequantize_q8", "moe_dispatch_layout", "moe_permute", "moe_permute_q8",
    "moe_dispatch_rows", "moe_dispatch_noalloc", "moe_combine_backward", "moe_permute_backward",
    "moe_expert_ffn_backward_workspace_size", "moe_expert_ffn_backward",
    "moe_expert_ffn_backward_packed_workspace_size", "moe_expert_ffn_backward_packed",
    "moe_expert_ffn_pack_weights_t",
    "moe_expert_ffn_workspace_size", "moe_expert_ffn", "moe_expert_ffn_plan",
    "moe_expert_ffn_up", "moe_expert_ffn_down", "moe_expert_ffn_pack_weights", "moe_combine",
    "moe_bias_update", "moe_status_string", "moe_router_backward_workspace_size",
    "moe_router_backward",
]


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: {msg} (status {status})")
        self.status = status


class RouteDesc(ctypes.Structure):
    """Mirror of ``moe_route_desc``."""

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


class FusedCombine(ctypes.Structure):
    """Mirror of ``moe_fused_combine`` (the down GEMM's scatter-add combine)."""

    _fields_ = [
        ("num_tokens", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("topk_w", ctypes.c_void_p),
        ("token_of_row", ctypes.c_void_p),
        ("slot_of_row", ctypes.c_void_p),
        ("y_acc", ctypes.c_void_p),
    ]


def fused_combine(num_tokens, top_k, topk_w, token_of_row, slot_of_row, y_acc) -> FusedCombine:
    """The fused combine argument of ``moe_expert_ffn`` / ``moe_expert_ffn_down``:
    topk_w [N, k] fp32, token_of_row / slot_of_row of the dispatch (int32 /
    int8, one per row), y_acc [N, d] fp32 (zeroed by the FFN call)."""
    N, k = int(num_tokens), int(top_k)
    f = FusedCombine(N, k)
    f.topk_w = _ptr(topk_w, "topk_w", torch.float32, N * k, N > 0)
    f.token_of_row = _ptr(token_of_row, "token_of_row", torch.int32, None, True)
    f.slot_of_row = _ptr(slot_of_row, "slot_of_row", torch.int8, None, True)
    f.y_acc = _ptr(y_acc, "y_acc", torch.float32, None, N > 0)
    return f


def route_desc(N, d, E, k, R=1, cf=0.0, G=1, kg=1, score="softmax_topk", dtype="bf16"):
    return RouteDesc(int(N), int(d), int(E), int(k), int(R), float(cf or 0.0), int(G), int(kg),
                     SCORE[score] if isinstance(score, str) else int(score),
                     DTYPE[dtype] if isinstance(dtype, str) else int(dtype))


def desc_from_workload(cfg: dict, N: int | None = None, cf: float | None = None) -> RouteDesc:
    """Descriptor from a workload dictionary (keys N d E k R cf G kg score dtype)."""
    return route_desc(cfg["N"] if N is None else N, cfg["d"], cfg["E"], cfg["k"],
                      cfg.get("R", 1), cfg.get("cf", 0.0) if cf is None else cf,
                      cfg.get("G", 1), cfg.get("kg", 1), cfg["score"], cfg["dtype"])


_lib = None


def lib() -> ctypes.CDLL:
    """Load the HIP library; fails loudly if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, SZ, F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
        D = ctypes.POINTER(RouteDesc)
        FC = ctypes.POINTER(FusedCombine)
        sigs = {
            "moe_route_workspace_size": ([D], SZ),
            "moe_route": ([D, P, P, P, P, P, P, P, P, P, SZ, P], I32),
            "moe_router_logits": ([D, P, P, P, P, P, SZ, P], I32),
            "moe_dispatch_workspace_size": ([D], SZ),
            "moe_dispatch": ([D, P, P, P, P, P, P, P, P, P, P, P, SZ, P], I32),
            "moe_dispatch_ex": ([D, I32, P, P, P, P, P, P, P, P, P, P, P, SZ, P], I32),
            "moe_dispatch_q8": ([D, I32, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P], I32),
            "moe_dequantize_q8": ([I32, I32, I32, P, P, P, P, P], I32),
            "moe_dispatch_layout": ([D, I32, P, P, P, P, P, P, P, P, P, SZ, P], I32),
            "moe_permute": ([D, P, P, P, P], I32),
            "moe_permute_q8": ([D, P, P, P, P, P], I32),
            "moe_dispatch_rows": ([D, I32], ctypes.c_int64),
            "moe_dispatch_noalloc": ([D, I32, P, P, P, P, P, P, P, P, P, P, P], I32),
            "moe_combine_backward": ([D, P, P, P, P, P, P, P], I32),
            "moe_permute_backward": ([D, P, P, P, P], I32),
            "moe_expert_ffn_backward_workspace_size": ([I32, I32, I32, I32, I32, I32], SZ),
            "moe_expert_ffn_backward": ([I32, I32, I32, I32, I32, I32, P, P, P, P, P, P, P, P, P,
                                         P, P, P, SZ, P], I32),
            "moe_expert_ffn_workspace_size": ([I32, I32, I32, I32, I32, I32], SZ),
            "moe_expert_ffn": ([I32, I32, I32, I32, I32, I32, P, P, P, P, P, P, FC, P, SZ, P],
                               I32),
            "moe_expert_ffn_plan": ([I32, I32, I32, I32, I32, I32, P, P, SZ, P], I32),
            "moe_expert_ffn_up": ([I32, I32, I32, I32, I32, I32, P, P, P, P, P, SZ, P], I32),
            "moe_expert_ffn_down": ([I32, I32, I32, I32, I32, I32, P, P, P, FC, P, SZ, P], I32),
            "moe_expert_ffn_pack_weights": ([I32, I32, I32, I32, P, P, P], I32),
            "moe_expert_ffn_pack_weights_t": ([I32, I32, I32, I32, I32, P, P, P, P], I32),
            "moe_expert_ffn_backward_packed_workspace_size": ([I32, I32, I32, I32, I32, I32], SZ),
            "moe_expert_ffn_backward_packed": ([I32, I32, I32, I32, I32, I32, P, P, P, P, P, P, P,
                                                P, P, P, P, P, P, SZ, P], I32),
            "moe_combine": ([D, P, P, P, P, P, P, P, P], I32),
            "moe_bias_update": ([I32, I32, I32, P, F32, P, P], I32),
            "moe_status_string": ([I32], ctypes.c_char_p),
            "moe_router_backward_workspace_size": ([D], SZ),
            "moe_router_backward": ([D, P, P, P, P, P, P, F32, P, P, P, P, I32, P, P, SZ, P], I32),
        }
        for name, (args, res) in sigs.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().moe_status_string(int(status)).decode()


def _raise(fn: str, status: int):
    if status != MOE_OK:
        raise MoeError(fn, status, status_string(status))


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _ptr(t, name, dtype=None, numel=None, required=True):
    """Device pointer of a contiguous CUDA tensor (None -> NULL)."""
    if t is None:
        if required:
            raise ValueError(f"{name} is required")
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a HIP device, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {numel}")
    return ctypes.c_void_p(t.data_ptr())


def moe_route_workspace_size(desc: RouteDesc) -> int:
    return int(lib().moe_route_workspace_size(ctypes.byref(desc)))


def moe_dispatch_workspace_size(desc: RouteDesc) -> int:
    return int(lib().moe_dispatch_workspace_size(ctypes.byref(desc)))


def moe_expert_ffn_workspace_size(num_experts, max_rows, hidden, ffn_hidden, act, dtype) -> int:
    act = ACT[act] if isinstance(act, str) else int(act)
    dtype = DTYPE[dtype] if isinstance(dtype, str) else int(dtype)
    return int(lib().moe_expert_ffn_workspace_size(num_experts, max_rows, hidden, ffn_hidden,
                                                   act, dtype))


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """Caller-owned scratch buffer (256-byte aligned by the caching allocator)."""
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def moe_route(desc, x, w_router, router_bias, sel_bias, logits, topk_idx, topk_w, counts,
              ws, stream=None):
    N, d, E, k = desc.num_tokens, desc.hidden, desc.num_experts, desc.top_k
    dt = TORCH_DTYPE.get(desc.dtype)
    st = lib().moe_route(
        ctypes.byref(desc), _ptr(x, "x", dt, N * d, N > 0), _ptr(w_router, "w_router", dt, E * d, N > 0),
        _ptr(router_bias, "router_bias", torch.float32, E, False),
        _ptr(sel_bias, "sel_bias", torch.float32, E, False),
        _ptr(logits, "logits", torch.float32, N * E, N > 0),
        _ptr(topk_idx, "topk_idx", torch.int32, N * k, N > 0),
        _ptr(topk_w, "topk_w", torch.float32, N * k, N > 0),
        _ptr(counts, "counts", torch.int32, E),
        _ptr(ws, "ws", None, None, False), 0 if ws is None else ws.numel() * ws.element_size(),
        _stream(stream))
    _raise("moe_route", st)


def moe_router_logits(desc, x, w_router, router_bias, logits, ws, stream=None):
    N, d, E = desc.num_tokens, desc.hidden, desc.num_experts
    dt = TORCH_DTYPE.get(desc.dtype)
    st = lib().moe_router_logits(
        ctypes.byref(desc), _ptr(x, "x", dt, N * d, N > 0),
        _ptr(w_router, "w_router", dt, E * d, N > 0),
        _ptr(router_bias, "router_bias", torch.float32, E, False),
        _ptr(logits, "logits", torch.float32, N * E, N > 0),
        _ptr(ws, "ws", None, None, False), 0 if ws is None else ws.numel() * ws.element_size(),
        _stream(stream))
    _raise("moe_router_logits", st)


def moe_dispatch(desc, x, topk_idx, x_perm, row_of_slot, token_of_row, slot_of_row,
                 expert_offsets, admitted, rank_offsets, rank_counts, ws, stream=None):
    _dispatch("moe_dispatch", desc, None, x, topk_idx, x_perm, row_of_slot, token_of_row,
              slot_of_row, expert_offsets, admitted, rank_offsets, rank_counts, ws, stream)


def moe_dispatch_ex(desc, admission, x, topk_idx, x_perm, row_of_slot, token_of_row,
                    slot_of_row, expert_offsets, admitted, rank_offsets, rank_counts, ws,
                    stream=None):
    """admission: "token" / MOE_ADMIT_TOKEN_ORDER or "first_choice" /
    MOE_ADMIT_FIRST_CHOICE, optionally | MOE_LAYOUT_PADDED (admission_flags());
    with the padded layout the row buffers need moe_dispatch_rows() rows."""
    adm = ADMISSION[admission] if isinstance(admission, str) else int(admission)
    _dispatch("moe_dispatch_ex", desc, adm, x, topk_idx, x_perm, row_of_slot, token_of_row,
              slot_of_row, expert_offsets, admitted, rank_offsets, rank_counts, ws, stream)


def moe_dispatch_q8(desc, admission, x, topk_idx, x_perm_q, row_scale, row_of_slot,
                    token_of_row, slot_of_row, expert_offsets, admitted, rank_offsets,
                    rank_counts, ws, stream=None):
    """Dispatch with the INT8 row payload: x_perm_q [N*k, d] int8 codes and
    row_scale [N*k] fp32 instead of dtype rows."""
    adm = ADMISSION[admission] if isinstance(admission, str) else int(admission)
    N, d, E, k, R = desc.num_tokens, desc.hidden, desc.num_experts, desc.top_k, desc.num_ranks
    dt = TORCH_DTYPE.get(desc.dtype)
    S = N * k
    rows = S if not adm & MOE_LAYOUT_PADDED else moe_dispatch_rows(desc, adm)
    st = lib().moe_dispatch_q8(
        ctypes.byref(desc), adm, _ptr(x, "x", dt, N * d, N > 0),
        _ptr(topk_idx, "topk_idx", torch.int32, S, N > 0),
        _ptr(x_perm_q, "x_perm_q", torch.int8, rows * d, N > 0),
        _ptr(row_scale, "row_scale", torch.float32, rows, N > 0),
        _ptr(row_of_slot, "row_of_slot", torch.int32, S, N > 0),
        _ptr(token_of_row, "token_of_row", torch.int32, rows, N > 0),
        _ptr(slot_of_row, "slot_of_row", torch.int8, rows, N > 0),
        _ptr(expert_offsets, "expert_offsets", torch.int32, E + 1),
        _ptr(admitted, "admitted", torch.int32, E),
        _ptr(rank_offsets, "rank_offsets", torch.int32, R + 1),
        _ptr(rank_counts, "rank_counts", torch.int32, R),
        _ptr(ws, "ws", None, None, False), 0 if ws is None else ws.numel() * ws.element_size(),
        _stream(stream))
    _raise("moe_dispatch_q8", st)


def moe_dispatch_noalloc(desc, admission, x, topk_idx, x_perm, row_of_slot, token_of_row,
                         slot_of_row, expert_offsets, admitted, rank_offsets, rank_counts,
                         stream=None):
    """moe_dispatch_ex without a workspace: the kernels' scratch is the
    library's own static device array (calls on one GPU must not overlap)."""
    adm = ADMISSION[admission] if isinstance(admission, str) else int(admission)
    N, d, E, k, R = desc.num_tokens, desc.hidden, desc.num_experts, desc.top_k, desc.num_ranks
    dt = TORCH_DTYPE.get(desc.dtype)
    S = N * k
    rows = S if not adm & MOE_LAYOUT_PADDED else moe_dispatch_rows(desc, adm)
    st = lib().moe_dispatch_noalloc(
        ctypes.byref(desc), adm, _ptr(x, "x", dt, N * d, N > 0),
        _ptr(topk_idx, "topk_idx", torch.int32, S, N > 0),
        _ptr(x_perm, "x_perm", dt, rows * d, N > 0),
        _ptr(row_of_slot, "row_of_slot", torch.int32, S, N > 0),
        _ptr(token_of_row, "token_of_row", torch.int32, rows, N > 0),
        _ptr(slot_of_row, "slot_of_row", torch.int8, rows, N > 0),
        _ptr(expert_offsets, "expert_offsets", torch.int32, E + 1),
        _ptr(admitted, "admitted", torch.int32, E),
        _ptr(rank_offsets, "rank_offsets", torch.int32, R + 1),
        _ptr(rank_counts, "rank_counts", torch.int32, R), _stream(stream))
    _raise("moe_dispatch_noalloc", st)


def admission_flags(admission="token", layout="compact") -> int:
    """Admission order plus layout as the C flags (strings or ints)."""
    adm = ADMISSION[admission] if isinstance(admission, str) else int(admission)
    return adm | (MOE_LAYOUT_PADDED if layout == "padded" else 0)


def moe_dispatch_rows(desc, admission) -> int:
    """Rows the dispatch lays out (N*k, or max(N*k, E*cap) when padded)."""
    r = int(lib().moe_dispatch_rows(ctypes.byref(desc), int(admission)))
    if r < 0:
        raise ValueError("moe_dispatch_rows: invalid descriptor or admission flags")
    return r


def moe_dispatch_layout(desc, admission, topk_idx, row_of_slot, token_of_row, slot_of_row,
                        expert_offsets, admitted, rank_offsets, rank_counts, ws, stream=None):
    """The layout half of moe_dispatch_ex (no rows are moved)."""
    adm = ADMISSION[admission] if isinstance(admission, str) else int(admission)
    N, E, k, R = desc.num_tokens, desc.num_experts, desc.top_k, desc.num_ranks
    S = N * k
    rows = S if not adm & MOE_LAYOUT_PADDED else moe_dispatch_rows(desc, adm)
    st = lib().moe_dispatch_layout(
        ctypes.byref(desc), adm, _ptr(topk_idx, "topk_idx", torch.int32, S, N > 0),
        _ptr(row_of_slot, "row_of_slot", torch.int32, S, N > 0),
        _ptr(token_of_row, "token_of_row", torch.int32, rows, N > 0),
        _ptr(slot_of_row, "slot_of_row", torch.int8, rows, N > 0),
        _ptr(expert_offsets, "expert_offsets", torch.int32, E + 1),
        _ptr(admitted, "admitted", torch.int32, E),
        _ptr(rank_offsets, "rank_offsets", torch.int32, R + 1),
        _ptr(rank_counts, "rank_counts", torch.int32, R),
        _ptr(ws, "ws", None, None, False), 0 if ws is None else ws.numel() * ws.element_size(),
        _stream(stream))
    _raise("moe_dispatch_layout", st)


def moe_permute(desc, x, row_of_slot, x_perm, stream=None):
    """The permute half of moe_dispatch: x_perm[row_of_slot[t, j]] = x[t]."""
    N, d, k = desc.num_tokens, desc.hidden, desc.top_k
    dt = TORCH_DTYPE.get(desc.dtype)
    st = lib().moe_permute(ctypes.byref(desc), _ptr(x, "x", dt, N * d, N > 0),
                           _ptr(row_of_slot, "row_of_slot", torch.int32, N * k, N > 0),
                           _ptr(x_perm, "x_perm", dt, N * k * d, N > 0), _stream(stream))
    _raise("moe_permute", st)


def moe_permute_q8(desc, x, row_of_slot, x_perm_q, row_scale, stream=None):
    """The permute half of moe_dispatch_q8 (INT8 payload rows and scales)."""
    N, d, k = desc.num_tokens, desc.hidden, desc.top_k
    dt = TORCH_DTYPE.get(desc.dtype)
    st = lib().moe_permute_q8(ctypes.byref(desc), _ptr(x, "x", dt, N * d, N > 0),
                              _ptr(row_of_slot, "row_of_slot", torch.int32, N * k, N > 0),
                              _ptr(x_perm_q, "x_perm_q", torch.int8, N * k * d, N > 0),
                              _ptr(row_scale, "row_scale", torch.float32, N * k, N > 0),
                              _stream(stream))
    _raise("moe_permute_q8", st)


def moe_dequantize_q8(max_rows, hidden, dtype, x_perm_q, row_scale, num_rows, x_perm,
                      stream=None):
    """x_perm[r] = dtype(x_perm_q[r] * row_scale[r]) for r < num_rows[0] (a
    one-element device tensor, e.g. expert_offsets[E:])."""
    dtype = DTYPE[dtype] if isinstance(dtype, str) else int(dtype)
    dt = TORCH_DTYPE.get(dtype)
    M, d = max_rows, hidden
    st = lib().moe_dequantize_q8(
        M, d, dtype, _ptr(x_perm_q, "x_perm_q", torch.int8, M * d, M > 0),
        _ptr(row_scale, "row_scale", torch.float32, M, M > 0),
        _ptr(num_rows, "num_rows", torch.int32, 1, M > 0),
        _ptr(x_perm, "x_perm", dt, M * d, M > 0), _stream(stream))
    _raise("moe_dequantize_q8", st)


def _dispatch(name, desc, admission, x, topk_idx, x_perm, row_of_slot, token_of_row,
              slot_of_row, expert_offsets, admitted, rank_offsets, rank_counts, ws, stream):
    N, d, E, k, R = desc.num_tokens, desc.hidden, desc.num_experts, desc.top_k, desc.num_ranks
    dt = TORCH_DTYPE.get(desc.dtype)
    S = N * k
    adm_flags = admission or 0
    rows = S if not adm_flags & MOE_LAYOUT_PADDED else moe_dispatch_rows(desc, adm_flags)
    fn = getattr(lib(), name)
    head = (ctypes.byref(desc),) if admission is None else (ctypes.byref(desc), admission)
    st = fn(
        *head, _ptr(x, "x", dt, N * d, N > 0),
        _ptr(topk_idx, "topk_idx", torch.int32, S, N > 0),
        _ptr(x_perm, "x_perm", dt, rows * d, N > 0),
        _ptr(row_of_slot, "row_of_slot", torch.int32, S, N > 0),
        _ptr(token_of_row, "token_of_row", torch.int32, rows, N > 0),
        _ptr(slot_of_row, "slot_of_row", torch.int8, rows, N > 0),
        _ptr(expert_offsets, "expert_offsets", torch.int32, E + 1),
        _ptr(admitted, "admitted", torch.int32, E),
        _ptr(rank_offsets, "rank_offsets", torch.int32, R + 1),
        _ptr(rank_counts, "rank_counts", torch.int32, R),
        _ptr(ws, "ws", None, None, False), 0 if ws is None else ws.numel() * ws.element_size(),
        _stream(stream))
    _raise(name, st)


def _fused_ref(fused):
    return None if fused is None else ctypes.byref(fused)


def moe_expert_ffn(num_experts, max_rows, hidden, ffn_hidden, act, dtype, x_rows,
                   group_offsets, w1, w3, w2, y_rows, fused, ws, stream=None):
    """fused: None, or ``fused_combine(...)`` (then y_rows may be None)."""
    act = ACT[act] if isinstance(act, str) else int(act)
    dtype = DTYPE[dtype] if isinstance(dtype, str) else int(dtype)
    dt = TORCH_DTYPE.get(dtype)
    E, M, d, h = num_experts, max_rows, hidden, ffn_hidden
    st = lib().moe_expert_ffn(
        E, M, d, h, act, dtype, _ptr(x_rows, "x_rows", dt, M * d, M > 0),
        _ptr(group_offsets, "group_offsets", torch.int32, E + 1),
        _ptr(w1, "w1", dt, E * h * d), _ptr(w3, "w3", dt, E * h * d, act == MOE_SWIGLU),
        _ptr(w2, "w2", dt, E * d * h),
        _ptr(y_rows, "y_rows", dt, M * d, M > 0 and fused is None), _fused_ref(fused),
        _ptr(ws, "ws", None, None, False), 0 if ws is None else ws.numel() * ws.element_size(),
        _stream(stream))
    _raise("moe_expert_ffn", st)


def moe_expert_ffn_pack_weights(num_experts, rows, cols, dtype, w, w_packed, stream=None):
    """Pack a bf16 [E, rows, cols] expert weight tensor into ``w_packed``
    (same size) in the layout the bf16 expert FFN reads (``include/moe.h``)."""
    dtype = DTYPE[dtype] if isinstance(dtype, str) else int(dtype)
    dt = TORCH_DTYPE.get(dtype)
    n = num_experts * rows * cols
    st = lib().moe_expert_ffn_pack_weights(num_experts, rows, cols, dtype, _ptr(w, "w", dt, n),
                                           _ptr(w_packed, "w_packed", dt, n), _stream(stream))
    _raise("moe_expert_ffn_pack_weights", st)


def moe_expert_ffn_pack_weights_t(num_experts, rows, cols_a, cols, dtype, wa, wb, w_packed,
                                  stream=None):
    """Pack the [E, rows, cols] matrix [wa^T | wb^T] (wa [E, cols_a, rows],
    wb [E, cols - cols_a, rows] or None when cols_a == cols) into ``w_packed``
    in the expert FFN's packed layout (the backward's W2^T and [W1^T | W3^T])."""
    dtype = DTYPE[dtype] if isinstance(dtype, str) else int(dtype)
    dt = TORCH_DTYPE.get(dtype)
    E = num_experts
    st = lib().moe_expert_ffn_pack_weights_t(
        E, rows, cols_a, cols, dtype, _ptr(wa, "wa", dt, E * cols_a * rows),
        _ptr(wb, "wb", dt, E * (cols - cols_a) * rows, cols_a < cols),
        _ptr(w_packed, "w_packed", dt, E * rows * cols), _stream(stream))
    _raise("moe_expert_ffn_pack_weights_t", st)


def _ws(ws):
    return (_ptr(ws, "ws", None, None, False),
            0 if ws is None else ws.numel() * ws.element_size())


def moe_expert_ffn_plan(num_experts, max_rows, hidden, ffn_hidden, act, dtype, group_offsets,
                        ws, stream=None):
    act = ACT[act] if isinstance(act, str) else int(act)
    dtype = DTYPE[dtype] if isinstance(dtype, str) else int(dtype)
    st = lib().moe_expert_ffn_plan(
        num_experts, max_rows, hidden, ffn_hidden, act, dtype,
        _ptr(group_offsets, "group_offsets", torch.int32, num_experts + 1), *_ws(ws),
        _stream(stream))
    _raise("moe_expert_ffn_plan", st)


def moe_expert_ffn_up(num_experts, max_rows, hidden, ffn_hidden, act, dtype, x_rows,
                      group_offsets, w1, w3, ws, stream=None):
    act = ACT[act] if isinstance(act, str) else int(act)
    dtype = DTYPE[dtype] if isinstance(dtype, str) else int(dtype)
    dt = TORCH_DTYPE.get(dtype)
    E, M, d, h = num_experts, max_rows, hidden, ffn_hidden
    st = lib().moe_expert_ffn_up(
        E, M, d, h, act, dtype, _ptr(x_rows, "x_rows", dt, M * d, M > 0),
        _ptr(group_offsets, "group_offsets", torch.int32, E + 1),
        _ptr(w1, "w1", dt, E * h * d), _ptr(w3, "w3", dt, E * h * d, act == MOE_SWIGLU),
        *_ws(ws), _stream(stream))
    _raise("moe_expert_ffn_up", st)


def moe_expert_ffn_down(num_experts, max_rows, hidden, ffn_hidden, act, dtype, group_offsets,
                        w2, y_rows, fused, ws, stream=None):
    """fused: None, or ``fused_combine(...)`` (then y_rows may be None)."""
    act = ACT[act] if isinstance(act, str) else int(act)
    dtype = DTYPE[dtype] if isinstance(dtype, str) else int(dtype)
    dt = TORCH_DTYPE.get(dtype)
    E, M, d, h = num_experts, max_rows, hidden, ffn_hidden
    st = lib().moe_expert_ffn_down(
        E, M, d, h, act, dtype, _ptr(group_offsets, "group_offsets", torch.int32, E + 1),
        _ptr(w2, "w2", dt, E * d * h),
        _ptr(y_rows, "y_rows", dt, M * d, M > 0 and fused is None), _fused_ref(fused),
        *_ws(ws), _stream(stream))
    _raise("moe_expert_ffn_down", st)


def moe_combine(desc, y_perm, row_of_slot, topk_w, residual, shared_out, y_acc, y, stream=None):
    """y_acc: None, or the fp32 accumulator a fused down GEMM filled (then
    y_perm, row_of_slot and topk_w are not read and may be None)."""
    N, d, k = desc.num_tokens, desc.hidden, desc.top_k
    dt = TORCH_DTYPE.get(desc.dtype)
    unfused = N > 0 and y_acc is None
    st = lib().moe_combine(
        ctypes.byref(desc), _ptr(y_perm, "y_perm", dt, None, unfused),
        _ptr(row_of_slot, "row_of_slot", torch.int32, N * k, unfused),
        _ptr(topk_w, "topk_w", torch.float32, N * k, unfused),
        _ptr(residual, "residual", dt, N * d, False),
        _ptr(shared_out, "shared_out", dt, N * d, False),
        _ptr(y_acc, "y_acc", torch.float32, N * d, False),
        _ptr(y, "y", dt, N * d, N > 0), _stream(stream))
    _raise("moe_combine", st)


def moe_combine_backward(desc, dy, y_perm, row_of_slot, topk_w, dy_perm, dtopk_w,
                         num_rows=None, stream=None):
    """dy_perm[r] = w * dy[t] and dtopk_w[t, j] = <dy[t], y_perm[r]> for every
    admitted slot (backward of the combine's expert terms)."""
    N, d, k = desc.num_tokens, desc.hidden, desc.top_k
    dt = TORCH_DTYPE.get(desc.dtype)
    rows = N * k if num_rows is None else num_rows
    st = lib().moe_combine_backward(
        ctypes.byref(desc), _ptr(dy, "dy", dt, N * d, N > 0),
        _ptr(y_perm, "y_perm", dt, rows * d, N > 0),
        _ptr(row_of_slot, "row_of_slot", torch.int32, N * k, N > 0),
        _ptr(topk_w, "topk_w", torch.float32, N * k, N > 0),
        _ptr(dy_perm, "dy_perm", dt, rows * d, N > 0),
        _ptr(dtopk_w, "dtopk_w", torch.float32, N * k, N > 0), _stream(stream))
    _raise("moe_combine_backward", st)


def moe_permute_backward(desc, dx_perm, row_of_slot, dx, num_rows=None, stream=None):
    """dx[t] = sum of the token's admitted rows of dx_perm (adjoint of the permute)."""
    N, d, k = desc.num_tokens, desc.hidden, desc.top_k
    dt = TORCH_DTYPE.get(desc.dtype)
    rows = N * k if num_rows is None else num_rows
    st = lib().moe_permute_backward(
        ctypes.byref(desc), _ptr(dx_perm, "dx_perm", dt, rows * d, N > 0),
        _ptr(row_of_slot, "row_of_slot", torch.int32, N * k, N > 0),
        _ptr(dx, "dx", dt, N * d, N > 0), _stream(stream))
    _raise("moe_permute_backward", st)


def moe_expert_ffn_backward_workspace_size(num_experts, max_rows, hidden, ffn_hidden, act,
                                           dtype) -> int:
    act = ACT[act] if isinstance(act, str) else int(act)
    dtype = DTYPE[dtype] if isinstance(dtype, str) else int(dtype)
    return int(lib().moe_expert_ffn_backward_workspace_size(num_experts, max_rows, hidden,
                                                             ffn_hidden, act, dtype))


def moe_expert_ffn_backward(num_experts, max_rows, hidden, ffn_hidden, act, dtype, x_rows,
                            group_offsets, group_rows, w1, w3, w2, dy_rows, dx_rows, dw1, dw3,
                            dw2, ws, stream=None):
    """Input gradients dx_rows and fp32 weight gradients dw1/dw3/dw2 of the
    grouped expert FFN; weights in plain row-major layout (not packed).
    group_rows: None, or [E] int32 rows of each segment that hold data (the
    dispatch's admitted for the padded layout)."""
    act = ACT[act] if isinstance(act, str) else int(act)
    dtype = DTYPE[dtype] if isinstance(dtype, str) else int(dtype)
    dt = TORCH_DTYPE.get(dtype)
    E, M, d, h = num_experts, max_rows, hidden, ffn_hidden
    sw = act == MOE_SWIGLU
    f32 = torch.float32
    st = lib().moe_expert_ffn_backward(
        E, M, d, h, act, dtype, _ptr(x_rows, "x_rows", dt, M * d, M > 0),
        _ptr(group_offsets, "group_offsets", torch.int32, E + 1),
        _ptr(group_rows, "group_rows", torch.int32, E, False),
        _ptr(w1, "w1", dt, E * h * d), _ptr(w3, "w3", dt, E * h * d, sw),
        _ptr(w2, "w2", dt, E * d * h), _ptr(dy_rows, "dy_rows", dt, M * d, M > 0),
        _ptr(dx_rows, "dx_rows", dt, M * d, M > 0), _ptr(dw1, "dw1", f32, E * h * d),
        _ptr(dw3, "dw3", f32, E * h * d, sw), _ptr(dw2, "dw2", f32, E * d * h),
        _ptr(ws, "ws", None, None, False), 0 if ws is None else ws.numel() * ws.element_size(),
        _stream(stream))
    _raise("moe_expert_ffn_backward", st)


def moe_expert_ffn_backward_packed_workspace_size(num_experts, max_rows, hidden, ffn_hidden,
                                                  act, dtype) -> int:
    act = ACT[act] if isinstance(act, str) else int(act)
    dtype = DTYPE[dtype] if isinstance(dtype, str) else int(dtype)
    return int(lib().moe_expert_ffn_backward_packed_workspace_size(num_experts, max_rows, hidden,
                                                                    ffn_hidden, act, dtype))


def moe_expert_ffn_backward_packed(num_experts, max_rows, hidden, ffn_hidden, act, dtype, x_rows,
                                   group_offsets, group_rows, w1_packed, w3_packed, w2t_packed,
                                   w13t_packed, dy_rows, dx_rows, dw1, dw3, dw2, ws,
                                   stream=None):
    """moe_expert_ffn_backward on the forward's grouped GEMM: w1/w3 packed as
    for moe_expert_ffn, w2t_packed and w13t_packed from
    moe_expert_ffn_pack_weights_t (see prepare_backward_weights)."""
    act = ACT[act] if isinstance(act, str) else int(act)
    dtype = DTYPE[dtype] if isinstance(dtype, str) else int(dtype)
    dt = TORCH_DTYPE.get(dtype)
    E, M, d, h = num_experts, max_rows, hidden, ffn_hidden
    sw = act == MOE_SWIGLU
    kg = 2 * h if sw else h
    f32 = torch.float32
    st = lib().moe_expert_ffn_backward_packed(
        E, M, d, h, act, dtype, _ptr(x_rows, "x_rows", dt, M * d, M > 0),
        _ptr(group_offsets, "group_offsets", torch.int32, E + 1),
        _ptr(group_rows, "group_rows", torch.int32, E, False),
        _ptr(w1_packed, "w1_packed", dt, E * h * d), _ptr(w3_packed, "w3_packed", dt, E * h * d, sw),
        _ptr(w2t_packed, "w2t_packed", dt, E * h * d), _ptr(w13t_packed, "w13t_packed", dt, E * d * kg),
        _ptr(dy_rows, "dy_rows", dt, M * d, M > 0), _ptr(dx_rows, "dx_rows", dt, M * d, M > 0),
        _ptr(dw1, "dw1", f32, E * h * d), _ptr(dw3, "dw3", f32, E * h * d, sw),
        _ptr(dw2, "dw2", f32, E * d * h), *_ws(ws), _stream(stream))
    _raise("moe_expert_ffn_backward_packed", st)


def moe_router_backward_workspace_size(desc: RouteDesc) -> int:
    return int(lib().moe_router_backward_workspace_size(ctypes.byref(desc)))


def moe_router_backward(desc, x, w_router, logits, topk_idx, dtopk_w, counts, aux_coef, dlogits,
                        dw_router, drouter_bias, dx, accumulate_dx, aux_loss, ws, stream=None):
    """Gradients of the router and of the auxiliary load-balancing loss
    (include/moe.h): dlogits [N,E] (nullable), dw_router [E,d] fp32,
    drouter_bias [E] (nullable), dx [N,d] (nullable; added to when
    accumulate_dx), aux_loss one-element fp32 tensor (nullable)."""
    N, d, E, k = desc.num_tokens, desc.hidden, desc.num_experts, desc.top_k
    dt = TORCH_DTYPE.get(desc.dtype)
    f32 = torch.float32
    st = lib().moe_router_backward(
        ctypes.byref(desc), _ptr(x, "x", dt, N * d, N > 0),
        _ptr(w_router, "w_router", dt, E * d, N > 0),
        _ptr(logits, "logits", f32, N * E, N > 0),
        _ptr(topk_idx, "topk_idx", torch.int32, N * k, N > 0),
        _ptr(dtopk_w, "dtopk_w", f32, N * k, N > 0),
        _ptr(counts, "counts", torch.int32, E, bool(aux_coef)), float(aux_coef),
        _ptr(dlogits, "dlogits", f32, N * E, False), _ptr(dw_router, "dw_router", f32, E * d),
        _ptr(drouter_bias, "drouter_bias", f32, E, False), _ptr(dx, "dx", dt, N * d, False),
        int(bool(accumulate_dx)), _ptr(aux_loss, "aux_loss", f32, 1, False),
        _ptr(ws, "ws", None, None, False), 0 if ws is None else ws.numel() * ws.element_size(),
        _stream(stream))
    _raise("moe_router_backward", st)


def moe_bias_update(num_experts, num_tokens, top_k, counts, step, sel_bias, stream=None):
    st = lib().moe_bias_update(
        int(num_experts), int(num_tokens), int(top_k),
        _ptr(counts, "counts", torch.int32, num_experts),
        float(step), _ptr(sel_bias, "sel_bias", torch.float32, num_experts), _stream(stream))
    _raise("moe_bias_update", st)


from .layer import (MoeBuffers, moe_forward, prepare_backward_weights,  # noqa: E402,F401
                    prepare_weights)  # composition of the calls above
