"""The whole MoE-layer forward as a sequence of library calls.

``MoeBuffers`` allocates (with torch) every output and workspace the five
entry points need for one workload; ``prepare_weights`` packs bf16 expert
weights once into the layout the expert FFN reads; ``moe_forward`` enqueues
route -> dispatch -> expert FFN (+ shared expert) -> combine on one stream,
with no host synchronisation.  No arithmetic happens here.
"""

from __future__ import annotations

import torch

from . import (ACT, DTYPE, TORCH_DTYPE, desc_from_workload, fused_combine, moe_bias_update,
               moe_combine,
               admission_flags, moe_dequantize_q8, moe_dispatch, moe_dispatch_ex,
               moe_dispatch_q8, moe_dispatch_rows,
               moe_dispatch_workspace_size, moe_expert_ffn,
               moe_expert_ffn_pack_weights, moe_expert_ffn_pack_weights_t,
               moe_expert_ffn_workspace_size, moe_route,
               moe_route_workspace_size, workspace)


def prepare_weights(cfg: dict, inp: dict, stream=None) -> dict:
    """A shallow copy of the device inputs ``inp`` whose expert weights (w1,
    w3, w2 and the shared expert's) are in the layout ``moe_expert_ffn``
    reads: packed by ``moe_expert_ffn_pack_weights`` for bf16, unchanged for
    fp32.  Done once per set of weights; the layer functions take the result."""
    out = dict(inp)
    out["weights_packed"] = True
    if cfg["dtype"] != "bf16":
        return out

    def pack(w, rows, cols):
        if w is None:
            return None
        wp = torch.empty_like(w)
        moe_expert_ffn_pack_weights(w.shape[0], rows, cols, "bf16", w, wp, stream)
        return wp

    d, h = cfg["d"], cfg["h"]
    out["w1"], out["w3"], out["w2"] = (pack(inp["w1"], h, d), pack(inp.get("w3"), h, d),
                                       pack(inp["w2"], d, h))
    if inp.get("shared") is not None:
        sw1, sw3, sw2 = inp["shared"]
        out["shared"] = (pack(sw1, h, d), pack(sw3, h, d), pack(sw2, d, h))
    return out


def prepare_backward_weights(cfg: dict, inp: dict, stream=None) -> dict:
    """Packed weights of the backward on the grouped GEMM (bf16), from the
    plain row-major w1, w3 [E, h, d] and w2 [E, d, h] of ``inp``: w1, w3 as
    the forward packs them, w2t = W2^T (rows h, cols d) and w13t = [W1^T | W3^T]
    (rows d, cols h or 2h).  Done once per weight update."""
    if cfg["dtype"] != "bf16":
        raise ValueError("the packed backward is bf16 only")
    d, h = cfg["d"], cfg["h"]
    w1, w3, w2 = inp["w1"], inp.get("w3"), inp["w2"]
    E = w1.shape[0]
    out = {}
    for name, w in (("w1", w1), ("w3", w3)):
        if w is None:
            out[name] = None
            continue
        wp = torch.empty_like(w)
        moe_expert_ffn_pack_weights(E, h, d, "bf16", w, wp, stream)
        out[name] = wp
    out["w2t"] = torch.empty(E, h, d, dtype=w2.dtype, device=w2.device)
    moe_expert_ffn_pack_weights_t(E, h, d, d, "bf16", w2, None, out["w2t"], stream)
    kg = 2 * h if w3 is not None else h
    out["w13t"] = torch.empty(E, d, kg, dtype=w1.dtype, device=w1.device)
    moe_expert_ffn_pack_weights_t(E, d, h, kg, "bf16", w1, w3, out["w13t"], stream)
    return out


class MoeBuffers:
    """Device buffers for one workload (N tokens, k slots, E experts, R ranks)."""

    def __init__(self, cfg: dict, device="cuda", N: int | None = None, cf: float | None = None):
        self.cfg = cfg
        self.desc = desc_from_workload(cfg, N=N, cf=cf)
        d = self.desc
        N, E, k, R, dim = d.num_tokens, d.num_experts, d.top_k, d.num_ranks, d.hidden
        S = N * k
        # Admission order and layout as the dispatch's flags; the padded layout
        # (fixed cap rows per expert) lays out max(N*k, E*cap) rows.
        self.flags = admission_flags(cfg.get("admission", "token"), cfg.get("layout", "compact"))
        self.rows = moe_dispatch_rows(d, self.flags)
        S_rows = max(self.rows, 1)
        dt = TORCH_DTYPE[d.dtype]
        i32 = dict(dtype=torch.int32, device=device)
        self.logits = torch.empty(N, E, dtype=torch.float32, device=device)
        self.topk_idx = torch.empty(N, k, **i32)
        self.topk_w = torch.empty(N, k, dtype=torch.float32, device=device)
        self.counts = torch.empty(E, **i32)
        self.ws_route = workspace(moe_route_workspace_size(d), device)
        self.x_perm = torch.empty(S_rows, dim, dtype=dt, device=device)
        # INT8 row payload of the dispatch exchange (workloads with
        # payload="int8"): codes and one scale per row, dequantised into x_perm.
        self.x_perm_q = self.row_scale = None
        if cfg.get("payload", "native") == "int8":
            self.x_perm_q = torch.empty(S_rows, dim, dtype=torch.int8, device=device)
            self.row_scale = torch.empty(S_rows, dtype=torch.float32, device=device)
        self.row_of_slot = torch.empty(N, k, **i32)
        self.token_of_row = torch.empty(S_rows, **i32)
        self.slot_of_row = torch.empty(S_rows, dtype=torch.int8, device=device)
        self.expert_offsets = torch.empty(E + 1, **i32)
        self.admitted = torch.empty(E, **i32)
        self.rank_offsets = torch.empty(R + 1, **i32)
        self.rank_counts = torch.empty(R, **i32)
        self.ws_dispatch = workspace(moe_dispatch_workspace_size(d), device)
        self.y_perm = torch.empty(S_rows, dim, dtype=dt, device=device)
        # Fused combine (workloads with combine="fused"): the down GEMM adds
        # w * O into this fp32 accumulator instead of writing y_perm.
        self.y_acc = None
        if cfg.get("combine", "unfused") == "fused":
            self.y_acc = torch.empty(max(N, 1), dim, dtype=torch.float32, device=device)
        h = cfg["h"]
        self.ws_ffn = workspace(moe_expert_ffn_workspace_size(E, self.rows, dim, h, cfg["act"],
                                                              cfg["dtype"]), device)
        self.shared_out = None
        if cfg.get("shared"):
            self.shared_out = torch.empty(N, dim, dtype=dt, device=device)
            self.shared_offsets = torch.tensor([0, N], **i32)
            # The shared expert needs only x: moe_forward runs it on this
            # stream (default priority) beside the routed path.
            self.side_stream = torch.cuda.Stream(device=device)
            self.ws_shared = workspace(moe_expert_ffn_workspace_size(1, N, dim, h, cfg["act"],
                                                                     cfg["dtype"]), device)
        self.y = torch.empty(N, dim, dtype=dt, device=device)

    def fused_args(self):
        """The down GEMM's fused combine argument (None on the unfused path)."""
        if self.y_acc is None:
            return None
        d = self.desc
        return fused_combine(d.num_tokens, d.top_k, self.topk_w, self.token_of_row,
                             self.slot_of_row, self.y_acc)


def route(buf: MoeBuffers, inp: dict, sel_bias=None, stream=None):
    moe_route(buf.desc, inp["x"], inp["w_router"], inp.get("router_bias"),
              inp.get("sel_bias") if sel_bias is None else sel_bias, buf.logits, buf.topk_idx,
              buf.topk_w, buf.counts, buf.ws_route, stream)


def dispatch(buf: MoeBuffers, inp: dict, stream=None):
    """Admission in token order unless the workload sets ``admission`` to
    ``"first_choice"``; the compact layout unless it sets ``layout`` to
    ``"padded"``.  With ``payload="int8"`` the rows travel as the INT8 payload
    and are dequantised into x_perm (what a receiving rank does)."""
    adm = buf.flags
    if buf.x_perm_q is not None:
        d = buf.desc
        moe_dispatch_q8(d, adm, inp["x"], buf.topk_idx, buf.x_perm_q, buf.row_scale,
                        buf.row_of_slot, buf.token_of_row, buf.slot_of_row, buf.expert_offsets,
                        buf.admitted, buf.rank_offsets, buf.rank_counts, buf.ws_dispatch, stream)
        moe_dequantize_q8(buf.rows, d.hidden, d.dtype, buf.x_perm_q, buf.row_scale,
                          buf.expert_offsets[d.num_experts:], buf.x_perm, stream)
    elif adm == 0:
        moe_dispatch(buf.desc, inp["x"], buf.topk_idx, buf.x_perm, buf.row_of_slot,
                     buf.token_of_row, buf.slot_of_row, buf.expert_offsets, buf.admitted,
                     buf.rank_offsets, buf.rank_counts, buf.ws_dispatch, stream)
    else:
        moe_dispatch_ex(buf.desc, adm, inp["x"], buf.topk_idx, buf.x_perm, buf.row_of_slot,
                        buf.token_of_row, buf.slot_of_row, buf.expert_offsets, buf.admitted,
                        buf.rank_offsets, buf.rank_counts, buf.ws_dispatch, stream)


def routed_ffn(buf: MoeBuffers, inp: dict, stream=None):
    """Every routed expert over its rows.  ``inp`` must come from
    ``prepare_weights`` (packed bf16 weights)."""
    d, cfg = buf.desc, buf.cfg
    if not inp.get("weights_packed"):
        raise ValueError("expert_ffn needs the weights from prepare_weights(cfg, inp)")
    fused = buf.fused_args()
    moe_expert_ffn(d.num_experts, buf.rows, d.hidden, cfg["h"], cfg["act"], cfg["dtype"], buf.x_perm,
                   buf.expert_offsets, inp["w1"], inp.get("w3"), inp["w2"],
                   None if fused is not None else buf.y_perm, fused, buf.ws_ffn, stream)


def has_shared(buf: MoeBuffers, inp: dict) -> bool:
    return buf.shared_out is not None and inp.get("shared") is not None


def shared_ffn(buf: MoeBuffers, inp: dict, stream=None):
    """The shared expert over every token, in token order (x itself)."""
    d, cfg = buf.desc, buf.cfg
    if not inp.get("weights_packed"):
        raise ValueError("expert_ffn needs the weights from prepare_weights(cfg, inp)")
    sw1, sw3, sw2 = inp["shared"]
    moe_expert_ffn(1, d.num_tokens, d.hidden, cfg["h"], cfg["act"], cfg["dtype"], inp["x"],
                   buf.shared_offsets, sw1, sw3, sw2, buf.shared_out, None, buf.ws_shared, stream)


def expert_ffn(buf: MoeBuffers, inp: dict, stream=None):
    """Routed experts, then the shared expert where there is one, on one stream."""
    routed_ffn(buf, inp, stream)
    if has_shared(buf, inp):
        shared_ffn(buf, inp, stream)


def combine(buf: MoeBuffers, inp: dict, residual=True, stream=None):
    moe_combine(buf.desc, buf.y_perm, buf.row_of_slot, buf.topk_w,
                inp["x"] if residual else None, buf.shared_out, buf.y_acc, buf.y, stream)


def bias_update(buf: MoeBuffers, sel_bias: torch.Tensor, step: float, stream=None):
    d = buf.desc
    moe_bias_update(d.num_experts, d.num_tokens, d.top_k, buf.counts, step, sel_bias, stream)


def moe_forward(buf: MoeBuffers, inp: dict, residual=True, stream=None):
    """route -> dispatch -> routed expert FFN -> combine, all enqueued on
    ``stream`` (default: torch's current stream).  A shared expert needs only
    x, so it runs on the buffers' side stream beside the routed path and is
    joined before the combine.  It is forked after the route: the route runs
    alone (with the shared expert beside it, it took 585 instead of 312 us
    on the DeepSeek-like layer), and the shared expert then overlaps the
    dispatch and the routed up GEMM (step 5.60 -> 5.49 ms).  The fork and join
    are stream waits on events, which a HIP graph capture follows."""
    main = stream if stream is not None else torch.cuda.current_stream()
    fork = has_shared(buf, inp)
    route(buf, inp, stream=main)
    if fork:
        buf.side_stream.wait_stream(main)
        shared_ffn(buf, inp, buf.side_stream)
    dispatch(buf, inp, main)
    routed_ffn(buf, inp, main)
    if fork:
        main.wait_stream(buf.side_stream)
    combine(buf, inp, residual, main)
    return buf.y
