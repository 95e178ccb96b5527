#!/usr/bin/env python3
"""MoE-layer forward throughput on one MI355X.

One step is one pass of the whole hot path over one batch of synthetic input,
already resident in HBM: route -> dispatch -> expert FFN (plan, up, down; plus
the shared expert where the workload has one) -> combine -> selection-bias
update.  Default workload: Switch-style top-1, N=16384 tokens, d=1024, 64
experts, softmax over all 64, capacity factor 1.25 (cap 320, token-order
admission), GELU experts 1024->4096->1024, 8 simulated EP ranks, bf16.

Prints one JSON line.  Every library call inside the timed region is bracketed
by HIP events on the stream it is launched on; the per-call averages give the
roofline of the dominant kernel and the per-step breakdown.  Two more passes
give the step-time percentiles (one event per step) and the cold-cache per-call
times (a 512 MiB write before each step evicts the Infinity Cache and the L2s).  The CPU oracle is
timed on a bounded sample of the same workload (``cpu_baseline``).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE layer tokens/sec at 1 GPU; grouped-GEMM % MFMA peak; permute % HBM BW"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp32": 157.3}  # dense, published
PROFILE_DIR = os.path.join(ROOT, "profiles")


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="switch",
                    choices=["toy", "switch", "mixtral", "deepseek", "zipf", "decode"])
    ap.add_argument("--cf", type=float, default=None, help="override the capacity factor")
    ap.add_argument("--admission", default="token", choices=["token", "first_choice"],
                    help="capacity admission order: token order, or every token's first "
                         "choice before any second choice")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target length of the oracle's timed sample")
    ap.add_argument("--layout", default="compact", choices=["compact", "padded"],
                    help="dispatch layout: compact rows, or fixed buffers of cap rows per "
                         "expert (the FFN then runs every row of them)")
    ap.add_argument("--payload", default="native", choices=["native", "int8"],
                    help="dispatched rows as the layer dtype, or as the INT8 payload "
                         "(quantised in the permute, dequantised before the FFN)")
    ap.add_argument("--no-clocks", action="store_true",
                    help="skip reading the clocks with rocm-smi (a child process; under a "
                         "profiler that has already initialised the GPU, leave it out)")
    ap.add_argument("--backward", action="store_true",
                    help="also time the data path's backward (moe_combine_backward, "
                         "moe_permute_backward) on this workload's layout")
    ap.add_argument("--rank-share", action="store_true",
                    help="also time the expert FFN on one rank's share of the experts at "
                         "its real shape (rows from all R source ranks)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run one device copy of this size (counter calibration)")
    return ap.parse_args()


def kernel_sources_digest() -> str:
    """Digest of the HIP sources the measured kernels are built from."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "expert_token_routing_router_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(kernel: str, workload: str, digest: str):
    """HBM bytes per launch from the committed counter summary, or None if it is
    missing or was taken from different kernel sources."""
    path = os.path.join(PROFILE_DIR, f"{kernel}_{workload}_pmc.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_sources_digest") != digest:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def read_clocks() -> dict:
    """Current clocks from rocm-smi, if it answers within a few seconds.  Runs
    before this process initialises the GPU."""
    info = {}
    try:
        import subprocess
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True,
                           text=True, timeout=20)
        card = next(iter(json.loads(r.stdout).values()))
        for key, val in card.items():
            kl = key.lower()
            if "sclk" in kl or "mclk" in kl:
                info[key] = val
    except Exception as exc:  # clocks are context, never a reason to fail
        info["clocks"] = f"unavailable ({type(exc).__name__})"
    return info


def rank_share(moe, torch, cfg, buf, wts, steps: int) -> dict:
    """The expert FFN on one rank's share at its real shape: rank 0's E/R local
    experts, each receiving rows from all R source ranks.  The receive buffer is
    this batch's rows for those experts repeated R times (each source rank sends
    its own tokens' rows; the repeat gives the same row count and shapes)."""
    d = buf.desc
    E, R, dim, h = d.num_experts, d.num_ranks, d.hidden, cfg["h"]
    El = E // R
    dev = buf.x_perm.device
    off = buf.expert_offsets.cpu().tolist()
    chunks = [buf.x_perm[off[e]:off[e + 1]].repeat(R, 1) for e in range(El)]
    rows = [c.shape[0] for c in chunks]
    recv = torch.cat(chunks)
    M = recv.shape[0]
    goff = torch.zeros(El + 1, dtype=torch.int32)
    goff[1:] = torch.cumsum(torch.tensor(rows, dtype=torch.int32), 0)
    goff = goff.to(dev)
    w1 = wts["w1"][:El]
    w3 = wts["w3"][:El] if wts.get("w3") is not None else None
    w2 = wts["w2"][:El]
    y = torch.empty_like(recv)
    ws = moe.workspace(moe.moe_expert_ffn_workspace_size(El, M, dim, h, cfg["act"], cfg["dtype"]),
                       device=dev)

    def run():
        moe.moe_expert_ffn(El, M, dim, h, cfg["act"], cfg["dtype"], recv, goff, w1, w3, w2, y, ws)

    for _ in range(3):
        run()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    ev[0].record()
    for _ in range(steps):
        run()
    ev[1].record()
    torch.cuda.synchronize()
    us = ev[0].elapsed_time(ev[1]) / steps * 1e3
    es = 2 if cfg["dtype"] == "bf16" else 4
    mats_up = 2 if cfg["act"] == "swiglu" else 1
    flops = 2.0 * M * dim * h * (mats_up + 1)
    nbytes = (El * (mats_up + 1) * h * dim + 2 * M * dim) * es
    peak = MFMA_PEAK_TFLOPS[cfg["dtype"]]
    # Each output row depends only on its input row and the expert's weights,
    # so every copy must equal the layer step's own output for that row.
    same = all(torch.equal(y[int(goff[e]) + c * (rows[e] // R):int(goff[e]) + (c + 1) * (rows[e] // R)],
                           buf.y_perm[off[e]:off[e + 1]])
               for e in range(El) for c in range(R))
    return {"local_experts": El, "rows": M, "rows_per_expert": rows, "us": round(us, 1),
            "rows_equal_layer_output": bool(same),
            "tflops": round(flops / (us * 1e-6) / 1e12, 1),
            "mfma_frac": round(flops / (us * 1e-6) / (peak * 1e12), 4),
            "hbm_frac": round(nbytes / (us * 1e-6) / (HBM_PEAK_GBS * 1e9), 4),
            "bound": "mfma" if flops / (peak * 1e12) >= nbytes / (HBM_PEAK_GBS * 1e9) else "hbm"}


def backward_pass(moe, torch, buf, inp, steps: int) -> dict:
    """The layer's backward on its last layout: the combine's expert terms
    (row and weight gradients), the expert FFN's backward (input and weight
    gradients, bf16) and the permute's adjoint, timed with events; per call,
    the algorithmic bytes (data path) or FLOPs (FFN) over the time."""
    d = buf.desc
    N, k, dim = d.num_tokens, d.top_k, d.hidden
    dev = buf.y.device
    dt = buf.y.dtype
    es = buf.y.element_size()
    M = int(buf.expert_offsets[d.num_experts].item())
    g = torch.Generator(device=dev).manual_seed(7)
    dy = torch.randn(N, dim, generator=g, device=dev).to(dt)
    dy_perm = torch.empty_like(buf.y_perm)
    dw = torch.empty(N, k, dtype=torch.float32, device=dev)
    dx = torch.empty(N, dim, dtype=dt, device=dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    cb = pb = 0.0

    def run():
        moe.moe_combine_backward(d, dy, buf.y_perm, buf.row_of_slot, buf.topk_w, dy_perm, dw,
                                 num_rows=buf.rows)
        moe.moe_permute_backward(d, dy_perm, buf.row_of_slot, dx, num_rows=buf.rows)

    for _ in range(3):
        run()
    torch.cuda.synchronize()
    for _ in range(steps):
        ev[0].record()
        moe.moe_combine_backward(d, dy, buf.y_perm, buf.row_of_slot, buf.topk_w, dy_perm, dw,
                                 num_rows=buf.rows)
        ev[1].record()
        moe.moe_permute_backward(d, dy_perm, buf.row_of_slot, dx, num_rows=buf.rows)
        ev[2].record()
        torch.cuda.synchronize()
        cb += ev[0].elapsed_time(ev[1])
        pb += ev[1].elapsed_time(ev[2])
    cb, pb = cb / steps * 1e3, pb / steps * 1e3
    S = N * k
    cb_bytes = N * dim * es + 2 * M * dim * es + S * 12  # dy, y_perm rows, dy_perm rows
    pb_bytes = M * dim * es + N * dim * es + S * 4       # dx_perm rows, dx
    frac = lambda nb, us: round(nb / (us * 1e-6) / (HBM_PEAK_GBS * 1e9), 4)
    out = {"combine_backward": {"us": round(cb, 2), "hbm_frac": frac(cb_bytes, cb)},
           "permute_backward": {"us": round(pb, 2), "hbm_frac": frac(pb_bytes, pb)}}
    cfg = buf.cfg
    if cfg["dtype"] != "bf16":
        return out
    # Expert FFN backward over the admitted rows, plain row-major weights.
    E, h, act = d.num_experts, cfg["h"], cfg["act"]
    w1, w3, w2 = inp["w1"], inp.get("w3"), inp["w2"]
    sw = act == "swiglu"
    dx_perm = torch.empty_like(buf.x_perm)
    dw1 = torch.empty(E, h, dim, dtype=torch.float32, device=dev)
    dw3 = torch.empty(E, h, dim, dtype=torch.float32, device=dev) if sw else None
    dw2 = torch.empty(E, dim, h, dtype=torch.float32, device=dev)
    ws = moe.workspace(moe.moe_expert_ffn_backward_workspace_size(E, buf.rows, dim, h, act, "bf16"),
                       dev)

    def ffn_bwd():
        moe.moe_expert_ffn_backward(E, buf.rows, dim, h, act, "bf16", buf.x_perm,
                                    buf.expert_offsets, w1, w3, w2, dy_perm, dx_perm, dw1, dw3,
                                    dw2, ws)

    for _ in range(2):
        ffn_bwd()
    torch.cuda.synchronize()
    fb = 0.0
    for _ in range(steps):
        ev[0].record()
        ffn_bwd()
        ev[1].record()
        torch.cuda.synchronize()
        fb += ev[0].elapsed_time(ev[1])
    fb = fb / steps * 1e3
    # Products per row: u (and v) and g over d, dx over h (2h), the weight
    # gradients over the rows: 2 d h FLOPs each.
    n_mm = 7 if sw else 4
    flops = 2.0 * M * dim * h * n_mm
    grad_bytes = (3 if sw else 2) * E * h * dim * 4  # fp32 weight gradients written
    out["ffn_backward"] = {
        "us": round(fb, 2), "tflops": round(flops / (fb * 1e-6) / 1e12, 1),
        "mfma_frac": round(flops / (fb * 1e-6) / (MFMA_PEAK_TFLOPS["bf16"] * 1e12), 4),
        "weight_grad_bytes": grad_bytes}
    return out


def describe(cfg) -> str:
    s = (f"{cfg['name']} N={cfg['N']} d={cfg['d']} h={cfg['h']} E={cfg['E']} k={cfg['k']} "
         f"score={cfg['score']} act={cfg['act']} R={cfg['R']}")
    if cfg.get("cf"):
        s += f" cf={cfg['cf']}"
    if cfg.get("G", 1) > 1:
        s += f" groups={cfg['G']}/keep{cfg['kg']}"
    if cfg.get("shared"):
        s += " +shared"
    if cfg.get("admission", "token") != "token":
        s += f" admission={cfg['admission']}"
    if cfg.get("payload", "native") != "native":
        s += f" payload={cfg['payload']}"
    if cfg.get("layout", "compact") != "compact":
        s += f" layout={cfg['layout']}"
    return s


def cpu_baseline(cfg, inp, target_s: float) -> dict:
    """Time the oracle (as it stands) on the first T tokens of the workload,
    taken as a batch of T (capacity recomputed for T): route, dispatch, FFN,
    combine and bias update.  T is chosen so the run lasts about target_s."""
    import numpy as np

    import moe_workloads as W
    import oracle

    threads = max(1, min(16, os.cpu_count() or 1))
    oracle.set_threads(threads)
    n = W.to_numpy
    wr, rb = n(inp["w_router"]), n(inp["router_bias"])
    sb = n(inp["sel_bias"])
    bias_state = sb if sb is not None else np.zeros(cfg["E"], np.float32)
    w1, w3, w2 = n(inp["w1"]), n(inp["w3"]), n(inp["w2"])
    shared = None
    if inp.get("shared") is not None:
        shared = tuple(None if t is None else n(t[0]) for t in inp["shared"])
    x_all = inp["x"]

    def run(T):
        c = dict(cfg)
        c["N"] = T
        x = n(x_all[:T])
        t0 = time.perf_counter()
        out = oracle.forward(c, x, wr, rb, sb, w1, w3, w2, shared=shared)
        oracle.bias_update(T, c["k"], out["counts"], bias_state, cfg.get("bias_step", 1e-3))
        return time.perf_counter() - t0

    # Grow the sample until it lasts about target_s (the oracle's per-token
    # cost falls as rows per expert grow and its threads fill up).
    T = min(cfg["N"], 64)
    elapsed = run(T)
    for _ in range(4):
        if elapsed >= target_s / 2 or T >= cfg["N"]:
            break
        T = int(min(cfg["N"], max(2 * T, T * target_s / max(elapsed, 1e-6))))
        elapsed = run(T)
    out = {"value": T / elapsed, "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": f"first {T} of {cfg['N']} tokens as one batch (capacity for {T}); "
                     f"route+dispatch+FFN+combine+bias update; {elapsed:.1f} s"}

    # The same on one thread, the plain loops as written, on a smaller sample.
    oracle.set_threads(1)
    T1 = min(cfg["N"], 16)
    e1 = run(T1)
    for _ in range(4):
        if e1 >= target_s / 4 or T1 >= cfg["N"]:
            break
        T1 = int(min(cfg["N"], max(2 * T1, T1 * (target_s / 2) / max(e1, 1e-6))))
        e1 = run(T1)
    oracle.set_threads(threads)
    out["single_thread"] = {"value": T1 / e1, "unit": "tokens/s", "cores": 1,
                            "sample": f"first {T1} of {cfg['N']} tokens as one batch; {e1:.1f} s"}
    return out


def main():
    args = parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    clocks = {} if args.no_clocks else read_clocks()
    import torch

    import expert_token_routing_router_amd as moe
    from expert_token_routing_router_amd import layer
    import moe_workloads as W

    dev = torch.device("cuda:0")
    cfg = W.full(args.workload)
    if args.cf is not None:
        cfg["cf"] = args.cf
    if args.admission != "token":
        cfg["admission"] = args.admission
    if args.payload != "native":
        cfg["payload"] = args.payload
    if args.layout != "compact":
        cfg["layout"] = args.layout
    # Inputs: the glossary snippet's stream for the toy workload (CPU), else
    # drawn on the device.
    gen_dev = "cpu" if args.workload == "toy" else "cuda"
    inp_src = W.make_inputs(cfg, device=gen_dev)
    inp = {k: (tuple(None if t is None else t.to(dev) for t in v) if isinstance(v, tuple)
               else (v.to(dev) if isinstance(v, torch.Tensor) else v))
           for k, v in inp_src.items()}
    buf = moe.MoeBuffers(cfg, dev)
    # bf16 expert weights are packed once, as a model load would, before any
    # timed work.
    wts = moe.prepare_weights(cfg, inp)
    d = buf.desc
    N, E, k, dim, h = d.num_tokens, d.num_experts, d.top_k, d.hidden, cfg["h"]
    S = N * k
    bias_state = (inp["sel_bias"].clone() if inp.get("sel_bias") is not None
                  else torch.zeros(E, dtype=torch.float32, device=dev))
    step_bias = cfg.get("bias_step", 1e-3)

    # Calls on the main stream, in order.  A shared expert (needs only x) is
    # forked onto a side stream at the start of the step and joined before
    # the combine, as the layer's forward does; it is timed by its own pair
    # of events on that stream.
    # Dispatch runs as its two halves (moe_dispatch_layout, then moe_permute or
    # the INT8 payload's moe_permute_q8 + moe_dequantize_q8): the same kernels
    # in the same order as one moe_dispatch call, timed apart.
    q8 = buf.x_perm_q is not None
    adm = buf.flags
    padded = cfg.get("layout", "compact") == "padded"
    R_ffn = buf.rows  # rows the FFN runs over (E*cap with the padded layout)
    # The padded layout's padding rows are zeroed by the whole-dispatch call,
    # so that layout runs the dispatch as one call.
    disp_calls = ["dispatch"] if padded else (["dispatch_layout", "permute"]
                                              + (["dequantize"] if q8 else []))
    calls = (["route"] + disp_calls
             + ["ffn_plan", "ffn_up", "ffn_down", "combine", "bias_update"])
    fork = layer.has_shared(buf, wts)
    main = torch.cuda.current_stream()

    def step(events=None, shared_events=None):
        def mark(i):
            if events is not None:
                events[i].record(main)
        if fork:
            buf.side_stream.wait_stream(main)
            if shared_events is not None:
                shared_events[0].record(buf.side_stream)
            layer.shared_ffn(buf, wts, buf.side_stream)
            if shared_events is not None:
                shared_events[1].record(buf.side_stream)
        i = 0
        mark(i)
        layer.route(buf, inp)
        i += 1
        mark(i)
        if padded:
            layer.dispatch(buf, inp)
        else:
            moe.moe_dispatch_layout(d, adm, buf.topk_idx, buf.row_of_slot, buf.token_of_row,
                                    buf.slot_of_row, buf.expert_offsets, buf.admitted,
                                    buf.rank_offsets, buf.rank_counts, buf.ws_dispatch)
            i += 1
            mark(i)
            if q8:
                moe.moe_permute_q8(d, inp["x"], buf.row_of_slot, buf.x_perm_q, buf.row_scale)
                i += 1
                mark(i)
                moe.moe_dequantize_q8(S, dim, cfg["dtype"], buf.x_perm_q, buf.row_scale,
                                      buf.expert_offsets[E:], buf.x_perm)
            else:
                moe.moe_permute(d, inp["x"], buf.row_of_slot, buf.x_perm)
        i += 1
        mark(i)
        moe.moe_expert_ffn_plan(E, R_ffn, dim, h, cfg["act"], cfg["dtype"], buf.expert_offsets,
                                buf.ws_ffn)
        i += 1
        mark(i)
        moe.moe_expert_ffn_up(E, R_ffn, dim, h, cfg["act"], cfg["dtype"], buf.x_perm,
                              buf.expert_offsets, wts["w1"], wts.get("w3"), buf.ws_ffn)
        i += 1
        mark(i)
        moe.moe_expert_ffn_down(E, R_ffn, dim, h, cfg["act"], cfg["dtype"], buf.expert_offsets,
                                wts["w2"], buf.y_perm, buf.ws_ffn)
        i += 1
        mark(i)
        if fork:
            main.wait_stream(buf.side_stream)
        layer.combine(buf, inp, residual=True)
        i += 1
        mark(i)
        layer.bias_update(buf, bias_state, step_bias)
        mark(i + 1)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: exactly K steps, nothing else on the stream, bracketed by
    # synchronisation (one GPU, so no barrier is needed beyond that).
    edge = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    edge[0].record()
    for _ in range(args.steps):
        step()
    edge[1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = edge[0].elapsed_time(edge[1])
    ms_per_step = max(gpu_ms, wall * 1e3) / args.steps
    value = N / (ms_per_step * 1e-3)

    # Per-call pass: the same K steps again with a HIP event at every call
    # boundary (on torch's current stream, which every call is launched on).
    # Each event drains the queue for a few microseconds, so this pass gives
    # the per-kernel durations and the roofline, not the step time.
    nev = len(calls) + 1
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(args.steps)]
    sh_events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)]
                 for _ in range(args.steps)]
    torch.cuda.synchronize()
    for s in range(args.steps):
        step(events[s], sh_events[s])
    torch.cuda.synchronize()
    per_call = {c: 0.0 for c in calls}
    for ev in events:
        for i, c in enumerate(calls):
            per_call[c] += ev[i].elapsed_time(ev[i + 1])
    per_call = {c: v / args.steps * 1e3 for c, v in per_call.items()}  # microseconds
    if fork:
        per_call["shared_ffn"] = sum(a.elapsed_time(b) for a, b in sh_events) / args.steps * 1e3
    instrumented_ms = sum(events[s][0].elapsed_time(events[s][-1])
                          for s in range(args.steps)) / args.steps

    # Step-time distribution: the same K steps with one event per step
    # boundary only.
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    marks[0].record()
    for s in range(args.steps):
        step()
        marks[s + 1].record()
    torch.cuda.synchronize()
    step_ms = sorted(marks[s].elapsed_time(marks[s + 1]) for s in range(args.steps))

    def pct(v, q):
        return v[min(len(v) - 1, int(q * (len(v) - 1) + 0.5))]

    # Cold pass: before each step a 512 MiB write evicts the 256 MB Infinity
    # Cache and every XCD's L2, then the step runs with per-call events.
    n_cold = min(args.steps, 20)
    flush = torch.empty(512 << 18, dtype=torch.float32, device=dev)
    cold_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(n_cold)]
    cold_sh = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n_cold)]
    torch.cuda.synchronize()
    for s in range(n_cold):
        flush.fill_(float(s))
        step(cold_ev[s], cold_sh[s])
    torch.cuda.synchronize()
    cold_call = {c: sum(ev[i].elapsed_time(ev[i + 1]) for ev in cold_ev) / n_cold * 1e3
                 for i, c in enumerate(calls)}
    if fork:
        cold_call["shared_ffn"] = sum(a.elapsed_time(b) for a, b in cold_sh) / n_cold * 1e3
    cold_step_ms = sum(ev[0].elapsed_time(ev[-1]) for ev in cold_ev) / n_cold
    del flush

    if args.copy_calibration_mib > 0:
        # A plain elementwise copy kernel (reads and writes nbytes each), whose
        # counters scale the HBM byte counters of the kernels above.
        nbytes = args.copy_calibration_mib << 20
        a = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        torch.add(a, 0.0, out=b)
        torch.cuda.synchronize()

    # Algorithmic work of this batch (rows actually admitted).
    M = int(buf.expert_offsets[E].item())  # rows laid out (E*cap when padded)
    admitted_rows = int(buf.admitted.sum().item())
    counts = buf.admitted.cpu()
    active = int((counts > 0).sum().item())
    es = 2 if cfg["dtype"] == "bf16" else 4
    mats_up = 2 if cfg["act"] == "swiglu" else 1
    up_flops = 2.0 * M * dim * h * mats_up
    up_bytes = (active * mats_up * h * dim + M * dim + M * h) * es
    down_flops = 2.0 * M * h * dim
    down_bytes = (active * dim * h + M * h + M * dim) * es
    # dispatch layout: ids read, row_of_slot + token_of_row + slot_of_row written
    layout_bytes = S * 4 + S * 4 + S * 4 + S
    # permute: x read once, every admitted row written (INT8 payload: d bytes + a
    # 4-byte scale per row), row_of_slot read; dequantisation reads the payload
    # back and writes dtype rows
    permute_bytes = (N * dim * es + (admitted_rows * (dim + 4) if q8 else admitted_rows * dim * es)
                     + S * 4)
    dequant_bytes = M * (dim + 4) + M * dim * es
    combine_bytes = M * dim * es + N * dim * es + N * dim * es + S * 8
    route_bytes = N * dim * es + E * dim * es + N * E * 4 + S * 8
    peak = MFMA_PEAK_TFLOPS[cfg["dtype"]]

    def roof(name, flops, nbytes, table=per_call):
        t = table[name] * 1e-6
        t_f, t_b = flops / (peak * 1e12), nbytes / (HBM_PEAK_GBS * 1e9)
        return {"us": round(table[name], 2), "tflops": round(flops / t / 1e12, 2),
                "gbs": round(nbytes / t / 1e9, 1), "mfma_frac": round(flops / t / (peak * 1e12), 4),
                "hbm_frac": round(nbytes / t / (HBM_PEAK_GBS * 1e9), 4),
                "bound": "mfma" if t_f >= t_b else "hbm"}

    kern = {
        "ffn_up": roof("ffn_up", up_flops, up_bytes),
        "ffn_down": roof("ffn_down", down_flops, down_bytes),
    }
    if padded:  # one whole-dispatch call; the padding rows are written as zeros
        hbm_calls = [("route", route_bytes),
                     ("dispatch", layout_bytes + permute_bytes
                      + (M - admitted_rows) * (dim + 4 if q8 else dim * es)
                      + (dequant_bytes if q8 else 0)),
                     ("combine", combine_bytes)]
    else:
        hbm_calls = [("route", route_bytes), ("dispatch_layout", layout_bytes),
                     ("permute", permute_bytes), ("combine", combine_bytes)]
        if q8:
            hbm_calls.append(("dequantize", dequant_bytes))
    for name, nbytes in hbm_calls:
        t = per_call[name] * 1e-6
        kern[name] = {"us": round(per_call[name], 2), "gbs": round(nbytes / t / 1e9, 1),
                      "hbm_frac": round(nbytes / t / (HBM_PEAK_GBS * 1e9), 4)}
    if not padded:
        kern["dispatch"] = {"us": round(sum(per_call[c] for c in
                                            ("dispatch_layout", "permute", "dequantize")
                                            if c in per_call), 2)}
    for name in per_call:
        kern.setdefault(name, {"us": round(per_call[name], 2)})
    cold = {"ms_per_step_with_per_call_events": round(cold_step_ms, 4), "steps": n_cold,
            "ffn_up": roof("ffn_up", up_flops, up_bytes, cold_call),
            "ffn_down": roof("ffn_down", down_flops, down_bytes, cold_call)}
    for name, nbytes in hbm_calls:
        cold[name] = {"us": round(cold_call[name], 2),
                      "hbm_frac": round(nbytes / (cold_call[name] * 1e-6) / (HBM_PEAK_GBS * 1e9), 4)}
    for name in cold_call:
        cold.setdefault(name, {"us": round(cold_call[name], 2)})

    dom = "ffn_up" if per_call["ffn_up"] >= per_call["ffn_down"] else "ffn_down"
    dk = kern[dom]
    kernel_name = {"ffn_up": "grouped_gemm_up", "ffn_down": "grouped_gemm_down"}[dom]
    digest = kernel_sources_digest()
    traffic = read_traffic(kernel_name, args.workload, digest)
    if dk["bound"] == "mfma":
        roofline = {"bound": "mfma", "achieved": dk["tflops"], "peak": peak, "unit": "TFLOP/s",
                    "frac": dk["mfma_frac"], "traffic": traffic}
    else:
        roofline = {"bound": "hbm", "achieved": dk["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": dk["hbm_frac"], "traffic": traffic}
    roofline["kernel"] = f"{kernel_name} ({dom})"
    roofline["mfma_frac"] = dk["mfma_frac"]

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg["dtype"],
        "data": "synthetic",
        "config": {"workload": describe(cfg), "global_batch": N,
                   "rows_admitted": admitted_rows, "dropped_slots": S - admitted_rows,
                   "rows_laid_out": M, "active_experts": active},
        "roofline": roofline,
        "grouped_gemm_mfma_frac": {"up": kern["ffn_up"]["mfma_frac"],
                                   "down": kern["ffn_down"]["mfma_frac"]},
        "permute_hbm_frac": kern["permute" if "permute" in kern else "dispatch"]["hbm_frac"],
        "kernels": kern,
        "ms_per_step_with_per_call_events": round(instrumented_ms, 4),
        "step_ms_p10_p50_p90": [round(pct(step_ms, q), 4) for q in (0.1, 0.5, 0.9)],
        "cold": cold,
        "platform": {"hip": torch.version.hip, "torch": torch.__version__,
                     "device": torch.cuda.get_device_name(0), **clocks},
        "timed_region": {"gpu_events_ms": round(gpu_ms, 3), "host_wall_ms": round(wall * 1e3, 3)},
        "kernel_sources_digest": digest,
    }
    if args.rank_share:
        out["rank_share"] = rank_share(moe, torch, cfg, buf, wts, max(5, min(args.steps, 30)))
    if args.backward:
        out["backward"] = backward_pass(moe, torch, buf, inp, max(5, min(args.steps, 30)))
    if not args.no_cpu_baseline:
        host = {}
        for key, v in inp.items():
            if isinstance(v, tuple):
                host[key] = tuple(None if t is None else t.cpu() for t in v)
            elif isinstance(v, torch.Tensor):
                host[key] = v.cpu()
            else:
                host[key] = v
        cb = cpu_baseline(cfg, host, args.cpu_seconds)
        cb["gpu_speedup"] = round(value / cb["value"], 1)
        cb["single_thread"]["gpu_speedup"] = round(value / cb["single_thread"]["value"], 1)
        out["cpu_baseline"] = cb
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
