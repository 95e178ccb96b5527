#!/usr/bin/env python3
"""MoE-layer forward throughput on one MI355X.

One step is one pass of the whole hot path over one batch of synthetic input,
already resident in HBM: route -> dispatch -> expert FFN (plan, up, down; plus
the shared expert where the workload has one) -> combine -> selection-bias
update.  Default workload: the largest configuration that fits one GPU, the
DeepSeek-V3-like layer (N=4096 tokens, d=7168, 256 routed experts plus one
shared expert, sigmoid affinities with a selection-only bias, 8 groups of 32
keeping 4, top-8, SwiGLU 7168->2048->7168, 64 simulated EP ranks, bf16).

Prints one JSON line.  Every library call inside a second pass over the same
steps is bracketed by HIP events on the stream it is launched on; the per-call
averages give the roofline of the dominant kernel (algorithmic bytes or FLOPs
over its average duration) and the per-step breakdown.  Two more passes give
the step-time percentiles (one event per step) and the cold-cache per-call
times (a 512 MiB write before each step evicts the Infinity Cache and the
L2s).  The CPU oracle is timed on a bounded sample of the same workload
(``cpu_baseline``).  Short passes over other workloads (``--extra-workloads``,
default the Switch-style and Mixtral-like layers) are reported beside it.
"""

from __future__ import annotations

import argparse
import glob
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
WORKLOADS = ["toy", "switch", "mixtral", "deepseek", "zipf", "decode"]


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="deepseek", choices=WORKLOADS)
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
    ap.add_argument("--combine", default="unfused", choices=["unfused", "fused"],
                    help="unfused: the down GEMM writes y_perm and moe_combine gathers it; "
                         "fused: the down GEMM scatter-adds w*O into an fp32 accumulator "
                         "that moe_combine finishes")
    ap.add_argument("--no-clocks", action="store_true", help="skip reading the clocks")
    ap.add_argument("--no-isolated", action="store_true",
                    help="skip timing each call alone (profiler runs: every launch in the trace "
                         "is then one of a step, so its per-launch averages are the step's)")
    ap.add_argument("--graph", action="store_true",
                    help="replay the step captured once in a HIP graph instead of launching "
                         "every call from the host (measured: no faster; launches overlap "
                         "the GPU work either way)")
    ap.add_argument("--backward", action="store_true",
                    help="also time the layer's backward calls on this workload's layout")
    ap.add_argument("--library-gemm", action="store_true",
                    help="also time the FFN's up and down launches on a uniform batch against "
                         "the vendor library's batched GEMM (torch.bmm) on the same shapes")
    ap.add_argument("--rank-share", action="store_true",
                    help="also time the expert FFN on one rank's share of the experts at "
                         "its real shape (rows from all R source ranks)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run one device copy of this size (counter calibration)")
    ap.add_argument("--extra-workloads", default="switch,mixtral",
                    help="comma-separated workloads timed briefly beside the headline "
                         "one ('none' for none)")
    ap.add_argument("--extra-steps", type=int, default=30)
    return ap.parse_args(argv)


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
    """The selected DPM levels of the first AMD GPU the kernel driver exposes in
    sysfs (pp_dpm_sclk / pp_dpm_mclk; the line marked '*' is the current one).
    Read in-process: no child process, so nothing is spawned under a profiler."""
    info = {}
    for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
        try:
            with open(os.path.join(dev, "vendor")) as f:
                if f.read().strip() != "0x1002":
                    continue
            for clk in ("sclk", "mclk"):
                with open(os.path.join(dev, f"pp_dpm_{clk}")) as f:
                    cur = [l.strip() for l in f if l.strip().endswith("*")]
                info[clk] = cur[0] if cur else "unknown"
            info["sysfs"] = dev
            return info
        except OSError:
            continue
    return {"clocks": "unavailable (no readable pp_dpm_* in sysfs)"}


class ClockSampler:
    """Samples the current gfx clock (the marked line of pp_dpm_sclk, in MHz)
    from a thread while the GPU works: under load the chip runs below its
    2.4 GHz peak clock, and the MFMA peak scales with it.  In-process sysfs
    reads only; a no-op when the file is missing."""

    def __init__(self, sysfs, period_s=0.004):
        import threading
        self.path = os.path.join(sysfs, "pp_dpm_sclk") if sysfs else None
        self.period, self.mhz = period_s, []
        self.stop_ev = threading.Event()
        self.thread = threading.Thread(target=self._loop, daemon=True)

    def _read(self):
        with open(self.path) as f:
            for line in f:
                line = line.strip()
                if line.endswith("*"):
                    num = "".join(ch for ch in line.split(":", 1)[-1] if ch.isdigit())
                    return int(num) if num else None
        return None

    def _loop(self):
        while not self.stop_ev.is_set():
            try:
                v = self._read()
            except OSError:
                return
            if v:
                self.mhz.append(v)
            self.stop_ev.wait(self.period)

    def __enter__(self):
        if self.path and os.path.exists(self.path):
            self.thread.start()
        return self

    def __exit__(self, *exc):
        self.stop_ev.set()
        if self.thread.is_alive():
            self.thread.join()

    def summary(self):
        if not self.mhz:
            return None
        v = sorted(self.mhz)
        return {"samples": len(v), "median": v[len(v) // 2], "min": v[0], "max": v[-1]}


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
    if cfg.get("combine", "unfused") != "unfused":
        s += f" combine={cfg['combine']}"
    return s


class LayerRun:
    """One workload's inputs (resident in HBM), packed weights, buffers and the
    step as a sequence of library calls on torch's current stream."""

    def __init__(self, cfg, dev):
        import torch

        import expert_token_routing_router_amd as moe
        from expert_token_routing_router_amd import layer
        import moe_workloads as W

        self.torch, self.moe, self.layer = torch, moe, layer
        self.cfg = cfg
        # Inputs: the glossary snippet's stream for the toy workload (CPU),
        # else drawn on the device.
        gen_dev = "cpu" if cfg["name"] == "toy" else "cuda"
        src = W.make_inputs(cfg, device=gen_dev)
        self.inp = {k: (tuple(None if t is None else t.to(dev) for t in v) if isinstance(v, tuple)
                        else (v.to(dev) if isinstance(v, torch.Tensor) else v))
                    for k, v in src.items()}
        self.buf = moe.MoeBuffers(cfg, dev)
        # bf16 expert weights are packed once, as a model load would, before any
        # timed work.
        self.wts = moe.prepare_weights(cfg, self.inp)
        d = self.buf.desc
        self.E = d.num_experts
        self.bias_state = (self.inp["sel_bias"].clone() if self.inp.get("sel_bias") is not None
                           else torch.zeros(self.E, dtype=torch.float32, device=dev))
        self.step_bias = cfg.get("bias_step", 1e-3)
        self.q8 = self.buf.x_perm_q is not None
        self.padded = cfg.get("layout", "compact") == "padded"
        self.fused = cfg.get("combine", "unfused") == "fused"
        # The padded layout's padding rows are zeroed by the whole-dispatch
        # call, so that layout runs the dispatch as one call; otherwise the
        # dispatch runs as its two halves (the same kernels in the same order
        # as one moe_dispatch call, timed apart).
        disp = (["dispatch"] if self.padded else
                ["dispatch_layout", "permute"] + (["dequantize"] if self.q8 else []))
        self.calls = ["route"] + disp + ["ffn_plan", "ffn_up", "ffn_down", "combine",
                                         "bias_update"]
        self.fork = layer.has_shared(self.buf, self.wts)
        self.main = torch.cuda.current_stream()

    def step(self, events=None, shared_events=None):
        """One layer step.  A shared expert (needs only x) is forked onto a side
        stream after the route and joined before the combine, as the layer's
        forward does, timed by its own pair of events on that stream."""
        moe, layer, buf, cfg, inp, wts = (self.moe, self.layer, self.buf, self.cfg, self.inp,
                                          self.wts)
        d = buf.desc
        E, dim, h = d.num_experts, d.hidden, cfg["h"]
        rows = buf.rows
        main = self.main
        marks = iter(events or [])

        def mark():
            if events is not None:
                next(marks).record(main)

        mark()
        layer.route(buf, inp)
        if self.fork:
            buf.side_stream.wait_stream(main)
            if shared_events is not None:
                shared_events[0].record(buf.side_stream)
            layer.shared_ffn(buf, wts, buf.side_stream)
            if shared_events is not None:
                shared_events[1].record(buf.side_stream)
        mark()
        if self.padded:
            layer.dispatch(buf, inp)
        else:
            moe.moe_dispatch_layout(d, buf.flags, buf.topk_idx, buf.row_of_slot,
                                    buf.token_of_row, buf.slot_of_row, buf.expert_offsets,
                                    buf.admitted, buf.rank_offsets, buf.rank_counts,
                                    buf.ws_dispatch)
            mark()
            if self.q8:
                moe.moe_permute_q8(d, inp["x"], buf.row_of_slot, buf.x_perm_q, buf.row_scale)
                mark()
                moe.moe_dequantize_q8(rows, dim, cfg["dtype"], buf.x_perm_q, buf.row_scale,
                                      buf.expert_offsets[E:], buf.x_perm)
            else:
                moe.moe_permute(d, inp["x"], buf.row_of_slot, buf.x_perm)
        mark()
        moe.moe_expert_ffn_plan(E, rows, dim, h, cfg["act"], cfg["dtype"], buf.expert_offsets,
                                buf.ws_ffn)
        mark()
        moe.moe_expert_ffn_up(E, rows, dim, h, cfg["act"], cfg["dtype"], buf.x_perm,
                              buf.expert_offsets, wts["w1"], wts.get("w3"), buf.ws_ffn)
        mark()
        moe.moe_expert_ffn_down(E, rows, dim, h, cfg["act"], cfg["dtype"], buf.expert_offsets,
                                wts["w2"], None if self.fused else buf.y_perm,
                                buf.fused_args(), buf.ws_ffn)
        mark()
        if self.fork:
            main.wait_stream(buf.side_stream)
        layer.combine(buf, inp, residual=True)
        mark()
        layer.bias_update(buf, self.bias_state, self.step_bias)
        mark()

    def single_calls(self) -> dict:
        """Each call of a step (compact native-payload layout) as a closure
        that repeats it on the main stream with the step's own buffers, for
        timing one call with nothing else running: every one rewrites the same
        outputs from the same inputs (the bias update, which changes the next
        route, is left out)."""
        moe, layer, buf, cfg, inp, wts = (self.moe, self.layer, self.buf, self.cfg, self.inp,
                                          self.wts)
        if self.padded or self.q8 or self.fused:
            return {}
        d = buf.desc
        E, dim, h, rows = d.num_experts, d.hidden, cfg["h"], buf.rows
        calls = {
            "route": lambda: layer.route(buf, inp),
            "dispatch_layout": lambda: moe.moe_dispatch_layout(
                d, buf.flags, buf.topk_idx, buf.row_of_slot, buf.token_of_row, buf.slot_of_row,
                buf.expert_offsets, buf.admitted, buf.rank_offsets, buf.rank_counts,
                buf.ws_dispatch),
            "permute": lambda: moe.moe_permute(d, inp["x"], buf.row_of_slot, buf.x_perm),
            "ffn_up": lambda: moe.moe_expert_ffn_up(E, rows, dim, h, cfg["act"], cfg["dtype"],
                                                    buf.x_perm, buf.expert_offsets, wts["w1"],
                                                    wts.get("w3"), buf.ws_ffn),
            "ffn_down": lambda: moe.moe_expert_ffn_down(E, rows, dim, h, cfg["act"],
                                                        cfg["dtype"], buf.expert_offsets,
                                                        wts["w2"], buf.y_perm, None, buf.ws_ffn),
            "combine": lambda: layer.combine(buf, inp, residual=True),
        }
        if self.fork:
            calls["shared_ffn"] = lambda: layer.shared_ffn(buf, wts, self.main)
        return calls

    def n_events(self):
        return len(self.calls) + 1

    def capture(self):
        """Capture one step (every launch, the shared expert's fork and join)
        in a HIP graph; afterwards replay() runs that step.  Warm-up on the
        capture stream first, as torch's capture requires."""
        torch = self.torch
        side = torch.cuda.Stream()
        side.wait_stream(self.main)
        with torch.cuda.stream(side):
            self.main = side
            self.step()
        self.main = torch.cuda.current_stream()
        self.main.wait_stream(side)
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self.main = torch.cuda.current_stream()
            self.step()
        self.main = torch.cuda.current_stream()
        torch.cuda.synchronize()

    def replay(self):
        self.graph.replay()

    def algorithmic(self) -> dict:
        """Algorithmic work of this batch per call, from the rows actually
        admitted and the experts that received any.  The FFN's hidden buffer H
        is implementation traffic, not algorithmic: it is in no byte count."""
        buf, cfg = self.buf, self.cfg
        d = buf.desc
        N, k, E, dim, h = d.num_tokens, d.top_k, d.num_experts, d.hidden, cfg["h"]
        S = N * k
        es = 2 if cfg["dtype"] == "bf16" else 4
        admitted = buf.admitted.cpu()
        M = int(admitted.sum().item())               # admitted rows
        laid = int(buf.expert_offsets[E].item())     # rows laid out (E*cap when padded)
        active = int((admitted > 0).sum().item())
        mats_up = 2 if cfg["act"] == "swiglu" else 1
        shared = buf.shared_out is not None
        w_up = active * mats_up * h * dim * es
        w_down = active * dim * h * es
        out = {
            "M": M, "laid": laid, "active": active, "es": es, "mats_up": mats_up,
            "ffn_up": (2.0 * M * dim * h * mats_up, w_up + M * dim * es),
            "ffn_down": (2.0 * M * h * dim, w_down + M * dim * es),
            "weight_bytes": w_up + w_down,
            # route: x and the router weight read, logits and the k choices written
            "route": (0.0, N * dim * es + E * dim * es + N * E * 4 + S * 8),
            # layout: ids read; row_of_slot, token_of_row, slot_of_row written
            "dispatch_layout": (0.0, S * 4 + S * 4 + buf.rows * 5),
            # permute: x read once, every admitted row written (INT8 payload: d
            # bytes + a 4-byte scale per row), row_of_slot read
            "permute": (0.0, N * dim * es + (M * (dim + 4) if self.q8 else M * dim * es) + S * 4),
            "dequantize": (0.0, laid * (dim + 4) + laid * dim * es),
            # combine: every admitted row (fused: the fp32 accumulator row per
            # token instead), the residual and y, the shared output, the weights
            "combine": (0.0, (N * dim * 4 if self.fused else M * dim * es) + 2 * N * dim * es
                        + (N * dim * es if shared else 0) + S * 8),
        }
        if self.fused:  # the down GEMM adds w*O into the accumulator instead of writing y_perm
            out["ffn_down"] = (2.0 * M * h * dim, w_down + M * dim * 4)
        if self.padded:
            out["dispatch"] = (0.0, out["dispatch_layout"][1] + out["permute"][1]
                               + (laid - M) * (dim + 4 if self.q8 else dim * es)
                               + (out["dequantize"][1] if self.q8 else 0))
        return out


def time_steps(run, steps, graph=False):
    """Exactly `steps` steps between two synchronisations (one GPU, so no
    barrier is needed beyond that); the step time is the larger of the HIP-event
    and the host wall time of the region.  graph: each step is one replay of
    the captured step."""
    torch = run.torch
    edge = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    one = run.replay if graph else run.step
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    edge[0].record()
    for _ in range(steps):
        one()
    edge[1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = edge[0].elapsed_time(edge[1])
    return max(gpu_ms, wall * 1e3) / steps, gpu_ms, wall


def per_call_pass(run, steps):
    """The same steps with a HIP event at every call boundary on the main
    stream (every call is launched on it; the shared expert has its own pair on
    the side stream).  Each event drains the queue for a few microseconds, so
    this pass gives per-kernel durations, not the step time."""
    torch = run.torch
    nev = run.n_events()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(steps)]
    sh = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    torch.cuda.synchronize()
    for s in range(steps):
        run.step(events[s], sh[s])
    torch.cuda.synchronize()
    per = {c: sum(ev[i].elapsed_time(ev[i + 1]) for ev in events) / steps * 1e3
           for i, c in enumerate(run.calls)}  # microseconds
    if run.fork:
        per["shared_ffn"] = sum(a.elapsed_time(b) for a, b in sh) / steps * 1e3
    inst = sum(ev[0].elapsed_time(ev[-1]) for ev in events) / steps
    return per, inst


def isolated_pass(run, reps) -> dict:
    """Each call of the step timed alone after a full step: 3 untimed calls,
    then `reps` back to back between two events on the main stream, nothing
    on any other stream.  Inside the step a call can share the GPU with the
    shared expert's side stream; this is the call's own rate."""
    torch = run.torch
    out = {}
    for name, fn in run.single_calls().items():
        for _ in range(3):
            fn()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        ev[0].record(run.main)
        for _ in range(reps):
            fn()
        ev[1].record(run.main)
        torch.cuda.synchronize()
        out[name] = ev[0].elapsed_time(ev[1]) / reps * 1e3
    # Leave the step's state as a step leaves it.
    run.step()
    torch.cuda.synchronize()
    return out


def kernel_table(run, alg, per) -> dict:
    peak = MFMA_PEAK_TFLOPS[run.cfg["dtype"]]
    kern = {}
    for name, us in per.items():
        ent = {"us": round(us, 2)}
        if name in alg and isinstance(alg[name], tuple):
            flops, nbytes = alg[name]
            t = us * 1e-6
            ent["gbs"] = round(nbytes / t / 1e9, 1)
            ent["hbm_frac"] = round(nbytes / t / (HBM_PEAK_GBS * 1e9), 4)
            if flops:
                t_f, t_b = flops / (peak * 1e12), nbytes / (HBM_PEAK_GBS * 1e9)
                ent["tflops"] = round(flops / t / 1e12, 2)
                ent["mfma_frac"] = round(flops / t / (peak * 1e12), 4)
                ent["bound"] = "mfma" if t_f >= t_b else "hbm"
        kern[name] = ent
    if "dispatch_layout" in per:
        kern["dispatch"] = {"us": round(sum(per[c] for c in ("dispatch_layout", "permute",
                                                             "dequantize") if c in per), 2)}
    return kern


def routed_ffn_floor(run, alg, per) -> dict:
    """The routed expert FFN (up + down launches) against its floor: the larger
    of streaming the active experts' weights at the HBM peak and the FLOPs at
    the MFMA peak."""
    peak = MFMA_PEAK_TFLOPS[run.cfg["dtype"]]
    t = (per["ffn_up"] + per["ffn_down"]) * 1e-6
    flops = alg["ffn_up"][0] + alg["ffn_down"][0]
    t_w = alg["weight_bytes"] / (HBM_PEAK_GBS * 1e9)
    t_f = flops / (peak * 1e12)
    return {"us": round(t * 1e6, 1), "weight_bytes": alg["weight_bytes"],
            "weight_floor_us": round(t_w * 1e6, 1), "mfma_floor_us": round(t_f * 1e6, 1),
            "frac_of_floor": round(max(t_w, t_f) / t, 4),
            "weight_stream_gbs": round(alg["weight_bytes"] / t / 1e9, 1)}


def load_metrics(run) -> dict:
    """Load the pages measure: assignments per expert and per simulated rank
    (the layer ends when its busiest GPU ends), and the drop rate.  The Zipf
    workload also gets its realised popularity: the share of the hottest
    experts and the exponent fitted to count versus popularity rank, and the
    drop rate each capacity factor of its sweep would give on these counts."""
    import numpy as np

    buf, cfg = run.buf, run.cfg
    d = buf.desc
    N, k, E, R = d.num_tokens, d.top_k, d.num_experts, d.num_ranks
    S = N * k
    counts = buf.counts.cpu().numpy().astype(np.int64)
    admitted = buf.admitted.cpu().numpy().astype(np.int64)
    rank_pre = counts.reshape(R, E // R).sum(1)
    rank_adm = buf.rank_counts.cpu().numpy().astype(np.int64)
    out = {
        "expert_count_max_over_mean": round(float(counts.max()) / (S / E), 3) if S else None,
        "expert_count_min_max": [int(counts.min()), int(counts.max())],
        "rank_load_max_over_mean": round(float(rank_pre.max()) / (S / R), 3) if S else None,
        "rank_admitted_max_over_mean": (round(float(rank_adm.max()) / max(rank_adm.mean(), 1e-9), 3)
                                        if S else None),
        "rank_admitted_min_max": [int(rank_adm.min()), int(rank_adm.max())],
        "drop_rate": round(1.0 - admitted.sum() / S, 5) if S else 0.0,
    }
    if cfg.get("zipf"):
        srt = np.sort(counts)[::-1].astype(np.float64)
        pos = srt > 0
        r = np.arange(1, E + 1, dtype=np.float64)
        slope = np.polyfit(np.log(r[pos]), np.log(srt[pos]), 1)[0]
        out["zipf"] = {"target_s": cfg["zipf"], "fitted_s": round(float(-slope), 3),
                       "top1_share": round(srt[0] / S, 4), "top8_share": round(srt[:8].sum() / S, 4)}
        sweep = {}
        for cf in cfg.get("cf_sweep", ()):
            cap = math.ceil(cf * S / E)
            sweep[str(cf)] = round(1.0 - np.minimum(counts, cap).sum() / S, 5)
        out["zipf"]["drop_rate_by_cf"] = sweep
    return out


def quick_workload(name, steps, warmup, dev, graph=False, sysfs=None, isolated=True) -> dict:
    """A short pass over another workload: step time and the per-call
    durations with their roofline fractions (no cold pass, no oracle), and the
    gfx clock sampled during the per-call pass."""
    import moe_workloads as W

    cfg = W.full(name)
    run = LayerRun(cfg, dev)
    if graph:
        run.capture()
    for _ in range(warmup):
        run.replay() if graph else run.step()
    ms, _, _ = time_steps(run, steps, graph)
    with ClockSampler(sysfs) as sampler:
        per, _ = per_call_pass(run, steps)
    sclk = sampler.summary()
    iso = isolated_pass(run, max(3, min(steps, 10))) if isolated else {}
    alg = run.algorithmic()
    kern = kernel_table(run, alg, per)
    if sclk:
        for k in ("ffn_up", "ffn_down"):
            kern[k]["mfma_frac_at_sampled_clock"] = round(kern[k]["mfma_frac"] * 2400.0 / sclk["median"], 4)
    out = {"workload": describe(cfg), "ms_per_step": round(ms, 4), "sclk_mhz_sampled": sclk,
           "tokens_per_s": round(cfg["N"] / (ms * 1e-3), 1), "steps": steps, "warmup": warmup,
           "grouped_gemm": {k: kern[k] for k in ("ffn_up", "ffn_down")},
           "routed_ffn": routed_ffn_floor(run, alg, per),
           "route_us": kern["route"]["us"], "combine_hbm_frac": kern["combine"]["hbm_frac"],
           "permute_hbm_frac": kern.get("permute", kern.get("dispatch", {})).get("hbm_frac"),
           "isolated": kernel_table(run, alg, iso)}
    del run
    run = None
    import torch
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


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
        moe.moe_expert_ffn(El, M, dim, h, cfg["act"], cfg["dtype"], recv, goff, w1, w3, w2, y, None,
                           ws)

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


def library_gemm(moe, torch, cfg, wts, inp, steps: int) -> dict:
    """The expert FFN's two GEMM launches on a uniform batch (every expert
    N*k/E rows) against the vendor library on the same shapes: torch.bmm
    (hipBLASLt) of X [E, rows, d] with [W1^T | W3^T] (or W1^T) as one
    [E, d, n_up] operand, and of H [E, rows, h] with W2^T [E, h, d], both
    operands contiguous.  The library computes the plain products; the up
    launch here also applies the activation (and the SwiGLU product) and
    writes H, the down launch reads that H.  For scale, not a step."""
    E, dim, h, act, k, N = cfg["E"], cfg["d"], cfg["h"], cfg["act"], cfg["k"], cfg["N"]
    if cfg["dtype"] != "bf16":
        return {}
    dev = wts["w2"].device
    per = max(1, (N * k) // E)
    M = E * per
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    x = torch.randn(M, dim, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    off = (torch.arange(E + 1, dtype=torch.int32) * per).to(dev)
    ws = moe.workspace(moe.moe_expert_ffn_workspace_size(E, M, dim, h, act, "bf16"), device=dev)
    y = torch.empty_like(x)
    moe.moe_expert_ffn_plan(E, M, dim, h, act, "bf16", off, ws)

    def timed(fn):
        for _ in range(3):
            fn()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        ev[0].record()
        for _ in range(steps):
            fn()
        ev[1].record()
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / steps * 1e3

    up = timed(lambda: moe.moe_expert_ffn_up(E, M, dim, h, act, "bf16", x, off, wts["w1"],
                                             wts.get("w3"), ws))
    down = timed(lambda: moe.moe_expert_ffn_down(E, M, dim, h, act, "bf16", off, wts["w2"], y,
                                                 None, ws))
    del ws, y
    w1, w3, w2 = inp["w1"], inp.get("w3"), inp["w2"]
    bt = torch.cat([w1, w3], 1) if w3 is not None else w1  # [E, n_up, d]
    b_up = bt.transpose(1, 2).contiguous()                  # [E, d, n_up]
    del bt
    x3 = x.view(E, per, dim)
    lib_up = timed(lambda: torch.bmm(x3, b_up))
    del b_up
    b_dn = w2.transpose(1, 2).contiguous()                  # [E, h, d]
    hh = torch.randn(E, per, h, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    lib_down = timed(lambda: torch.bmm(hh, b_dn))
    del b_dn, hh, x
    torch.cuda.empty_cache()
    n_up = 2 * h if w3 is not None else h
    f_up, f_dn = 2.0 * M * dim * n_up, 2.0 * M * h * dim
    peak = MFMA_PEAK_TFLOPS["bf16"] * 1e12

    def rate(f, us):
        return {"us": round(us, 1), "tflops": round(f / (us * 1e-6) / 1e12, 1),
                "mfma_frac": round(f / (us * 1e-6) / peak, 4)}

    return {"rows_per_expert": per, "experts": E,
            "up": {"ours": rate(f_up, up), "library": rate(f_up, lib_up)},
            "down": {"ours": rate(f_dn, down), "library": rate(f_dn, lib_down)},
            "library": f"torch.bmm (hipBLASLt) {torch.version.hip}"}


def backward_pass(moe, torch, buf, inp, steps: int) -> dict:
    """The layer's backward on its last layout: the combine's expert terms
    (row and weight gradients), the expert FFN's backward (input and weight
    gradients, bf16), the permute's adjoint and the router's backward, timed
    with events; per call, the algorithmic bytes (data path) or FLOPs (FFN)
    over the time."""
    d = buf.desc
    N, k, dim = d.num_tokens, d.top_k, d.hidden
    dev = buf.y.device
    dt = buf.y.dtype
    es = buf.y.element_size()
    M = int(buf.admitted.sum().item())
    g = torch.Generator(device=dev).manual_seed(7)
    dy = torch.randn(N, dim, generator=g, device=dev).to(dt)
    # Rows of dy_perm that no slot maps to (padding rows of a padded layout)
    # are never written by moe_combine_backward: start from zeros.
    dy_perm = torch.zeros_like(buf.y_perm)
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
    frac = lambda nb, us: round(nb / (us * 1e-6) / (HBM_PEAK_GBS * 1e9), 4)  # noqa: E731
    out = {"combine_backward": {"us": round(cb, 2), "hbm_frac": frac(cb_bytes, cb)},
           "permute_backward": {"us": round(pb, 2), "hbm_frac": frac(pb_bytes, pb)}}
    # Router backward from the combine backward's weight gradients, with the
    # auxiliary load-balancing loss, adding the router's term into dx.
    E = d.num_experts
    dl = torch.empty(N, E, device=dev)
    dwr = torch.empty(E, dim, device=dev)
    dbr = torch.empty(E, device=dev)
    loss = torch.empty(1, device=dev)
    rws = moe.workspace(moe.moe_router_backward_workspace_size(d), dev)

    def router_bwd():
        moe.moe_router_backward(d, inp["x"], inp["w_router"], buf.logits, buf.topk_idx, dw,
                                buf.counts, 0.01, dl, dwr, dbr, dx, True, loss, rws)

    for _ in range(2):
        router_bwd()
    torch.cuda.synchronize()
    rb = 0.0
    for _ in range(steps):
        ev[0].record()
        router_bwd()
        ev[1].record()
        torch.cuda.synchronize()
        rb += ev[0].elapsed_time(ev[1])
    rb = rb / steps * 1e3
    # two contractions of N x E x d (dW_r and dx), plus the logits pass
    rflops = 2.0 * 2 * N * E * dim
    out["router_backward"] = {"us": round(rb, 2), "tflops": round(rflops / (rb * 1e-6) / 1e12, 2),
                              "aux_loss": round(float(loss.item()), 6)}
    cfg = buf.cfg
    if cfg["dtype"] != "bf16":
        return out
    # Expert FFN backward over the laid-out rows, plain row-major weights.
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
                                    buf.expert_offsets, buf.admitted, w1, w3, w2, dy_perm,
                                    dx_perm, dw1, dw3, dw2, ws)

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
    # Algorithmic products per admitted row, 2 d h FLOPs each: g = dy W2, dx
    # (one product per gate/up matrix), and one weight gradient per weight
    # matrix: 6 for SwiGLU (g, dx over W1 and W3, dW1, dW3, dW2), 4 otherwise.
    # The kernels also recompute u (and v): 8 and 5 products executed.
    n_alg, n_exec = (6, 8) if sw else (4, 5)
    flops = 2.0 * M * dim * h * n_alg
    grad_bytes = (3 if sw else 2) * E * h * dim * 4  # fp32 weight gradients written
    pk = MFMA_PEAK_TFLOPS["bf16"] * 1e12
    out["ffn_backward"] = {
        "us": round(fb, 2), "tflops": round(flops / (fb * 1e-6) / 1e12, 1),
        "mfma_frac": round(flops / (fb * 1e-6) / pk, 4),
        "executed_tflops": round(2.0 * M * dim * h * n_exec / (fb * 1e-6) / 1e12, 1),
        "weight_grad_bytes": grad_bytes}
    # The same backward on the forward's grouped GEMM (packed weights, packed
    # once per weight update like the forward's, outside the timed region).
    if dim % 64 == 0 and h % 64 == 0:
        pw = moe.prepare_backward_weights(cfg, {"w1": w1, "w3": w3, "w2": w2})
        wsp = moe.workspace(moe.moe_expert_ffn_backward_packed_workspace_size(
            E, buf.rows, dim, h, act, "bf16"), dev)
        dx_p = torch.empty_like(buf.x_perm)

        def ffn_bwd_packed():
            moe.moe_expert_ffn_backward_packed(E, buf.rows, dim, h, act, "bf16", buf.x_perm,
                                               buf.expert_offsets, buf.admitted, pw["w1"],
                                               pw["w3"], pw["w2t"], pw["w13t"], dy_perm, dx_p,
                                               dw1, dw3, dw2, wsp)

        for _ in range(2):
            ffn_bwd_packed()
        torch.cuda.synchronize()
        fp = 0.0
        for _ in range(steps):
            ev[0].record()
            ffn_bwd_packed()
            ev[1].record()
            torch.cuda.synchronize()
            fp += ev[0].elapsed_time(ev[1])
        fp = fp / steps * 1e3
        out["ffn_backward_packed"] = {
            "us": round(fp, 2), "tflops": round(flops / (fp * 1e-6) / 1e12, 1),
            "mfma_frac": round(flops / (fp * 1e-6) / pk, 4),
            "executed_tflops": round(2.0 * M * dim * h * n_exec / (fp * 1e-6) / 1e12, 1)}
        del pw, wsp, dx_p
    return out


def cpu_baseline(cfg, inp, target_s: float) -> dict:
    """Time the oracle (as it stands) on the first T tokens of the workload,
    taken as a batch of T (capacity recomputed for T): route, dispatch, FFN,
    combine and bias update.  T is chosen so the run lasts about target_s.  Each
    token's FFN work is independent of the others, so tokens/s on the sample
    is the rate the oracle would sustain over the whole batch (extrapolated)."""
    import numpy as np

    import moe_workloads as W
    import oracle

    threads = max(1, min(16, os.cpu_count() or 1))
    oracle.set_threads(threads)
    n = W.to_numpy
    wr, rb = n(inp["w_router"]), n(inp["router_bias"])
    sb = n(inp["sel_bias"])
    bias_state = sb.copy() if sb is not None else np.zeros(cfg["E"], np.float32)
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
    full = T >= cfg["N"]
    label = "" if full else " (a sample: tokens/s extrapolated to the whole batch)"
    out = {"value": T / elapsed, "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": f"first {T} of {cfg['N']} tokens as one batch (capacity for {T}); "
                     f"route+dispatch+FFN+combine+bias update; {elapsed:.1f} s{label}"}

    # The same on one thread, the plain loops as written, on a smaller sample.
    oracle.set_threads(1)
    T1 = min(cfg["N"], 8)
    e1 = run(T1)
    for _ in range(4):
        if e1 >= target_s / 4 or T1 >= cfg["N"]:
            break
        T1 = int(min(cfg["N"], max(2 * T1, T1 * (target_s / 2) / max(e1, 1e-6))))
        e1 = run(T1)
    oracle.set_threads(threads)
    out["single_thread"] = {"value": T1 / e1, "unit": "tokens/s", "cores": 1,
                            "sample": f"first {T1} of {cfg['N']} tokens as one batch; {e1:.1f} s"
                                      + ("" if T1 >= cfg["N"] else " (extrapolated)")}
    return out


def main(argv=None):
    args = parse_args(argv)
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    clocks = {} if args.no_clocks else read_clocks()
    import torch

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
    if args.combine != "unfused":
        cfg["combine"] = args.combine
    run = LayerRun(cfg, dev)
    N = cfg["N"]
    graph = args.graph
    if graph:
        run.capture()  # two untimed steps: the capture stream's warm-up and the capture
    one = run.replay if graph else run.step

    for _ in range(args.warmup):
        one()
    torch.cuda.synchronize()
    # Timed region: exactly K steps.
    ms_per_step, gpu_ms, wall = time_steps(run, args.steps, graph)
    value = N / (ms_per_step * 1e-3)

    # The per-call pass, with the gfx clock sampled beside it (the clock the
    # kernels' durations were taken at).
    with ClockSampler(clocks.get("sysfs")) as sampler:
        per_call, instrumented_ms = per_call_pass(run, args.steps)
    sclk = sampler.summary()
    iso_call = {} if args.no_isolated else isolated_pass(run, max(3, min(args.steps, 10)))

    # Step-time distribution: the same K steps with one event per step
    # boundary only.
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    marks[0].record()
    for s in range(args.steps):
        one()
        marks[s + 1].record()
    torch.cuda.synchronize()
    step_ms = sorted(marks[s].elapsed_time(marks[s + 1]) for s in range(args.steps))

    def pct(v, q):
        return v[min(len(v) - 1, int(q * (len(v) - 1) + 0.5))]

    # Cold pass: before each step a 512 MiB write evicts the 256 MB Infinity
    # Cache and every XCD's L2, then the step runs with per-call events.
    n_cold = min(args.steps, 20)
    nev = run.n_events()
    flush = torch.empty(512 << 18, dtype=torch.float32, device=dev)
    cold_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(n_cold)]
    cold_sh = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n_cold)]
    torch.cuda.synchronize()
    for s in range(n_cold):
        flush.fill_(float(s))
        run.step(cold_ev[s], cold_sh[s])
    torch.cuda.synchronize()
    cold_call = {c: sum(ev[i].elapsed_time(ev[i + 1]) for ev in cold_ev) / n_cold * 1e3
                 for i, c in enumerate(run.calls)}
    if run.fork:
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
        del a, b

    alg = run.algorithmic()
    kern = kernel_table(run, alg, per_call)
    iso = kernel_table(run, alg, iso_call)
    cold = {"ms_per_step_with_per_call_events": round(cold_step_ms, 4), "steps": n_cold}
    cold.update(kernel_table(run, alg, cold_call))

    dom = "ffn_up" if per_call["ffn_up"] >= per_call["ffn_down"] else "ffn_down"
    dk = kern[dom]
    kernel_name = {"ffn_up": "grouped_gemm_up", "ffn_down": "grouped_gemm_down"}[dom]
    digest = kernel_sources_digest()
    traffic = read_traffic(kernel_name, args.workload, digest)
    peak = MFMA_PEAK_TFLOPS[cfg["dtype"]]
    if dk["bound"] == "mfma":
        roofline = {"bound": "mfma", "achieved": dk["tflops"], "peak": peak, "unit": "TFLOP/s",
                    "frac": dk["mfma_frac"], "traffic": traffic}
    else:
        roofline = {"bound": "hbm", "achieved": dk["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": dk["hbm_frac"], "traffic": traffic}
    roofline["kernel"] = f"{kernel_name} ({dom})"
    roofline["us_per_launch"] = dk["us"]
    roofline["algorithmic"] = ("active experts' weights + x_perm rows read"
                               + (" + y_perm rows written" if dom == "ffn_down" else "")
                               + "; H excluded")
    roofline["mfma_frac"] = dk["mfma_frac"]
    if sclk:
        # The same product against the MFMA peak at the sampled clock
        # (the 2.5 PFLOP/s figure assumes 2.4 GHz).
        roofline["mfma_frac_at_sampled_clock"] = round(dk["mfma_frac"] * 2400.0 / sclk["median"], 4)

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
                   "rows_admitted": alg["M"], "dropped_slots": N * cfg["k"] - alg["M"],
                   "rows_laid_out": alg["laid"], "active_experts": alg["active"]},
        "roofline": roofline,
        "routed_ffn": routed_ffn_floor(run, alg, per_call),
        "grouped_gemm_mfma_frac": {"up": kern["ffn_up"]["mfma_frac"],
                                   "down": kern["ffn_down"]["mfma_frac"]},
        # the permute call with its events inside the step (where the shared
        # expert's side stream may share the GPU), and the call timed alone
        "permute_hbm_frac": kern.get("permute", kern.get("dispatch", {})).get("hbm_frac"),
        "permute_hbm_frac_isolated": iso.get("permute", {}).get("hbm_frac"),
        "combine_hbm_frac_isolated": iso.get("combine", {}).get("hbm_frac"),
        "isolated": iso,
        "load": load_metrics(run),
        "kernels": kern,
        "ms_per_step_with_per_call_events": round(instrumented_ms, 4),
        "step_ms_p10_p50_p90": [round(pct(step_ms, q), 4) for q in (0.1, 0.5, 0.9)],
        "cold": cold,
        "platform": {"hip": torch.version.hip, "torch": torch.__version__,
                     "device": torch.cuda.get_device_name(0), **clocks,
                     "sclk_mhz_sampled_in_per_call_pass": sclk},
        "timed_region": {"gpu_events_ms": round(gpu_ms, 3), "host_wall_ms": round(wall * 1e3, 3),
                         "launch": "HIP graph replay of the captured step" if graph
                         else "eager launches"},
        "kernel_sources_digest": digest,
    }
    if args.library_gemm:
        out["library_gemm"] = library_gemm(run.moe, torch, cfg, run.wts, run.inp,
                                           max(5, min(args.steps, 20)))
    if args.rank_share:
        out["rank_share"] = rank_share(run.moe, torch, cfg, run.buf, run.wts,
                                       max(5, min(args.steps, 30)))
    if args.backward:
        out["backward"] = backward_pass(run.moe, torch, run.buf, run.inp,
                                        max(5, min(args.steps, 30)))
    host = None
    if not args.no_cpu_baseline:
        host = {}
        for key, v in run.inp.items():
            if isinstance(v, tuple):
                host[key] = tuple(None if t is None else t.cpu() for t in v)
            elif isinstance(v, torch.Tensor):
                host[key] = v.cpu()
            else:
                host[key] = v
    # Free the headline workload's device memory before the other workloads.
    del run
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    extras = [w for w in args.extra_workloads.split(",") if w and w != "none"]
    if extras:
        out["other_workloads"] = {}
        for w in extras:
            if w == args.workload or w not in WORKLOADS:
                continue
            out["other_workloads"][w] = quick_workload(w, args.extra_steps, 10, dev,
                                                       args.graph, clocks.get("sysfs"),
                                                       not args.no_isolated)
    if host is not None:
        cb = cpu_baseline(cfg, host, args.cpu_seconds)
        cb["gpu_speedup"] = round(value / cb["value"], 1)
        cb["single_thread"]["gpu_speedup"] = round(value / cb["single_thread"]["value"], 1)
        out["cpu_baseline"] = cb
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
