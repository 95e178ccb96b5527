"""Helpers for the GPU parity tests: device transfer, error metric, and
oracle references computed on the CPU from the same input tensors."""

from __future__ import annotations

import os

import numpy as np
import torch

import moe_workloads as W
import oracle

TOL = {"fp32": 1e-4, "bf16": 2e-2}  # max |gpu - ref| / max |ref| per tensor
TOPK_W_TOL = 1e-5


def threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def to_dev(inp: dict, dev="cuda") -> dict:
    out = {}
    for k, v in inp.items():
        if isinstance(v, tuple):
            out[k] = tuple(None if t is None else t.to(dev) for t in v)
        elif isinstance(v, torch.Tensor):
            out[k] = v.to(dev)
        else:
            out[k] = v
    return out


def n(t):
    return W.to_numpy(t)


def rel_err(got, ref) -> float:
    g = got.double().cpu() if isinstance(got, torch.Tensor) else torch.from_numpy(np.asarray(got, np.float64))
    r = ref.double().cpu() if isinstance(ref, torch.Tensor) else torch.from_numpy(np.asarray(ref, np.float64))
    den = r.abs().max().item()
    return (g - r).abs().max().item() / (den if den > 0 else 1.0)


def as_tensor(a, dtype: str) -> torch.Tensor:
    """Oracle numpy output (bf16 as uint16 bits) -> CPU tensor."""
    if dtype == "bf16":
        return W.from_numpy_bf16(a)
    return torch.from_numpy(np.ascontiguousarray(a))


def bits(t: torch.Tensor) -> np.ndarray:
    """Bit pattern of a tensor (for bitwise comparisons)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy()
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy()
    return t.numpy()


def shared_np(inp):
    if inp.get("shared") is None:
        return None
    return tuple(None if t is None else n(t[0]) for t in inp["shared"])


def oracle_reference(cfg: dict, inp_cpu: dict, sel_bias=None) -> dict:
    oracle.set_threads(threads())
    sb = inp_cpu.get("sel_bias") if sel_bias is None else sel_bias
    return oracle.forward(cfg, n(inp_cpu["x"]), n(inp_cpu["w_router"]), n(inp_cpu["router_bias"]),
                          n(sb), n(inp_cpu["w1"]), n(inp_cpu["w3"]), n(inp_cpu["w2"]),
                          shared=shared_np(inp_cpu))
