"""Seeded synthetic workloads for the MoE-layer forward.

This module only describes shapes and draws seeded random tensors; it holds
none of the layer's arithmetic.  Both the CPU oracle's tests and the HIP path's
tests and benchmark feed it the same tensors.

Six workload families (full sizes), after the configurations the pages'
examples and the systems they name suggest:

* ``toy``      -- the routing snippet of the "Expert Parallelism" glossary page
                  ("How tokens travel between GPUs"): 4096 tokens ~N(0,1) of
                  width 512, a Linear(512, 8) router, top-2, 8 experts on 4
                  simulated GPUs; plus ReLU experts 512->256->512 ~N(0, 0.02).
                  fp32.  The first draws reproduce the snippet's own RNG stream
                  (``torch.manual_seed(0)``, ``randn``, ``nn.Linear``).
* ``switch``   -- top-1 (Switch style): 16384 tokens, d=1024, 64 experts,
                  softmax over all 64, capacity factor 1.25, GELU
                  1024->4096->1024, 8 ranks.  bf16.
* ``mixtral``  -- top-2 over 8 experts, softmax over the 2 selected logits,
                  SwiGLU 4096->14336->4096, 8192 tokens, 8 ranks.  bf16.
* ``deepseek`` -- 256 routed + 1 shared expert, sigmoid affinities plus a
                  per-expert selection bias ~N(0, 0.01), 8 groups of 32 (keep
                  4), top-8, SwiGLU 7168->2048->7168, 4096 tokens, 64 ranks.
* ``zipf``     -- 32768 tokens, d=2048, 128 experts, top-2 softmax, router
                  offsets that make expert popularity roughly Zipf(1.1),
                  SwiGLU 2048->1408->2048, 16 ranks, capacity factor in
                  {1.0, 1.25, 2.0}, one selection-bias update then re-routing.
* ``decode``   -- one decode step of the ``deepseek`` layer: 256 tokens (one
                  per sequence), every other parameter as ``deepseek`` but 32
                  ranks of 8 experts (DeepSeek-V3 decodes with EP = 40 over
                  320 expert slots, 8 per GPU; without redundant experts 256
                  experts make 32 such ranks).  About 8 rows per expert: the
                  expert FFN streams every weight for a few rows each.

``small(name)`` gives a reduced version of each (same routing structure,
smaller N/d/h with ragged sizes) that the oracle finishes in seconds.

Distributions: hidden states ~N(0,1); router weight (and bias when present)
~U(-1/sqrt(d), 1/sqrt(d)) as nn.Linear initialises them; expert weights
~N(0, 0.02); all drawn in fp32 and rounded to bf16 (round-to-nearest-even, by
torch's cast) where the workload is bf16.
"""

from __future__ import annotations

import math
import zlib

import torch

FULL = {
    "toy": dict(N=4096, d=512, h=256, E=8, k=2, R=4, cf=0.0, G=1, kg=1,
                score="softmax_topk", act="relu", dtype="fp32",
                router_bias="linear", sel_bias=None, shared=False, zipf=None),
    "switch": dict(N=16384, d=1024, h=4096, E=64, k=1, R=8, cf=1.25, G=1, kg=1,
                   score="softmax_all", act="gelu", dtype="bf16",
                   router_bias=None, sel_bias=None, shared=False, zipf=None),
    "mixtral": dict(N=8192, d=4096, h=14336, E=8, k=2, R=8, cf=0.0, G=1, kg=1,
                    score="softmax_topk", act="swiglu", dtype="bf16",
                    router_bias=None, sel_bias=None, shared=False, zipf=None),
    "deepseek": dict(N=4096, d=7168, h=2048, E=256, k=8, R=64, cf=0.0, G=8, kg=4,
                     score="sigmoid_norm", act="swiglu", dtype="bf16",
                     router_bias=None, sel_bias=0.01, shared=True, zipf=None),
    "zipf": dict(N=32768, d=2048, h=1408, E=128, k=2, R=16, cf=1.25, G=1, kg=1,
                 score="softmax_topk", act="swiglu", dtype="bf16",
                 router_bias="zipf", sel_bias="zeros", shared=False, zipf=1.1,
                 cf_sweep=(1.0, 1.25, 2.0), bias_step=1e-3),
    "decode": dict(N=256, d=7168, h=2048, E=256, k=8, R=32, cf=0.0, G=8, kg=4,
                   score="sigmoid_norm", act="swiglu", dtype="bf16",
                   router_bias=None, sel_bias=0.01, shared=True, zipf=None),
}

_SMALL = {
    "toy": dict(N=1001, d=192, h=128),
    "switch": dict(N=2053, d=256, h=512),
    "mixtral": dict(N=1531, d=512, h=448),
    "deepseek": dict(N=517, d=384, h=192),
    "zipf": dict(N=3001, d=256, h=192),
    "decode": dict(N=67, d=384, h=192),
}

ORDER = ["toy", "switch", "mixtral", "deepseek", "zipf", "decode"]


def full(name: str) -> dict:
    cfg = dict(FULL[name])
    cfg["name"] = name
    cfg["size"] = "full"
    return cfg


def small(name: str) -> dict:
    cfg = dict(FULL[name])
    cfg.update(_SMALL[name])
    cfg["name"] = name
    cfg["size"] = "small"
    return cfg


def with_(cfg: dict, **kw) -> dict:
    out = dict(cfg)
    out.update(kw)
    return out


def torch_dtype(cfg: dict) -> torch.dtype:
    return torch.float32 if cfg["dtype"] == "fp32" else torch.bfloat16


def seed_of(cfg: dict, tensor: str) -> int:
    """Deterministic seed per (workload, size, tensor)."""
    key = f"{cfg['name']}/{cfg.get('size', 'full')}/{cfg['N']}x{cfg['d']}x{cfg['h']}/{tensor}"
    return zlib.crc32(key.encode()) & 0x7FFFFFFF


def _gen(cfg, tensor, device):
    g = torch.Generator(device=device)
    g.manual_seed(seed_of(cfg, tensor))
    return g


def _normal(cfg, tensor, shape, std, device, chunk_dim0=None):
    """~N(0, std) in the workload dtype; drawn in fp32 chunks along dim 0."""
    dt = torch_dtype(cfg)
    out = torch.empty(shape, dtype=dt, device=device)
    g = _gen(cfg, tensor, device)
    n0 = shape[0]
    step = chunk_dim0 or n0
    for i in range(0, n0, step):
        j = min(n0, i + step)
        blk = torch.randn((j - i,) + tuple(shape[1:]), generator=g, device=device,
                          dtype=torch.float32)
        out[i:j] = (blk * std).to(dt)
    return out


def _uniform(cfg, tensor, shape, bound, device, dtype=None):
    g = _gen(cfg, tensor, device)
    u = torch.rand(shape, generator=g, device=device, dtype=torch.float32)
    return ((u * 2.0 - 1.0) * bound).to(dtype or torch_dtype(cfg))


def zipf_offsets(E: int, s: float, logit_std: float) -> torch.Tensor:
    """Per-expert router offsets that make expert popularity roughly Zipf(s).

    With i.i.d. Gumbel logits of scale beta, adding beta*ln(p_e) makes the top-1
    choice land on expert e with probability exactly p_e.  The router logits
    here are close to Gaussian with std ``logit_std``; the Gumbel scale of
    matching variance is logit_std*sqrt(6)/pi.  The realised shares are
    reported, not asserted.  Expert 0 is the most popular.
    """
    e = torch.arange(1, E + 1, dtype=torch.float64)
    p = e.pow(-s)
    p = p / p.sum()
    beta = logit_std * math.sqrt(6.0) / math.pi
    return (beta * torch.log(p)).to(torch.float32)


def make_inputs(cfg: dict, device="cpu", weights=True) -> dict:
    """Draw every input tensor of a workload (on ``device``).

    Draw order and seeds are fixed per tensor, so any tensor can be redrawn
    alone.  ``weights=False`` skips the expert weights (route/dispatch tests).
    """
    N, d, h, E = cfg["N"], cfg["d"], cfg["h"], cfg["E"]
    dt = torch_dtype(cfg)
    out = {}
    if cfg["name"] == "toy" and cfg.get("size") == "full" and device == "cpu":
        # The glossary snippet's own stream: seed 0, randn(4096, 512), Linear(512, 8).
        torch.manual_seed(0)
        x = torch.randn(N, d)
        router = torch.nn.Linear(d, E)
        out["x"] = x
        out["w_router"] = router.weight.detach().clone()
        out["router_bias"] = router.bias.detach().clone()
    else:
        out["x"] = _normal(cfg, "x", (N, d), 1.0, device)
        bound = 1.0 / math.sqrt(d)
        out["w_router"] = _uniform(cfg, "w_router", (E, d), bound, device)
        if cfg.get("router_bias") == "linear":
            out["router_bias"] = _uniform(cfg, "router_bias", (E,), bound, device,
                                          dtype=torch.float32)
        elif cfg.get("router_bias") == "zipf":
            # logit std of x ~N(0,1) against U(+-1/sqrt(d)) weights is 1/sqrt(3)
            out["router_bias"] = zipf_offsets(E, cfg["zipf"], 1.0 / math.sqrt(3.0)).to(device)
        else:
            out["router_bias"] = None
    sb = cfg.get("sel_bias")
    if sb is None:
        out["sel_bias"] = None
    elif sb == "zeros":
        out["sel_bias"] = torch.zeros(E, dtype=torch.float32, device=device)
    else:
        g = _gen(cfg, "sel_bias", device)
        out["sel_bias"] = torch.randn(E, generator=g, device=device,
                                      dtype=torch.float32) * float(sb)
    if weights:
        chunk = max(1, (1 << 28) // max(1, h * d))  # bound fp32 temporaries to ~1 GiB
        if cfg["name"] == "toy" and cfg.get("size") == "full" and device == "cpu":
            g = torch.Generator().manual_seed(101)
            out["w1"] = (torch.randn(E, h, d, generator=g) * 0.02).to(dt)
            out["w3"] = None
            out["w2"] = (torch.randn(E, d, h, generator=g) * 0.02).to(dt)
        else:
            out["w1"] = _normal(cfg, "w1", (E, h, d), 0.02, device, chunk)
            out["w3"] = (_normal(cfg, "w3", (E, h, d), 0.02, device, chunk)
                         if cfg["act"] == "swiglu" else None)
            out["w2"] = _normal(cfg, "w2", (E, d, h), 0.02, device, chunk)
        if cfg.get("shared"):
            out["shared"] = (
                _normal(cfg, "shared_w1", (1, h, d), 0.02, device),
                _normal(cfg, "shared_w3", (1, h, d), 0.02, device) if cfg["act"] == "swiglu" else None,
                _normal(cfg, "shared_w2", (1, d, h), 0.02, device),
            )
        else:
            out["shared"] = None
    return out


def to_numpy(t):
    """Tensor -> numpy for the oracle: bf16 becomes its uint16 bit pattern."""
    if t is None:
        return None
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    return t.numpy()


def from_numpy_bf16(a) -> torch.Tensor:
    import numpy as np
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
