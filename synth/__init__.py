"""Seeded synthetic inputs for the int4-g64 MoE expert path.

This module only draws random numbers and routes them; it holds none of the
expert-matmul arithmetic (no packing, no dequantisation, no matmul).  Both the
CPU oracle (``oracle/``) and the GPU path (``grouped_int4_expert_amd``) take
their inputs from here, so the two sides never share anything else.

Distributions (one f32 scale per 64 inputs, uniform signed int4, N(0,1)
activations, top-k routing renormalised over the chosen k) follow the workload
statements that accompany the grouped-int4 (fmt=4, gs=64) pull request
"cuda+engine: full fmt=4 (grouped int4 gs=64) support" (Summary / Problem:
one f32 scale per 64 elements).  Where that page is silent (the logit
distributions, Zipf popularity) the plainest reading is taken:

* router logits ~ N(0,1) for the small decode layer, U(0,1) for the 8K
  prefill layer;
* Zipf(s) popularity: expert of rank r (1-based) has p_r proportional to
  r**-s, ranks are assigned to expert ids by a seeded permutation, and each
  token's logits are ``log p_e + Gumbel(0,1)`` so that top-k is sampling
  without replacement proportional to p;
* top-k: k rounds of "largest logit among experts not yet taken" (a
  taken-flag array, ties to the lower expert id), slot order = descending
  logit; weights = softmax over the k chosen logits in fp64, rounded to f32.

Draw order inside one workload: q, s, x, logits.  Everything uses
``torch.Generator`` on the CPU unless a device generator is asked for
explicitly (large benchmark weights).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

GROUP = 64


def generator(seed: int, device: str = "cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def rand_q(gen: torch.Generator, shape, device="cpu") -> torch.Tensor:
    """Uniform signed int4 codes in [-8, 7] as int8."""
    return torch.randint(-8, 8, tuple(shape), generator=gen, dtype=torch.int8,
                         device=device)


def rand_scales(gen: torch.Generator, shape, lo=0.005, hi=0.02,
                device="cpu") -> torch.Tensor:
    """f32 group scales ~ U(lo, hi)."""
    u = torch.rand(tuple(shape), generator=gen, dtype=torch.float32,
                   device=device)
    return lo + (hi - lo) * u


def rand_x(gen: torch.Generator, shape, device="cpu") -> torch.Tensor:
    """f32 activations ~ N(0, 1)."""
    return torch.randn(tuple(shape), generator=gen, dtype=torch.float32,
                       device=device)


def normal_logits(gen, tokens, experts):
    return torch.randn((tokens, experts), generator=gen, dtype=torch.float32)


def uniform_logits(gen, tokens, experts):
    return torch.rand((tokens, experts), generator=gen, dtype=torch.float32)


def zipf_logits(gen, tokens, experts, s=1.1):
    """log p_e + Gumbel(0,1): top-k of these samples k experts without
    replacement with probability proportional to the Zipf(s) popularity."""
    perm = torch.randperm(experts, generator=gen)
    ranks = torch.empty(experts, dtype=torch.float64)
    ranks[perm] = torch.arange(1, experts + 1, dtype=torch.float64)
    logp = -s * torch.log(ranks)
    logp = logp - torch.logsumexp(logp, 0)
    u = torch.rand((tokens, experts), generator=gen, dtype=torch.float64)
    u = u.clamp_(min=1e-300)
    gumbel = -torch.log(-torch.log(u))
    return (logp[None, :] + gumbel).to(torch.float32)


def route_topk(logits: torch.Tensor, k: int):
    """Host router used only to make routing inputs.

    k rounds of "max over experts not yet taken" with a strict '>' so ties go
    to the lower expert id; softmax over the k chosen logits in fp64, rounded
    to f32.  Returns (ids int32 [T,k], weights f32 [T,k]).
    """
    lg = logits.detach().to(torch.float64).cpu().numpy()
    T, E = lg.shape
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    for t in range(T):
        taken = np.zeros(E, dtype=bool)
        picked = []
        row = lg[t]
        for _ in range(k):
            best = -1
            for e in range(E):
                if taken[e]:
                    continue
                if best < 0 or row[e] > row[best]:
                    best = e
            taken[best] = True
            picked.append(best)
        ids[t] = picked
        sel = row[picked]
        ex = np.exp(sel - sel.max())
        w[t] = (ex / ex.sum()).astype(np.float32)
    return torch.from_numpy(ids), torch.from_numpy(w)


def route_topk_fast(logits: torch.Tensor, k: int):
    """Vectorised equivalent of :func:`route_topk` for large token counts.

    A stable descending sort keeps equal logits in ascending expert order,
    which is the same tie rule as the taken-flag loop."""
    lg = logits.detach().to(torch.float64).cpu()
    order = torch.sort(lg, dim=1, descending=True, stable=True).indices[:, :k]
    sel = torch.gather(lg, 1, order)
    w = torch.softmax(sel, dim=1).to(torch.float32)
    return order.to(torch.int32).contiguous(), w.contiguous()


def to_bf16_rne(x: torch.Tensor) -> torch.Tensor:
    """f32 -> bf16 with round-to-nearest-even (torch's cast does RNE)."""
    return x.to(torch.bfloat16)


@dataclass
class Workload:
    """One named, seeded workload shape."""
    name: str
    experts: int
    hidden: int
    inter: int
    topk: int
    tokens: int
    x_dtype: str            # "f32" (decode path) or "bf16" (prefill path)
    logits: str             # "normal" | "uniform" | "zipf"
    seed: int
    zipf_s: float = 1.1
    extra: dict = field(default_factory=dict)


# Workloads.  The single matvec (256 x 1024, seed 0) and the single expert
# (4096/1536) are separate shapes; the layers below share one set of draws per
# name.
MATVEC = dict(name="matvec_256x1024", rows=256, cols=1024, batch=1, seed=0)
EXPERT = dict(name="expert_ffn_h4096_f1536", hidden=4096, inter=1536,
              batch=1, seed=1)
LAYERS = {
    "decode_e128_t1": Workload("decode_e128_t1", 128, 4096, 1536, 8, 1,
                               "f32", "normal", 2),
    "decode_e128_t4": Workload("decode_e128_t4", 128, 4096, 1536, 8, 4,
                               "f32", "normal", 2),
    "decode_e128_t16": Workload("decode_e128_t16", 128, 4096, 1536, 8, 16,
                                "f32", "normal", 2),
    "prefill_e128_t8192": Workload("prefill_e128_t8192", 128, 4096, 1536, 8,
                                   8192, "bf16", "uniform", 3),
    "decode_e256_t64_zipf": Workload("decode_e256_t64_zipf", 256, 6144, 2048,
                                     8, 64, "f32", "zipf", 4),
    "prefill_e256_t2048_zipf": Workload("prefill_e256_t2048_zipf", 256, 6144,
                                        2048, 8, 2048, "bf16", "zipf", 4),
}


def make_logits(wl: Workload, gen, tokens=None):
    t = wl.tokens if tokens is None else tokens
    if wl.logits == "normal":
        return normal_logits(gen, t, wl.experts)
    if wl.logits == "uniform":
        return uniform_logits(gen, t, wl.experts)
    if wl.logits == "zipf":
        return zipf_logits(gen, t, wl.experts, wl.zipf_s)
    raise ValueError(wl.logits)


def layer_weights(gen, experts, hidden, inter, device="cpu", group=GROUP):
    """Stacked int4 codes and scales for gate/up [E,F,H] and down [E,H,F],
    one scale per `group` inputs (64 unless asked otherwise).

    Draw order q (gate, up, down), then s (gate, up, down)."""
    qg = rand_q(gen, (experts, inter, hidden), device)
    qu = rand_q(gen, (experts, inter, hidden), device)
    qd = rand_q(gen, (experts, hidden, inter), device)
    sg = rand_scales(gen, (experts, inter, math.ceil(hidden / group)),
                     device=device)
    su = rand_scales(gen, (experts, inter, math.ceil(hidden / group)),
                     device=device)
    sd = rand_scales(gen, (experts, hidden, math.ceil(inter / group)),
                     device=device)
    return dict(qg=qg, qu=qu, qd=qd, sg=sg, su=su, sd=sd)


def layer_inputs(wl: Workload, gen, tokens=None, device="cpu"):
    """x (f32 N(0,1), or its RNE bf16 image) and routing for a layer."""
    t = wl.tokens if tokens is None else tokens
    x = rand_x(gen, (t, wl.hidden), device)
    if wl.x_dtype == "bf16":
        x = to_bf16_rne(x)
    logits = make_logits(wl, gen, t)
    router = route_topk if t * wl.experts <= 64 * 256 else route_topk_fast
    ids, w = router(logits, wl.topk)
    return x, ids, w
