"""Helpers shared by the GPU parity tests: seeded inputs from ``synth``,
device layers built through qmoe_pack, the oracle fed with the same codes,
and the relative-L2 metric."""
from __future__ import annotations

import concurrent.futures as cf
import os
import sys

import numpy as np
import torch

import grouped_int4_expert_amd as qm
import oracle
import synth

F32_TOL = 1e-4     # decode path (f32 activations), relative L2
BF16_TOL = 2e-3    # prefill path (bf16 activations, MFMA), relative L2

# Per-element bounds |got - ref| <= C * u * M, M the oracle's first-order
# magnitude of the terms (matvec_abs / layer_mag; the maintainer comment
# "Here's the oracle you're missing": judge a result against the sum of the
# magnitudes of its terms).  Error model of each path:
#  * f32: every rounded quantity (a product's running sum, the scale product,
#    h, the routing-weight product, the atomic adds) carries at most one
#    rounding of u = 2^-24 per step of its longest chain: at most 32 FMAs per
#    lane chunk, 1 scale product, 6 DPP adds, 7 slice and atomic adds, the
#    SiLU (exp, add, divide, product: 4) -- C = 64 covers the depth of the
#    gate+up chain plus the down chain with room.  The matrix-core passes
#    (planned calls) form the products exactly (x and h as three f16 parts,
#    codes in f16) and round only in the additions: the MFMA's f32 sums of
#    32 products (two per 64-input group), the group-scale FMAs (8 per
#    512-input slice), the part and slice sums (at most 2 + 11) and the same
#    SiLU and atomic steps, a chain no deeper than the VALU one.
#  * bf16: q*s, h and every down product pass through one f16 rounding
#    (u = 2^-11 relative) that M counts once each; the f16 Y blocks add at
#    most one more, and the f32 accumulation is 2^13 times smaller: C = 2.
F32_C, F32_U = 64.0, 2.0 ** -24
BF16_C, BF16_U = 2.0, 2.0 ** -11
ORACLE_THREADS = max(1, min(16, os.cpu_count() or 1))


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_l2(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def check(got, ref, mag=None, path="f32", what=""):
    """Parity of a float output against the oracle: the same NaN pattern, the
    path's relative-L2 bar over the finite elements and, when the term
    magnitudes M are given, |got - ref| <= C u M element by element.  Returns
    (rel_l2, worst |got - ref| / (u M))."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    nan_ref = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan_ref), f"{what}: NaN pattern differs"
    fin = ~nan_ref
    assert np.array_equal(got[~fin], ref[~fin], equal_nan=True)
    inf_ref = np.isinf(ref) & fin
    assert np.array_equal(got[inf_ref], ref[inf_ref]), f"{what}: infinities differ"
    fin &= ~inf_ref
    tol = BF16_TOL if path == "bf16" else F32_TOL
    err = rel_l2(got[fin], ref[fin])
    assert err <= tol, f"{what}: rel_l2 {err:.3e} > {tol}"
    worst = None
    if mag is not None:
        c, u = (BF16_C, BF16_U) if path == "bf16" else (F32_C, F32_U)
        mag = np.asarray(mag, dtype=np.float64)
        d = np.abs(got - ref)[fin]
        scale = u * mag[fin] + 1e-38
        ratio = d / scale
        worst = float(ratio.max()) if ratio.size else 0.0
        nbad = int((ratio > c).sum())
        assert nbad == 0, (f"{what}: {nbad} elements with |got - ref| > {c} u M "
                           f"(worst {worst:.2f} u M)")
    say(f"  {what} rel_l2 = {err:.3e}" + ("" if worst is None else
                                           f", worst |err| = {worst:.2f} u M"))
    return err, worst


def cover_tokens(ids, E, tile=256, extra=(), pass_rows=0, pass_tile=16):
    """Tokens whose rows touch every tile of every expert's rows in the
    worklist (the stable sort of pairs by expert, cut into `tile`-row tiles,
    or into `pass_tile`-row passes for experts with at most `pass_rows`
    pairs): a greedy set cover, plus the given extra tokens.  ids int32
    [T, k]."""
    ids = np.asarray(ids)
    T, k = ids.shape
    wl = orc().worklist(ids.astype(np.int32), E)
    tiles = []
    for e in range(E):
        off, c = int(wl["offsets"][e]), int(wl["counts"][e])
        step = pass_tile if c <= pass_rows else tile
        for i in range(0, c, step):
            pos = wl["pairs"][off + i: off + min(i + step, c)]
            tiles.append(set(int(p) // k for p in pos))
    chosen = set(int(t) for t in extra)
    left = [tl for tl in tiles if not (tl & chosen)]
    while left:
        count = {}
        for tl in left:
            for t in tl:
                count[t] = count.get(t, 0) + 1
        best = max(sorted(count), key=lambda t: count[t])
        chosen.add(best)
        left = [tl for tl in left if best not in tl]
    return sorted(chosen)


def pass_rows_for(L, dtype):
    """qmoe_prefill_pass_rows() where layer L's bf16 call takes passes (hidden
    and inter multiples of 512, hidden up to 6144, inter up to 4608, groups of
    64 or more), else 0."""
    ok = (dtype == "bf16" and L.H % 512 == 0 and L.F % 512 == 0 and L.H <= 6144
          and L.F <= 4608 and L.group >= 64)
    return qm.qmoe_prefill_pass_rows() if ok else 0


_ORC = None


def orc():
    global _ORC
    if _ORC is None:
        _ORC = oracle.Oracle()
    return _ORC


class Layer:
    """Codes q (kept for the oracle) and the device layer packed by qmoe_pack."""

    def __init__(self, E, H, F, seed, device="cuda", gen_device="cpu", group=64):
        gen = synth.generator(seed, gen_device)
        w = synth.layer_weights(gen, E, H, F, device=gen_device, group=group)
        self.E, self.H, self.F, self.group = E, H, F, group
        self.q = {k: w[k] for k in ("qg", "qu", "qd")}
        self.s = {k: w[k] for k in ("sg", "su", "sd")}
        dq = {k: v.to(device) for k, v in self.q.items()}
        self.packed = {k: qm.qmoe_pack(v) for k, v in dq.items()}
        self.s_dev = {k: v.to(device).contiguous() for k, v in self.s.items()}
        del dq
        self.dev = qm.QLayer(self.packed["qg"], self.s_dev["sg"], self.packed["qu"],
                             self.s_dev["su"], self.packed["qd"], self.s_dev["sd"], H, F,
                             group=group)
        self.gen = gen

    def cpu_weights(self):
        """Host copies of the codes and scales (made once, on the calling
        thread, so that the oracle's worker threads never touch the GPU)."""
        if getattr(self, "_cpu", None) is None:
            self._cpu = {k: v.cpu() for k, v in list(self.q.items()) + list(self.s.items())}
        return self._cpu

    def oracle_subset(self, experts):
        """Oracle-packed stacks of the listed experts (ids remapped 0..n-1)."""
        o = orc()
        sel = torch.as_tensor(list(experts), dtype=torch.long)
        host = self.cpu_weights()

        def cpu(t):
            return t.index_select(0, sel).numpy()
        pg, _ = o.pack(cpu(host["qg"]))
        pu, _ = o.pack(cpu(host["qu"]))
        pd, _ = o.pack(cpu(host["qd"]))
        return pg, cpu(host["sg"]), pu, cpu(host["su"]), pd, cpu(host["sd"])

    def _oracle_rows(self, x, ids, w, mag):
        valid = ids[(ids >= 0) & (ids < self.E)]
        used = sorted(set(valid.tolist()))
        remap = {e: i for i, e in enumerate(used)}
        ids2 = ids.clone()
        for t in range(ids.shape[0]):
            for j in range(ids.shape[1]):
                e = int(ids[t, j])
                ids2[t, j] = remap[e] if e in remap else -1
        if not used:
            z = np.zeros((x.shape[0], self.H))
            return z, z.copy()
        stacks = self.oracle_subset(used)
        ids2 = ids2.numpy().astype(np.int32)
        out, _ = orc().layer(*stacks, self.H, self.F, x, ids2, w.numpy(), gs=self.group)
        m = orc().layer_mag(*stacks, self.H, self.F, x, ids2, w.numpy(),
                            gs=self.group) if mag else None
        return out, m

    def oracle_layer(self, x, ids, w, tokens=None, mag=False):
        """Oracle output for the given token rows (all if tokens is None);
        with mag=True also the term magnitudes M (returns (out, M)).  Tokens
        are split over threads (the oracle's C calls release the GIL)."""
        x = x.detach().cpu()
        ids = ids.detach().cpu()
        w = w.detach().cpu()
        if tokens is not None:
            idx = torch.as_tensor(tokens, dtype=torch.long)
            x, ids, w = x[idx], ids[idx], w[idx]
        self.cpu_weights()            # host copies first: the threads below run CPU code only
        T = x.shape[0]
        nchunk = max(1, min(ORACLE_THREADS, T))
        bounds = np.linspace(0, T, nchunk + 1).astype(int)
        parts = [(int(a), int(b)) for a, b in zip(bounds[:-1], bounds[1:]) if b > a]
        with cf.ThreadPoolExecutor(len(parts)) as ex:
            res = list(ex.map(lambda ab: self._oracle_rows(x[ab[0]:ab[1]], ids[ab[0]:ab[1]],
                                                           w[ab[0]:ab[1]], mag), parts))
        out = np.concatenate([r[0] for r in res], axis=0)
        if not mag:
            return out
        return out, np.concatenate([r[1] for r in res], axis=0)


def routing(wl: synth.Workload, gen, tokens=None):
    x, ids, w = synth.layer_inputs(wl, gen, tokens=tokens)
    return x, ids, w
