"""Helpers shared by the GPU parity tests: seeded inputs from ``synth``,
device layers built through qmoe_pack, the oracle fed with the same codes,
and the relative-L2 metric."""
from __future__ import annotations

import sys

import numpy as np
import torch

import grouped_int4_expert_amd as qm
import oracle
import synth

F32_TOL = 1e-4     # decode path (f32 activations), relative L2
BF16_TOL = 2e-3    # prefill path (bf16 activations, MFMA), relative L2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_l2(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


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

    def oracle_subset(self, experts):
        """Oracle-packed stacks of the listed experts (ids remapped 0..n-1)."""
        o = orc()
        sel = torch.as_tensor(list(experts), dtype=torch.long)

        def cpu(t):
            return t.index_select(0, sel.to(t.device)).cpu().numpy()
        pg, _ = o.pack(cpu(self.q["qg"]))
        pu, _ = o.pack(cpu(self.q["qu"]))
        pd, _ = o.pack(cpu(self.q["qd"]))
        return pg, cpu(self.s["sg"]), pu, cpu(self.s["su"]), pd, cpu(self.s["sd"])

    def oracle_layer(self, x, ids, w, tokens=None):
        """Oracle output for the given token rows (all if tokens is None)."""
        x = x.detach().cpu()
        ids = ids.detach().cpu()
        w = w.detach().cpu()
        if tokens is not None:
            idx = torch.as_tensor(tokens, dtype=torch.long)
            x, ids, w = x[idx], ids[idx], w[idx]
        valid = ids[(ids >= 0) & (ids < self.E)]
        used = sorted(set(valid.tolist()))
        remap = {e: i for i, e in enumerate(used)}
        ids2 = ids.clone()
        for t in range(ids.shape[0]):
            for j in range(ids.shape[1]):
                e = int(ids[t, j])
                ids2[t, j] = remap[e] if e in remap else -1
        if not used:
            return np.zeros((x.shape[0], self.H))
        stacks = self.oracle_subset(used)
        out, _ = orc().layer(*stacks, self.H, self.F, x, ids2.numpy().astype(np.int32),
                             w.numpy(), gs=self.group)
        return out


def routing(wl: synth.Workload, gen, tokens=None):
    x, ids, w = synth.layer_inputs(wl, gen, tokens=tokens)
    return x, ids, w
