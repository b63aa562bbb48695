"""The bf16 (prefill) path's input range.  Its matrix-core operands are f16:
q * s is rounded to f16 per weight and the intermediate h is stored as f16.
Both stay within the path's error model while the scales are f16 normal
numbers (|s| >= 2^-14) and |h| < 65504; these tests sit at both edges:
scales just above 2^-14, and activations that drive max |h| to a few 1e4."""
import numpy as np
import pytest
import torch

import grouped_int4_expert_amd as qm
import synth
from gpu_util import BF16_TOL, Layer, check, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _rescaled_layer(E, H, F, seed, factor):
    """A Layer whose scales are multiplied by `factor` (device layer rebuilt,
    oracle copies reset)."""
    L = Layer(E, H, F, seed=seed)
    L.s = {k: (v * factor).contiguous() for k, v in L.s.items()}
    L.s_dev = {k: v.to(DEV).contiguous() for k, v in L.s.items()}
    L.dev = qm.QLayer(L.packed["qg"], L.s_dev["sg"], L.packed["qu"], L.s_dev["su"],
                      L.packed["qd"], L.s_dev["sd"], H, F, group=L.group)
    L._cpu = None
    return L


def _dense(q, s, group):
    """Dequantised f64 matrices [E][rows][cols] (q * s per group)."""
    q = q.double().numpy()
    s = s.double().numpy()
    return q * np.repeat(s, group, axis=2)[:, :, :q.shape[2]]


def _max_h(L, x, ids):
    G = _dense(L.q["qg"].cpu(), L.s["sg"].cpu(), L.group)
    U = _dense(L.q["qu"].cpu(), L.s["su"].cpu(), L.group)
    xd = x.double().numpy()
    m = 0.0
    for t in range(ids.shape[0]):
        for e in set(int(v) for v in ids[t]):
            g = G[e] @ xd[t]
            u = U[e] @ xd[t]
            h = g / (1.0 + np.exp(-g)) * u
            m = max(m, float(np.abs(h).max()))
    return m


def test_bf16_scales_just_above_f16_normal_limit():
    # scales in [2^-14 * 1.02, 4 * 2^-14]: every q * s is an f16 normal number
    E, H, F, T, k = 8, 512, 256, 96, 4
    lo = 2.0 ** -14 * 1.02
    L = _rescaled_layer(E, H, F, 110, 1.0)
    g = synth.generator(111)
    for key in ("sg", "su", "sd"):
        u = torch.rand(L.s[key].shape, generator=g, dtype=torch.float32)
        L.s[key] = (lo + u * 3 * 2.0 ** -14).contiguous()
    L.s_dev = {kk: v.to(DEV).contiguous() for kk, v in L.s.items()}
    L.dev = qm.QLayer(L.packed["qg"], L.s_dev["sg"], L.packed["qu"], L.s_dev["su"],
                      L.packed["qd"], L.s_dev["sd"], H, F, group=L.group)
    L._cpu = None
    wl = synth.Workload("r", E, H, F, k, T, "bf16", "normal", 112)
    x, ids, w = synth.layer_inputs(wl, g)
    out = qm.qmoe_layer(L.dev, x.to(DEV), ids.to(DEV), w.to(DEV)).cpu().numpy()
    ref, mag = L.oracle_layer(x.float(), ids, w, mag=True)
    err, worst = check(out, ref, mag, path="bf16", what="small scales")
    say(f"bf16 scales ~2^-14: rel_l2 {err:.2e}, worst {worst:.2f} u M")
    assert err <= BF16_TOL


def test_bf16_large_intermediate():
    # activations scaled so that max |h| lands between 1e4 and 6e4 (f16 holds
    # it; the per-element bound still applies)
    E, H, F, T, k = 8, 512, 256, 64, 4
    L = _rescaled_layer(E, H, F, 113, 1.0)
    g = synth.generator(114)
    wl = synth.Workload("r", E, H, F, k, T, "bf16", "normal", 115)
    x, ids, w = synth.layer_inputs(wl, g)
    m0 = _max_h(L, x.float(), ids)
    c = (3.0e4 / m0) ** 0.5
    x = synth.to_bf16_rne(x.float() * c)
    mh = _max_h(L, x.float(), ids)
    say(f"bf16 large h: x scaled by {c:.2f}, max |h| {mh:.3g}")
    assert 1.0e4 <= mh < 6.0e4
    out = qm.qmoe_layer(L.dev, x.to(DEV), ids.to(DEV), w.to(DEV)).cpu().numpy()
    ref, mag = L.oracle_layer(x.float(), ids, w, mag=True)
    err, worst = check(out, ref, mag, path="bf16", what="large h")
    say(f"  rel_l2 {err:.2e}, worst {worst:.2f} u M")
    assert np.isfinite(out).all()
    assert err <= BF16_TOL
