"""Device router against the oracle's router (top-k with a taken flag per
expert, ties to the lower id, NaN ranking as -infinity; softmax over the
picked logits).  Picks are unique, so ids must match exactly; the weights are
f32 arithmetic against the oracle's double, so they match to a few ulp."""
import numpy as np
import pytest
import torch

import grouped_int4_expert_amd as qm
import synth
from gpu_util import Layer, orc, rel_l2, say, F32_TOL

pytestmark = pytest.mark.gpu
DEV = "cuda"
W_TOL = 1e-6    # max |w_gpu - w_oracle|; weights are in [0, 1]


def _check(logits, k, what):
    say(f"route {what}: T={logits.shape[0]} E={logits.shape[1]} k={k}")
    ids, w = qm.qmoe_route(logits.to(DEV), k)
    ids, w = ids.cpu().numpy(), w.cpu().numpy()
    rids, rw = orc().route(logits.numpy(), k)
    bad = np.nonzero((ids != rids).any(axis=1))[0]
    assert bad.size == 0, (what, int(bad[0]), ids[bad[0]].tolist(), rids[bad[0]].tolist())
    fin = np.isfinite(rw)
    assert np.array_equal(np.isfinite(w), fin)
    err = float(np.abs(w[fin].astype(np.float64) - rw[fin]).max()) if fin.any() else 0.0
    say(f"  max |dw| = {err:.2e}")
    assert err <= W_TOL


@pytest.mark.parametrize("T,E,k,kind,seed", [
    (1, 128, 8, "normal", 2), (4, 128, 8, "normal", 2), (16, 128, 8, "normal", 2),
    (8192, 128, 8, "uniform", 3), (64, 256, 8, "zipf", 4), (2048, 256, 8, "zipf", 4),
    (37, 1000, 16, "normal", 5), (9, 64, 16, "normal", 6), (5, 16, 16, "normal", 7),
    (7, 65, 1, "normal", 8), (3, 1, 1, "normal", 9), (130, 1024, 8, "normal", 10)])
def test_route_random(T, E, k, kind, seed):
    wl = synth.Workload("route", E, 64, 64, k, T, "f32", kind, seed)
    logits = synth.make_logits(wl, synth.generator(seed), T)
    _check(logits, k, kind)


def test_route_ties_and_specials():
    g = synth.generator(11)
    T, E = 64, 96
    # few distinct values: many equal logits per row
    logits = torch.randint(-2, 3, (T, E), generator=g).to(torch.float32) * 0.5
    logits[0] = 1.0                                   # all equal
    logits[1, :] = -float("inf")
    logits[1, 17] = 0.0
    logits[2, ::3] = float("nan")
    logits[3, 5] = float("inf")
    logits[4, 40:] = float("nan")
    _check(logits, 8, "ties/specials")
    _check(logits, 16, "ties/specials k16")


def test_route_feeds_layer():
    # logits -> device router -> device layer, against oracle router -> oracle layer
    say("route -> layer, E=16 H=256 F=128 T=40 k=4 f32")
    L = Layer(16, 256, 128, seed=25)
    g = synth.generator(26)
    x = synth.rand_x(g, (40, 256))
    logits = synth.normal_logits(g, 40, 16)
    ids, w = qm.qmoe_route(logits.to(DEV), 4)
    out = qm.qmoe_layer(L.dev, x.to(DEV), ids, w).cpu().numpy()
    rids, rw = orc().route(logits.numpy(), 4)
    ref = L.oracle_layer(x, torch.from_numpy(rids), torch.from_numpy(rw))
    err = rel_l2(out, ref)
    say(f"  rel_l2 = {err:.3e}")
    assert err <= F32_TOL


# (512, 512, bf16, 40 tokens: every expert takes the prefill passes)
@pytest.mark.parametrize("dtype,T,H,F", [("f32", 9, 256, 128), ("bf16", 300, 256, 128),
                                         ("bf16", 40, 512, 512)])
def test_layer_logits_matches_route_then_layer(dtype, T, H, F):
    say(f"layer from logits E=16 H={H} F={F} T={T} k=4 {dtype}")
    L = Layer(16, H, F, seed=27)
    g = synth.generator(28)
    x = synth.rand_x(g, (T, H))
    if dtype == "bf16":
        x = synth.to_bf16_rne(x)
    logits = synth.normal_logits(g, T, 16)
    out = qm.qmoe_layer_logits(L.dev, x.to(DEV), logits.to(DEV), 4).cpu().numpy()
    rids, rw = orc().route(logits.numpy(), 4)
    ref = L.oracle_layer(x.float() if dtype == "bf16" else x, torch.from_numpy(rids),
                         torch.from_numpy(rw))
    err = rel_l2(out, ref)
    say(f"  rel_l2 = {err:.3e}")
    assert err <= (F32_TOL if dtype == "f32" else 2e-3)
