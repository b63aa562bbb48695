"""Experts resident in host memory behind an HBM slot cache: every call's
output must equal the oracle layer on the original routing (the cache only
moves bytes), across calls that hit, miss and evict; the slot bookkeeping
follows its stated policy."""
import numpy as np
import pytest
import torch

import grouped_int4_expert_amd as qm
import synth
from gpu_util import F32_TOL, BF16_TOL, Layer, orc, rel_l2, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _host_and_slots(L, slots):
    pin = lambda t: t.cpu().pin_memory()
    host = qm.HostLayer(pin(L.packed["qg"]), pin(L.s_dev["sg"]), pin(L.packed["qu"]),
                        pin(L.s_dev["su"]), pin(L.packed["qd"]), pin(L.s_dev["sd"]),
                        L.H, L.F, group=L.group)
    dev = {k: torch.zeros((slots,) + tuple(v.shape[1:]), dtype=v.dtype, device=DEV)
           for k, v in list(L.packed.items()) + list(L.s_dev.items())}
    slot_layer = qm.QLayer(dev["qg"], dev["sg"], dev["qu"], dev["su"], dev["qd"], dev["sd"],
                           L.H, L.F, group=L.group)
    return qm.ExpertCache(host, slot_layer), slot_layer


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_cache_calls_match_oracle(dtype):
    # calls alternate 3 and up to 6 experts: 9 of the 10 slots at most
    # (this call plus the previous one), so later calls evict
    E, H, F, slots = 14, 256, 128, 10
    say(f"cache E={E} slots={slots} {dtype}")
    L = Layer(E, H, F, seed=80)
    cache, slot_layer = _host_and_slots(L, slots)
    g = synth.generator(81)
    st = torch.cuda.current_stream()
    for call in range(8):
        T, k = (3, 2) if call % 2 else (1, 3)
        wl = synth.Workload("c", E, H, F, k, T, dtype, "normal", 82 + call)
        x, ids, w = synth.layer_inputs(wl, g)
        if call == 5:
            ids[0, 0] = -1                  # an invalid id stays invalid
            ids[-1, -1] = ids[-1, 0]        # a duplicate expert in one token
        slot_ids, nb = cache.prepare(ids.contiguous(), stream=st)
        used = sorted(set(int(e) for e in ids.flatten() if 0 <= e < E))
        assert all(cache.resident(e) >= 0 for e in used)
        assert all((slot_ids[t, j] == -1) == (not 0 <= ids[t, j] < E) for t in range(T)
                   for j in range(k))
        out = qm.qmoe_layer(slot_layer, x.to(DEV), slot_ids.to(DEV), w.to(DEV)).cpu().numpy()
        ref = L.oracle_layer(x, ids, w)
        err = rel_l2(out, ref)
        say(f"  call {call}: {len(used)} experts, {nb} B copied, rel_l2 {err:.2e}")
        assert err <= (F32_TOL if dtype == "f32" else BF16_TOL)
    cache.close()


def test_cache_policy():
    E, H, F, slots = 10, 128, 64, 4
    L = Layer(E, H, F, seed=83)
    cache, _ = _host_and_slots(L, slots)
    per_expert = 2 * (F * H // 2 + F * (H // 64) * 4) + (H * F // 2 + H * (F // 64) * 4)
    st = torch.cuda.current_stream()

    def call(ids):
        return cache.prepare(torch.tensor([ids], dtype=torch.int32), stream=st)

    _, nb = call([0, 1])
    assert nb == 2 * per_expert
    _, nb = call([2, 3])
    assert nb == 2 * per_expert
    _, nb = call([0, 1])                    # both still resident: nothing copied
    assert nb == 0
    # needs 4 (missing) and 0: may not evict 0/1 (this and the previous call)
    # so it takes the least recently used of 2 and 3
    slots_before = {e: cache.resident(e) for e in range(4)}
    _, nb = call([4, 0])
    assert nb == per_expert
    assert cache.resident(1) == slots_before[1] and cache.resident(0) == slots_before[0]
    assert sum(cache.resident(e) >= 0 for e in (2, 3)) == 1
    # this call plus the previous call's other slot exceed the 4 slots
    with pytest.raises(qm.QmoeError):
        call([5, 6, 7])
    torch.cuda.synchronize()
    cache.close()
