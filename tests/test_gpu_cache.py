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


class _PolicyModel:
    """The device prepare's residency policy, step by step: resident experts
    keep their slots; the missing ones, in ascending id order, take the
    candidate slots (not used by this call or kept from the previous one)
    oldest first: free slots by index, then by last use, then by index."""

    def __init__(self, E, S):
        self.E, self.S = E, S
        self.slot_of = [-1] * E
        self.expert_in = [-1] * S
        self.last_use = [0] * S
        self.keep = [False] * S
        self.tick = 0
        self.status = 0

    def call(self, ids):
        need = sorted(set(int(e) for e in ids if 0 <= e < self.E))
        used = {self.slot_of[e] for e in need if self.slot_of[e] >= 0}
        missing = [e for e in need if self.slot_of[e] < 0]
        cand = [s for s in range(self.S) if s not in used and not self.keep[s]]
        cand.sort(key=lambda s: (0 if self.expert_in[s] < 0 else self.last_use[s] + 1, s))
        placed = min(len(missing), len(cand))
        copies = []
        for e, s in zip(missing[:placed], cand[:placed]):
            if self.expert_in[s] >= 0:
                self.slot_of[self.expert_in[s]] = -1
            self.expert_in[s] = e
            self.slot_of[e] = s
            used.add(s)
            copies.append(e)
        self.tick += 1
        for s in range(self.S):
            if s in used:
                self.last_use[s] = self.tick
            self.keep[s] = s in used
        if len(missing) > len(cand):
            self.status = 1
        return copies


def _state_tables(state, E, S):
    st = state.cpu().numpy()
    return dict(tick=int(st[0]), status=int(st[1]), n_copy=int(st[2]),
                slot_of=st[4:4 + E].tolist(), expert_in=st[4 + E:4 + E + S].tolist())


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_cache_device_prepare_matches_oracle_and_policy(dtype):
    # the routing ids stay on the device: the slots are chosen and filled by
    # the GPU; outputs equal the oracle on the original ids, the residency
    # tables follow the policy model exactly, and every resident slot holds
    # its expert's bytes
    E, H, F, slots = 14, 256, 128, 10
    say(f"device cache E={E} slots={slots} {dtype}")
    L = Layer(E, H, F, seed=90)
    cache, slot_layer = _host_and_slots(L, slots)
    st = torch.cuda.current_stream()
    state = cache.device_state(stream=st)
    model = _PolicyModel(E, slots)
    g = synth.generator(91)
    for call in range(10):
        T, k = (3, 2) if call % 2 else (1, 3)
        wl = synth.Workload("c", E, H, F, k, T, dtype, "normal", 92 + call)
        x, ids, w = synth.layer_inputs(wl, g)
        if call == 5:
            ids[0, 0] = -1
            ids[-1, -1] = ids[-1, 0]
        ids_d = ids.to(DEV).contiguous()
        slot_ids = cache.prepare_device(state, ids_d, stream=st)
        out = qm.qmoe_layer(slot_layer, x.to(DEV), slot_ids, w.to(DEV)).cpu().numpy()
        copies = model.call(ids.flatten().tolist())
        tab = _state_tables(state, E, slots)
        assert tab["status"] == 0 and tab["tick"] == call + 1
        assert tab["n_copy"] == len(copies)
        assert tab["expert_in"] == model.expert_in and tab["slot_of"] == model.slot_of
        sid = slot_ids.cpu()
        for t in range(T):
            for j in range(k):
                e = int(ids[t, j])
                assert int(sid[t, j]) == (model.slot_of[e] if 0 <= e < E else -1)
        for s, e in enumerate(model.expert_in):
            if e < 0:
                continue
            for name, src in (("qg", L.packed["qg"]), ("qu", L.packed["qu"]),
                              ("qd", L.packed["qd"]), ("sg", L.s_dev["sg"]),
                              ("su", L.s_dev["su"]), ("sd", L.s_dev["sd"])):
                i = ("qg", "sg", "qu", "su", "qd", "sd").index(name)
                assert torch.equal(slot_layer.tensors[i][s].cpu(), src[e].cpu()), (call, s, e, name)
        ref = L.oracle_layer(x, ids, w)
        err = rel_l2(out, ref)
        say(f"  call {call}: {len(copies)} copied, rel_l2 {err:.2e}")
        assert err <= (F32_TOL if dtype == "f32" else BF16_TOL)
    cache.close()


def test_cache_device_prepare_overflow_sets_status():
    # a call whose experts plus the previous call's other slots exceed the
    # slots: the experts without a slot route to -1 and the status word is set
    E, H, F, slots = 10, 128, 64, 4
    L = Layer(E, H, F, seed=95)
    cache, slot_layer = _host_and_slots(L, slots)
    st = torch.cuda.current_stream()
    state = cache.device_state(stream=st)
    model = _PolicyModel(E, slots)
    for ids in ([0, 1], [2, 3], [5, 6, 7]):
        ids_d = torch.tensor([ids], dtype=torch.int32, device=DEV)
        sid = cache.prepare_device(state, ids_d, stream=st).cpu()
        model.call(ids)
        tab = _state_tables(state, E, slots)
        assert tab["status"] == model.status
        assert tab["expert_in"] == model.expert_in
        assert [int(v) for v in sid[0]] == [model.slot_of[e] for e in ids]
    assert model.status == 1 and _state_tables(state, E, slots)["status"] == 1
    assert [model.slot_of[e] for e in (5, 6, 7)].count(-1) == 1
    cache.close()
