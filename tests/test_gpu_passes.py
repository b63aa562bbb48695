"""GPU parity of the bf16 prefill passes: experts that receive at most
qmoe_prefill_pass_rows() pairs are cut into passes of up to 16 pairs that
stream the expert's weights on the matrix cores, beside the row tiles of
the other experts (hidden and inter multiples of 512, groups of 64 or
more).  Every case is checked against the oracle element by element
(|got - ref| <= 2 u M, u = 2^-11) and by relative L2 (2e-3); the pass
borders (1, 15, 16, 17, 31, 32, 33 ... rows), the pass/tile threshold, one,
three and twelve waves across the input width, group sizes 128 and one per
row, the f16 range edges of the routed down outputs and a NaN in x are
covered."""
import numpy as np
import pytest
import torch

import grouped_int4_expert_amd as qm
import synth
from gpu_util import Layer, check, orc, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qm.load()
    yield
    torch.cuda.synchronize()


def _run(L, x, ids, w):
    return qm.qmoe_layer(L.dev, x.to(DEV), ids.to(DEV), w.to(DEV)).cpu().numpy()


def _inputs(L, T, k, seed, logits="normal"):
    wl = synth.Workload("t", L.E, L.H, L.F, k, T, "bf16", logits, seed)
    return synth.layer_inputs(wl, synth.generator(2000 + seed))


def _fixed_rows(counts, seed):
    """k = 1 routing that gives expert e exactly counts[e] rows, in a random
    token order."""
    T = sum(counts)
    perm = torch.randperm(T, generator=torch.Generator().manual_seed(seed))
    assign = torch.repeat_interleave(torch.arange(len(counts)), torch.tensor(counts))[perm]
    return assign.view(T, 1).to(torch.int32), T


def test_pass_rows_reported():
    pr = qm.qmoe_prefill_pass_rows()
    say(f"prefill pass rows: {pr}")
    assert 0 <= pr <= 256


@pytest.mark.parametrize("H,F", [(512, 512), (1536, 1024)])
def test_passes_every_row_count(H, F):
    # Expert e gets exactly counts[e] rows: passes end on and beside every
    # 16-row border, and the experts above the threshold take tiles in the
    # same call; each expert's rows are checked on their own.  Two calls
    # give identical bits.
    pr = qm.qmoe_prefill_pass_rows()
    counts = [1, 2, 3, 15, 16, 17, 31, 32, 33, 47, 48, 49, 63, 64, 65, 100, 0]
    if pr not in counts:
        counts += [pr, pr + 1]
    say(f"bf16 passes E={len(counts)} H={H} F={F} k=1, fixed rows per expert (threshold {pr})")
    L = Layer(len(counts), H, F, seed=71)
    assign, T = _fixed_rows(counts, 71)
    x, _, _ = _inputs(L, T, 1, 71)
    w = torch.ones(T, 1)
    out = _run(L, x, assign, w)
    again = _run(L, x, assign, w)
    assert np.array_equal(out.view(np.uint32), again.view(np.uint32)), "not bit-reproducible"
    ref, mag = L.oracle_layer(x, assign, w, mag=True)
    for e, c in enumerate(counts):
        if c == 0:
            continue
        rows = (assign[:, 0] == e).nonzero().flatten().numpy()
        kind = "passes" if c <= pr else "tiles"
        check(out[rows], ref[rows], mag[rows], "bf16", f"expert {e} ({c} rows, {kind})")
    check(out, ref, mag, "bf16", "layer")


@pytest.mark.parametrize("E,H,F,T,k", [(16, 1536, 1536, 40, 4), (8, 512, 512, 300, 2),
                                        (128, 4096, 1536, 24, 8)])
def test_passes_routed_layer(E, H, F, T, k):
    # Normal routing with several pairs per token: the combine adds rows
    # written by passes (and, at 300 tokens over 8 experts, by tiles) in pick
    # order.  4096/1536 at 24 tokens x top-8 is the decode-sized prefill
    # call: every expert takes passes.  Every token is checked.
    say(f"bf16 passes E={E} H={H} F={F} T={T} k={k}")
    L = Layer(E, H, F, seed=72 + T)
    x, ids, w = _inputs(L, T, k, 72 + T)
    out = _run(L, x, ids, w)
    ref, mag = L.oracle_layer(x, ids, w, mag=True)
    check(out, ref, mag, "bf16", "layer")


@pytest.mark.parametrize("group", [128, 512])
def test_passes_group_sizes(group):
    # groups of 128 and one scale per row (512 = the row width of every
    # matrix here)
    say(f"bf16 passes E=8 H=512 F=512 T=60 k=2 group {group}")
    L = Layer(8, 512, 512, seed=73, group=group)
    x, ids, w = _inputs(L, 60, 2, 73)
    out = _run(L, x, ids, w)
    ref, mag = L.oracle_layer(x, ids, w, mag=True)
    check(out, ref, mag, "bf16", f"layer group {group}")


def test_passes_outputs_beyond_f16_range():
    # Down scales x30000: per-pair down outputs beyond 65504 keep their
    # precision through the exponent of each row's 16-column block.
    say("bf16 passes with outputs beyond the f16 range")
    L = Layer(8, 512, 512, seed=74)
    L.s["sd"] = L.s["sd"] * 30000.0
    L.s_dev["sd"].mul_(30000.0)
    x, ids, w = _inputs(L, 50, 2, 74)
    out = _run(L, x, ids, w)
    ref, mag = L.oracle_layer(x, ids, w, mag=True)
    assert np.abs(ref).max() > 1e5
    assert np.isfinite(out).all()
    check(out, ref, mag, "bf16", f"layer, max |ref| = {np.abs(ref).max():.3e}")


def test_passes_tiny_routing_weights():
    # Routing weights ~1e-36: the exponent is clamped so that the scale
    # factors stay finite normal numbers.
    say("bf16 passes with routing weights x1e-36")
    L = Layer(8, 512, 512, seed=75)
    x, ids, w = _inputs(L, 50, 2, 75)
    w = w * 1e-36
    out = _run(L, x, ids, w)
    ref, mag = L.oracle_layer(x, ids, w, mag=True)
    assert np.abs(ref).max() < 2.0 ** -100
    assert np.isfinite(out).all()
    check(out, ref, mag, "bf16", f"layer, max |ref| = {np.abs(ref).max():.3e}")


def test_passes_nan_reaches_its_token_only():
    say("bf16 passes: NaN in one token")
    L = Layer(8, 512, 512, seed=76)
    g = synth.generator(77)
    x = synth.to_bf16_rne(synth.rand_x(g, (9, 512)))
    x[4, 77] = float("nan")
    ids, w = synth.route_topk_fast(synth.normal_logits(g, 9, 8), 2)
    out = _run(L, x, ids, w)
    ref = L.oracle_layer(x, ids, w)
    assert np.isnan(ref[4]).all()
    assert np.isnan(out[4]).all()
    keep = [t for t in range(9) if t != 4]
    assert np.isfinite(out[keep]).all()
    check(out[keep], ref[keep], None, "bf16", "other tokens")


def test_passes_worklist_lists_passes():
    # The worklist left in the workspace is the oracle's (passes change only
    # which kernel takes an expert, not the sort).
    say("bf16 passes: worklist in the workspace")
    L = Layer(16, 512, 512, seed=78)
    x, ids, w = _inputs(L, 50, 4, 78)
    ws = torch.empty(L.dev.workspace_bytes(50, 4, qm.QMOE_BF16), dtype=torch.uint8, device=DEV)
    qm.qmoe_layer(L.dev, x.to(DEV), ids.to(DEV), w.to(DEV), ws=ws)
    got = qm.layer_worklist_from_ws(L.dev, ws, 50, 4, qm.QMOE_BF16)
    ref = orc().worklist(ids.numpy(), 16)
    for key in ("counts", "offsets", "pairs", "inv"):
        assert np.array_equal(got[key].cpu().numpy(), ref[key]), key


def test_passes_max_experts_invalid_and_duplicate_ids():
    # E = 1024 (most experts get one pair or none), ids outside [0, E) in some
    # slots (dropped) and a repeated expert inside some tokens.
    say("bf16 passes E=1024 H=512 F=512 T=60 k=8, invalid and duplicate ids")
    L = Layer(1024, 512, 512, seed=79)
    x, ids, w = _inputs(L, 60, 8, 79)
    ids = ids.clone()
    ids[3, 2] = -1
    ids[7, 0] = 1024
    ids[11, 5] = 99999
    ids[20, 1] = ids[20, 0]
    ids[21, 4] = ids[21, 3]
    out = _run(L, x, ids, w)
    ref, mag = L.oracle_layer(x, ids, w, mag=True)
    check(out, ref, mag, "bf16", "layer")


def test_passes_graph_replays_match_eager():
    # The pass kernels under HIP graph capture (hidden 6144: the gate+up
    # passes use more than 64 KB of LDS): every replay (with a stale
    # workspace and eager work in between) gives the eager result bit for bit.
    say("bf16 passes: graph replays")
    L = Layer(4, 6144, 512, seed=80)
    x, ids, w = _inputs(L, 33, 2, 80)
    xd, idd, wd = x.to(DEV), ids.to(DEV), w.to(DEV)
    ws = torch.empty(L.dev.workspace_bytes(33, 2, qm.QMOE_BF16), dtype=torch.uint8, device=DEV)
    out = torch.empty(33, 6144, device=DEV)
    qm.qmoe_layer(L.dev, xd, idd, wd, out=out, ws=ws)
    torch.cuda.synchronize()
    eager = out.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=torch.cuda.Stream()):
        qm.qmoe_layer(L.dev, xd, idd, wd, out=out, ws=ws)
    for rep in range(4):
        out.fill_(float("nan"))
        ws.fill_(0xAB)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), rep


@pytest.mark.parametrize("F", [4608, 6144])
def test_passes_widest_inter(F):
    # inter 4608 is the widest whose down passes fit the LDS (9 waves, 153 KB);
    # at 6144 every expert takes tiles.  Either way the layer matches.
    say(f"bf16 E=8 H=512 F={F} T=20 k=2 (few pairs per expert)")
    L = Layer(8, 512, F, seed=81)
    x, ids, w = _inputs(L, 20, 2, 81)
    out = _run(L, x, ids, w)
    ref, mag = L.oracle_layer(x, ids, w, mag=True)
    check(out, ref, mag, "bf16", "layer")
