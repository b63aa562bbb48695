"""GPU parity: every C-ABI entry point against the CPU oracle on the same
seeded inputs.  Integer work (pack, worklist) is bit-exact; floating outputs
meet relative L2 <= 1e-4 on the f32 (decode) path and <= 2e-3 on the bf16
(prefill, MFMA) path, and element by element |got - ref| <= C u M with M the
oracle's term magnitudes (gpu_util.check).  Full-size layers are checked on
token samples chosen so that every worklist tile (expert x 256-row part) of
the launch has rows among them; decode sizes check every token."""
import numpy as np
import pytest
import torch

import grouped_int4_expert_amd as qm
import synth
from gpu_util import (BF16_TOL, F32_TOL, Layer, check, cover_tokens, orc, pass_rows_for,
                      rel_l2, say)

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qm.load()
    yield
    torch.cuda.synchronize()


# ------------------------------------------------------------------ pack ---

@pytest.mark.parametrize("rows,cols", [(1, 1), (3, 5), (7, 64), (33, 4097), (256, 1024)])
def test_pack_bit_exact(rows, cols):
    say(f"pack {rows}x{cols}")
    g = synth.generator(100 + rows + cols)
    q = synth.rand_q(g, (rows, cols))
    ref, bad = orc().pack(q.numpy())
    got = qm.qmoe_pack(q.to(DEV))
    assert np.array_equal(got.cpu().numpy(), ref)
    back = qm.qmoe_unpack(got, cols)
    assert torch.equal(back.cpu(), q)


def test_pack_counts_out_of_range():
    say("pack out of range")
    q = torch.tensor([[8, -9, 0, 7, 127, -128]], dtype=torch.int8)
    ref, bad = orc().pack(q.numpy())
    got, nbad = qm.qmoe_pack(q.to(DEV), count_bad=True)
    assert np.array_equal(got.cpu().numpy(), ref)
    assert int(nbad.item()) == bad == 4


def test_pack_all_bytes_roundtrip():
    say("unpack all bytes")
    allb = torch.arange(256, dtype=torch.uint8).reshape(256, 1)
    got = qm.qmoe_unpack(allb.to(DEV), 2).cpu().numpy()
    assert np.array_equal(got, orc().unpack(allb.numpy(), 2))


# -------------------------------------------------------------- worklist ---

def _wl_check(ids, E):
    ref = orc().worklist(ids.numpy(), E)
    got = qm.qmoe_worklist(ids.to(DEV), E)
    for key in ("counts", "offsets", "pairs", "inv"):
        assert np.array_equal(got[key].cpu().numpy(), ref[key]), key
    assert int(got["n_invalid"].item()) == ref["n_invalid"]


def test_worklist_64_random_cases():
    rng = np.random.default_rng(7)
    for case in range(64):
        T = int(rng.integers(0, 300))
        k = int(rng.integers(1, 9))
        E = int(rng.integers(1, 300))
        ids = torch.from_numpy(rng.integers(-2, E + 2, size=(T, k)).astype(np.int32))
        say(f"worklist case {case}: T={T} k={k} E={E}")
        _wl_check(ids, E)


@pytest.mark.parametrize("T,k,E", [(8192, 8, 128), (2048, 8, 256), (5000, 3, 1024),
                                   (4096, 2, 1)])
def test_worklist_large_multiblock(T, k, E):
    say(f"worklist large T={T} k={k} E={E}")
    g = synth.generator(T + E)
    logits = torch.rand((T, E), generator=g)
    ids, _ = synth.route_topk_fast(logits, min(k, E))
    if ids.shape[1] < k:
        ids = ids.repeat(1, k)[:, :k].contiguous()
    ids[::97, 0] = -1          # a sprinkle of dropped ids
    ids[::89, -1] = E
    _wl_check(ids, E)


# ---------------------------------------------------------------- matvec ---

def _matvec_inputs(rows, cols, seed, batch=1):
    g = synth.generator(seed)
    q = synth.rand_q(g, (rows, cols))
    s = synth.rand_scales(g, (rows, cols // 64))
    x = synth.rand_x(g, (batch, cols))
    return q, s, x


def test_matvec_one_hot_bit_exact():
    """x = e_j: y[o] = fl(s[o, j/64] * q[o, j]) exactly, which pins nibble
    order, offset and scale index in the kernel."""
    rows, cols = 37, 192
    q, s, _ = _matvec_inputs(rows, cols, 5)
    pq = qm.qmoe_pack(q.to(DEV))
    sd = s.to(DEV)
    for j in (0, 1, 31, 32, 63, 64, 127, 130, 191):
        say(f"matvec one-hot j={j}")
        x = torch.zeros(1, cols)
        x[0, j] = 1.0
        y = qm.qmoe_matvec(pq, sd, cols, x.to(DEV)).cpu().numpy()[0]
        want = (q[:, j].double().numpy() * s[:, j // 64].double().numpy()).astype(np.float32)
        assert np.array_equal(y, want), j


@pytest.mark.parametrize("rows,cols,batch,seed", [(256, 1024, 1, 0), (100, 320, 3, 9),
                                                  (64, 6144, 2, 10), (513, 1536, 1, 11),
                                                  (37, 12288, 2, 12), (70, 8256, 1, 13),
                                                  (45, 4160, 3, 14)])
def test_matvec_random(rows, cols, batch, seed):
    say(f"matvec {rows}x{cols} batch {batch}")
    q, s, x = _matvec_inputs(rows, cols, seed, batch)
    y = qm.qmoe_matvec(qm.qmoe_pack(q.to(DEV)), s.to(DEV), cols, x.to(DEV)).cpu().numpy()
    pq, _ = orc().pack(q.numpy())
    ref = orc().matvec(pq, s.numpy(), cols, x.numpy())
    mag = orc().matvec_abs(pq, s.numpy(), cols, x.numpy())
    check(y, ref, mag, "f32", f"matvec {rows}x{cols}")


# ------------------------------------------------------------ expert ffn ---

@pytest.mark.parametrize("H,F,batch,dtype", [(4096, 1536, 1, "f32"), (4096, 1536, 1, "bf16"),
                                             (256, 128, 5, "f32"), (256, 128, 130, "bf16"),
                                             (256, 128, 600, "bf16")])
def test_expert_ffn(H, F, batch, dtype):
    say(f"expert ffn H={H} F={F} batch={batch} {dtype}")
    L = Layer(1, H, F, seed=1)
    x = synth.rand_x(L.gen, (batch, H))
    if dtype == "bf16":
        x = x.to(torch.bfloat16)
    out = qm.qmoe_expert_ffn(L.packed["qg"][0], L.s_dev["sg"][0], L.packed["qu"][0],
                             L.s_dev["su"][0], L.packed["qd"][0], L.s_dev["sd"][0], H, F,
                             x.to(DEV)).cpu().numpy()
    st = L.oracle_subset([0])
    ref = orc().ffn(st[0][0], st[1][0], st[2][0], st[3][0], st[4][0], st[5][0], H, F, x)
    _, mag = L.oracle_layer(x, torch.zeros(batch, 1, dtype=torch.int32), torch.ones(batch, 1),
                            mag=True)
    check(out, ref, mag, dtype, "expert ffn")


# ----------------------------------------------------------------- layer ---

def _layer_case(L, T, k, dtype, logits="normal", seed=0, tokens=None, mutate=None,
                cover=False):
    """Run the layer on the GPU and the oracle on `tokens` (all if None; with
    cover=True a set of tokens touching every worklist tile, plus `tokens`).
    Returns (out, ref, mag) on the checked tokens."""
    g = synth.generator(1000 + seed)
    wl = synth.Workload("t", L.E, L.H, L.F, k, T, dtype, logits, seed)
    x, ids, w = synth.layer_inputs(wl, g)
    if mutate:
        ids, w = mutate(ids, w)
    out = qm.qmoe_layer(L.dev, x.to(DEV), ids.to(DEV), w.to(DEV)).cpu().numpy()
    if cover:
        tokens = cover_tokens(ids.numpy(), L.E, 256, extra=tokens or (),
                              pass_rows=pass_rows_for(L, dtype))
        say(f"  {len(tokens)} tokens cover every worklist tile")
    ref, mag = L.oracle_layer(x, ids, w, tokens, mag=True)
    if tokens is not None:
        out = out[np.asarray(tokens)]
    return out, ref, mag


@pytest.mark.parametrize("dtype,T,k", [("f32", 1, 4), ("f32", 37, 4), ("bf16", 37, 4),
                                       ("bf16", 300, 4), ("f32", 300, 2)])
def test_layer_small_full(dtype, T, k):
    say(f"layer small E=16 H=256 F=128 T={T} k={k} {dtype}")
    L = Layer(16, 256, 128, seed=21)
    out, ref, mag = _layer_case(L, T, k, dtype, seed=T)
    check(out, ref, mag, dtype, "layer")


@pytest.mark.parametrize("T,k", [(777, 2), (1500, 1)])
def test_layer_bf16_multi_tile(T, k):
    # Few experts and many tokens: each expert spans several 256-row tiles
    # plus a ragged tail that ends inside a 32-row fragment.
    say(f"layer multi-tile E=4 H=256 F=128 T={T} k={k} bf16")
    L = Layer(4, 256, 128, seed=24)
    out, ref, mag = _layer_case(L, T, k, "bf16", seed=T)
    check(out, ref, mag, "bf16", "layer")


def test_layer_bf16_every_fragment_count():
    # Expert e gets exactly COUNTS[e] rows, so tiles end after each number of
    # 32-row fragments (1 .. 8), on and beside fragment and tile borders;
    # every expert's rows are checked on their own.
    counts = [1, 31, 32, 33, 63, 64, 65, 95, 96, 97, 128, 129, 160, 161, 192, 193,
              224, 225, 255, 256, 257, 300, 511, 513, 0]
    E, T = len(counts), sum(counts)
    say(f"layer bf16 E={E} H=256 F=128 T={T} k=1, fixed rows per expert")
    L = Layer(E, 256, 128, seed=27)
    perm = torch.randperm(T, generator=torch.Generator().manual_seed(27))
    assign = torch.repeat_interleave(torch.arange(E), torch.tensor(counts))[perm]
    out, ref, mag = _layer_case(L, T, 1, "bf16", seed=27,
                                mutate=lambda ids, w: (assign.view(T, 1).to(ids.dtype), w))
    for e in range(E - 1):
        rows = (assign == e).nonzero().flatten().numpy()
        check(out[rows], ref[rows], mag[rows], "bf16", f"expert {e} ({counts[e]} rows)")
    check(out, ref, mag, "bf16", "layer")


@pytest.mark.parametrize("E", [16, 1024])
def test_layer_f32_fixed_rows_per_expert(E):
    # Decode plan: an expert with c pairs gets ceil(c / tb) weight-pass
    # records; counts below make passes of one and two tokens end on and
    # beside every split.  16 experts: two tokens per gate+up pass; 1024
    # experts (fewer pairs than half the experts): one.
    counts = [1, 2, 3, 4, 5, 7, 8, 9, 16, 17, 33, 0]
    T = sum(counts)
    say(f"layer f32 E={E} H=256 F=128 T={T} k=1, fixed rows per expert")
    L = Layer(E, 256, 128, seed=28)
    perm = torch.randperm(T, generator=torch.Generator().manual_seed(28))
    assign = torch.repeat_interleave(torch.arange(len(counts)), torch.tensor(counts))[perm]
    assign = (assign * (E // 16)).to(torch.int32)   # spread over the experts
    out, ref, mag = _layer_case(L, T, 1, "f32", seed=28,
                                mutate=lambda ids, w: (assign.view(T, 1).to(ids.dtype), w))
    for e in range(len(counts) - 1):
        rows = (assign == e * (E // 16)).nonzero().flatten().numpy()
        check(out[rows], ref[rows], mag[rows], "f32", f"expert {e} ({counts[e]} rows)")
    check(out, ref, mag, "f32", "layer")


def test_layer_f32_more_pairs_than_a_grid_dimension():
    # 8200 tokens x top-8 = 65600 pairs: more decode plan records than one
    # grid dimension holds (65535), so the record index spans grid y and z.
    say("layer f32 E=16 H=256 F=128 T=8200 k=8 (sampled tokens)")
    L = Layer(16, 256, 128, seed=29)
    toks = [0, 1, 4099, 8198, 8199]
    out, ref, mag = _layer_case(L, 8200, 8, "f32", seed=29, tokens=toks, cover=True)
    check(out, ref, mag, "f32", "layer")


def test_layer_bf16_more_tokens_than_a_grid_dimension():
    # 65600 tokens: the combine's token index spans grid y and z.
    say("layer bf16 E=8 H=256 F=128 T=65600 k=2 (sampled tokens)")
    L = Layer(8, 256, 128, seed=30)
    toks = [0, 1, 65534, 65535, 65536, 65599]
    out, ref, mag = _layer_case(L, 65600, 2, "bf16", seed=30, tokens=toks)
    check(out, ref, mag, "bf16", "layer")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_layer_every_pair_on_one_expert(dtype):
    # 40 tokens x 4 slots all routed to expert 3 (duplicates within a token
    # included): one expert with 160 pairs, the others idle.
    say(f"layer E=8 H=256 F=128 T=40 k=4 {dtype}, every pair on expert 3")
    L = Layer(8, 256, 128, seed=31)
    out, ref, mag = _layer_case(L, 40, 4, dtype, seed=31,
                                mutate=lambda ids, w: (torch.full_like(ids, 3), w))
    check(out, ref, mag, dtype, "layer")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_layer_invalid_and_duplicate_ids(dtype):
    say(f"layer invalid/duplicate ids {dtype}")
    L = Layer(8, 256, 128, seed=22)

    def mutate(ids, w):
        ids = ids.clone()
        ids[0, 0] = -1
        ids[1, :] = 8          # every slot of token 1 invalid -> zero output
        ids[2, 1] = ids[2, 0]  # a duplicate expert in one token
        return ids, w
    out, ref, mag = _layer_case(L, 9, 3, dtype, seed=5, mutate=mutate)
    assert np.all(out[1] == 0.0)
    check(out, ref, mag, dtype, "layer")


@pytest.mark.parametrize("T", [1, 4, 16])
def test_layer_decode_e128(T):
    say(f"decode layer E=128 H=4096 F=1536 T={T} (every token)")
    L = _big_layer(128, 4096, 1536, 2)
    out, ref, mag = _layer_case(L, T, 8, "f32", seed=T)
    check(out, ref, mag, "f32", "layer")


def test_layer_prefill_e128_t8192():
    say("prefill layer E=128 H=4096 F=1536 T=8192")
    L = _big_layer(128, 4096, 1536, 3)
    out, ref, mag = _layer_case(L, 8192, 8, "bf16", logits="uniform", seed=3,
                                tokens=[0, 8191], cover=True)
    check(out, ref, mag, "bf16", "layer")


_BIG = {}


def _big_layer(E, H, F, seed):
    key = (E, H, F, seed)
    if key not in _BIG:
        _BIG.clear()
        torch.cuda.empty_cache()
        _BIG[key] = Layer(E, H, F, seed=seed, gen_device=DEV)
    return _BIG[key]


def test_layer_worklist_left_in_workspace():
    say("layer workspace worklist")
    L = Layer(16, 256, 128, seed=23)
    g = synth.generator(9)
    wl = synth.Workload("t", 16, 256, 128, 4, 50, "f32", "normal", 9)
    x, ids, w = synth.layer_inputs(wl, g)
    for dtype, xx in ((qm.QMOE_F32, x), (qm.QMOE_F32_DIGITS, x),
                      (qm.QMOE_BF16, x.to(torch.bfloat16))):
        ws = torch.empty(L.dev.workspace_bytes(50, 4, dtype), dtype=torch.uint8, device=DEV)
        ws.fill_(0xAB)
        qm.qmoe_layer(L.dev, xx.to(DEV), ids.to(DEV), w.to(DEV), ws=ws, x_dtype=dtype)
        got = qm.layer_worklist_from_ws(L.dev, ws, 50, 4, dtype)
        ref = orc().worklist(ids.numpy(), 16)
        for key in ("counts", "offsets", "pairs", "inv"):
            assert np.array_equal(got[key].cpu().numpy(), ref[key]), key


# ------------------------------------------- large skewed layer (Zipf) ---

@pytest.mark.parametrize("dtype,T", [("f32", 64), ("bf16", 2048)])
def test_layer_e256_zipf(dtype, T):
    say(f"zipf layer E=256 H=6144 F=2048 T={T} {dtype}")
    L = _big_layer(256, 6144, 2048, 4)
    if dtype == "f32":        # every token
        out, ref, mag = _layer_case(L, T, 8, dtype, logits="zipf", seed=40 + T)
    else:
        out, ref, mag = _layer_case(L, T, 8, dtype, logits="zipf", seed=40 + T,
                                    tokens=[0, T - 1], cover=True)
    check(out, ref, mag, dtype, "layer")


# ------------------------------------------------------------ edge cases ---

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_layer_single_expert_k1_equals_expert_ffn(dtype):
    """E = 1, k = 1, weight 1: the layer is the expert FFN (GPU vs GPU, both
    also within tolerance of the oracle)."""
    say(f"layer E=1 k=1 {dtype}")
    L = Layer(1, 256, 128, seed=31)
    g = synth.generator(77)
    x = synth.rand_x(g, (70, 256))
    if dtype == "bf16":
        x = x.to(torch.bfloat16)
    ids = torch.zeros(70, 1, dtype=torch.int32)
    w = torch.ones(70, 1)
    lay = qm.qmoe_layer(L.dev, x.to(DEV), ids.to(DEV), w.to(DEV)).cpu().numpy()
    ffn = qm.qmoe_expert_ffn(L.packed["qg"][0], L.s_dev["sg"][0], L.packed["qu"][0],
                             L.s_dev["su"][0], L.packed["qd"][0], L.s_dev["sd"][0], 256, 128,
                             x.to(DEV)).cpu().numpy()
    ref, mag = L.oracle_layer(x, ids, w, mag=True)
    check(lay, ref, mag, dtype, "layer")
    check(ffn, ref, mag, dtype, "expert ffn")
    tol = F32_TOL if dtype == "f32" else BF16_TOL
    assert rel_l2(lay, ffn) <= tol


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_layer_all_ids_invalid_gives_zero(dtype):
    say(f"layer all ids invalid {dtype}")
    L = Layer(4, 256, 128, seed=32)
    x = synth.rand_x(synth.generator(5), (6, 256))
    if dtype == "bf16":
        x = x.to(torch.bfloat16)
    ids = torch.tensor([[-1, 4]] * 6, dtype=torch.int32)
    w = torch.ones(6, 2)
    out = qm.qmoe_layer(L.dev, x.to(DEV), ids.to(DEV), w.to(DEV))
    assert torch.count_nonzero(out).item() == 0


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_layer_max_experts(dtype):
    """E = 1024 (the largest expert count): most experts get one pair or none."""
    say(f"layer E=1024 H=256 F=128 T=60 k=8 {dtype}")
    L = Layer(1024, 256, 128, seed=35)
    out, ref, mag = _layer_case(L, 60, 8, dtype, seed=36)
    check(out, ref, mag, dtype, "layer")


@pytest.mark.parametrize("dtype,T", [("bf16", 1), ("bf16", 2), ("bf16", 3), ("f32", 2)])
def test_layer_tiny_batches(dtype, T):
    """A handful of tokens, including the MFMA path with single-row tiles."""
    say(f"layer E=16 H=512 F=256 T={T} k=4 {dtype}")
    L = Layer(16, 512, 256, seed=37)
    out, ref, mag = _layer_case(L, T, 4, dtype, seed=38 + T)
    check(out, ref, mag, dtype, "layer")


@pytest.mark.parametrize("H,F", [(512, 1024), (1536, 512), (320, 192), (192, 320)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_layer_other_aspect_ratios(H, F, dtype):
    """Intermediate wider than hidden and the reverse, beside the 4096/1536
    and 6144/2048 shapes; 320 and 192 leave the last 128-feature (gate+up)
    and 256-feature (down) column blocks of the prefill kernels partly
    empty and give the decode kernels rows of 3 or 5 groups."""
    say(f"layer E=8 H={H} F={F} T=33 k=2 {dtype}")
    L = Layer(8, H, F, seed=39)
    out, ref, mag = _layer_case(L, 33, 2, dtype, seed=40)
    check(out, ref, mag, dtype, "layer")


def test_layer_bf16_outputs_beyond_f16_range():
    """Per-pair down outputs beyond 65504 (down scales x30000, so |q s| stays
    below 4800 while outputs reach ~1e5): the f16 intermediate of the routed
    down projection carries a power-of-two exponent per 4 x 16 block, so
    nothing overflows."""
    say("layer bf16 with outputs beyond the f16 range")
    L = Layer(8, 512, 256, seed=41)
    L.s["sd"] = L.s["sd"] * 30000.0
    L.s_dev["sd"].mul_(30000.0)
    out, ref, mag = _layer_case(L, 50, 2, "bf16", seed=42)
    assert np.abs(ref).max() > 1e5
    assert np.isfinite(out).all()
    check(out, ref, mag, "bf16", f"layer, max |ref| = {np.abs(ref).max():.3e}")


def test_layer_bf16_tiny_routing_weights():
    """Routing weights of ~1e-36 put whole 4 x 16 blocks of the routed down
    outputs below 2^-111: the block exponent is clamped so that its scale
    factors stay finite normal f32 numbers, and the outputs keep their
    relative accuracy."""
    say("layer bf16 with routing weights x1e-36")
    L = Layer(8, 512, 256, seed=43)
    out, ref, mag = _layer_case(L, 50, 2, "bf16", seed=44, mutate=lambda ids, w: (ids, w * 1e-36))
    assert np.abs(ref).max() < 2.0 ** -100
    assert np.isfinite(out).all()
    check(out, ref, mag, "bf16", f"layer, max |ref| = {np.abs(ref).max():.3e}")


def test_layer_wide_topk():
    """k = 16 of 32 experts, f32 and bf16."""
    L = Layer(32, 256, 128, seed=33)
    for dtype in ("f32", "bf16"):
        say(f"layer k=16 {dtype}")
        out, ref, mag = _layer_case(L, 20, 16, dtype, seed=16)
        check(out, ref, mag, dtype, "layer")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_layer_graph_replays_match_eager(dtype):
    """Capture qmoe_layer in a HIP graph and replay it several times with
    eager work and synchronisation in between; every replay must match the
    eager result (the library records no memset nodes)."""
    say(f"layer graph replay {dtype}")
    L = Layer(16, 256, 128, seed=34)
    g = synth.generator(3)
    wl = synth.Workload("t", 16, 256, 128, 4, 33, dtype, "normal", 3)
    x, ids, w = synth.layer_inputs(wl, g)
    xd, idd, wd = x.to(DEV), ids.to(DEV), w.to(DEV)
    code = qm.QMOE_F32 if dtype == "f32" else qm.QMOE_BF16
    ws = torch.empty(L.dev.workspace_bytes(33, 4, code), dtype=torch.uint8, device=DEV)
    out = torch.empty(33, 256, device=DEV)
    qm.qmoe_layer(L.dev, xd, idd, wd, out=out, ws=ws)
    torch.cuda.synchronize()
    eager = out.clone()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.graph(graph, stream=s):
        qm.qmoe_layer(L.dev, xd, idd, wd, out=out, ws=ws)
    for rep in range(4):
        out.fill_(float("nan"))
        ws.fill_(0xAB)                 # stale workspace must not matter
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(out).all()
        assert rel_l2(out.cpu().numpy(), eager.cpu().numpy()) <= 1e-6, rep


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_layer_side_stream_internal_workspace(dtype):
    """A call on a side stream with no workspace argument: the binding's
    internal workspace must not be handed out again on the current stream
    while the side stream's kernels still use it.  The side stream is kept
    busy first, so the layer's kernels run well after the call returns; the
    current stream then allocates the same size and overwrites it."""
    say(f"side-stream layer with internal workspace {dtype}")
    L = Layer(16, 256, 128, seed=35)
    g = synth.generator(36)
    wl = synth.Workload("t", 16, 256, 128, 4, 33, dtype, "normal", 36)
    x, ids, w = synth.layer_inputs(wl, g)
    xd, idd, wd = x.to(DEV), ids.to(DEV), w.to(DEV)
    code = qm.QMOE_F32 if dtype == "f32" else qm.QMOE_BF16
    ref = qm.qmoe_layer(L.dev, xd, idd, wd)
    torch.cuda.synchronize()
    nb = L.dev.workspace_bytes(33, 4, code)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    out = torch.empty_like(ref)
    a = torch.full((2048, 2048), 1.0 / 2048, device=DEV)
    with torch.cuda.stream(side):
        b = a
        for _ in range(24):
            b = torch.mm(b, a)             # keeps the side stream busy
    qm.qmoe_layer(L.dev, xd, idd, wd, out=out, stream=side)
    junk = torch.empty(max(nb, 16), dtype=torch.uint8, device=DEV)
    junk.fill_(0xAB)
    torch.cuda.synchronize()
    del b
    assert torch.isfinite(out).all()
    assert rel_l2(out.cpu().numpy(), ref.cpu().numpy()) <= 1e-6


@pytest.mark.parametrize("rows,cols,offset", [(5, 4096, 0), (7, 33, 0), (3, 1000, 3), (1, 1, 0)])
def test_import_twos(rows, cols, offset):
    say(f"import two's complement rows={rows} cols={cols} offset={offset}")
    g = synth.generator(70)
    rb = (cols + 1) // 2
    raw = torch.randint(0, 256, (rows * rb + offset,), generator=g, dtype=torch.int64).to(torch.uint8)
    twos = raw[offset:].reshape(rows, rb)
    ref = orc().import_twos(twos.numpy(), cols)
    d = raw.to(DEV)[offset:].view(rows, rb)
    got = qm.qmoe_import_twos(d, cols).cpu().numpy()
    assert np.array_equal(got, ref)
    qm.qmoe_import_twos(d, cols, out=d)                  # in place
    assert np.array_equal(d.cpu().numpy(), ref)
