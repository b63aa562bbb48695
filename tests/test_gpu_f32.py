"""The f32 decode path (QMOE_F32: every code unpacked to f32, f32 FMA chains,
f32 group scale) and its digit variant (QMOE_F32_DIGITS), against the oracle:
activations whose 64-element groups span a large dynamic range, NaN and
infinity in x, the pass grouping of the two-launch call (at most 64 pairs)
and of the planned call past it, and the digit variant selected explicitly."""
import numpy as np
import pytest
import torch

import grouped_int4_expert_amd as qm
import synth
from gpu_util import F32_TOL, Layer, check, orc, rel_l2, say

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qm.load()
    yield
    torch.cuda.synchronize()


def _outlier_x(g, rows, cols, ratio=1e4):
    """Every 64-element group holds one element `ratio` times the scale of
    the others (which are N(0,1) * 1e-3), at a random place and sign."""
    x = synth.rand_x(g, (rows, cols)) * 1e-3
    ng = cols // 64
    pos = torch.randint(0, 64, (rows, ng), generator=g)
    sign = torch.randint(0, 2, (rows, ng), generator=g).float() * 2 - 1
    idx = torch.arange(ng) * 64 + pos
    x.scatter_(1, idx, sign * 1e-3 * ratio)
    return x


def test_matvec_outlier_groups():
    say("matvec 512x4096, one element per group 1e4x the rest")
    g = synth.generator(501)
    q = synth.rand_q(g, (512, 4096))
    s = synth.rand_scales(g, (512, 64))
    x = _outlier_x(g, 3, 4096)
    y = qm.qmoe_matvec(qm.qmoe_pack(q.to(DEV)), s.to(DEV), 4096, x.to(DEV)).cpu().numpy()
    pq, _ = orc().pack(q.numpy())
    ref = orc().matvec(pq, s.numpy(), 4096, x.numpy())
    mag = orc().matvec_abs(pq, s.numpy(), 4096, x.numpy())
    err, worst = check(y, ref, mag, "f32", "matvec outliers")
    assert err <= 1e-6


def test_layer_outlier_groups_f32_and_digits():
    """The f32 path keeps f32 accuracy on groups with a 1e4 dynamic range;
    the digit variant rounds each group to 18 bits of its largest element,
    so its small elements keep few bits and its error is far larger."""
    say("layer E=16 H=1024 F=512 T=12 k=4, outlier groups")
    L = Layer(16, 1024, 512, seed=502)
    g = synth.generator(503)
    x = _outlier_x(g, 12, 1024)
    ids, w = synth.route_topk_fast(synth.normal_logits(g, 12, 16), 4)
    xd, idd, wd = x.to(DEV), ids.to(DEV), w.to(DEV)
    ref, mag = L.oracle_layer(x, ids, w, mag=True)
    out = qm.qmoe_layer(L.dev, xd, idd, wd).cpu().numpy()
    err_f32, _ = check(out, ref, mag, "f32", "f32 path")
    dig = qm.qmoe_layer(L.dev, xd, idd, wd, x_dtype=qm.QMOE_F32_DIGITS).cpu().numpy()
    err_dig = rel_l2(dig, ref)
    say(f"  digit variant rel_l2 = {err_dig:.3e} (f32 path {err_f32:.3e})")
    assert err_f32 <= 1e-6
    assert err_dig > 10 * err_f32


def test_matvec_nan_and_inf():
    say("matvec NaN / inf in x")
    g = synth.generator(504)
    q = synth.rand_q(g, (96, 256))
    s = synth.rand_scales(g, (96, 4))
    x = synth.rand_x(g, (4, 256))
    x[1, 5] = float("nan")
    x[2, 200] = float("inf")
    x[3, 17] = -float("inf")
    y = qm.qmoe_matvec(qm.qmoe_pack(q.to(DEV)), s.to(DEV), 256, x.to(DEV)).cpu().numpy()
    pq, _ = orc().pack(q.numpy())
    ref = orc().matvec(pq, s.numpy(), 256, x.numpy())
    assert np.isnan(ref[1]).all() and not np.isfinite(ref[2]).any()
    check(y, ref, None, "f32", "matvec nan/inf")


@pytest.mark.parametrize("code", [qm.QMOE_F32, qm.QMOE_F32_DIGITS, qm.QMOE_BF16])
def test_layer_nan_reaches_its_token_only(code):
    say(f"layer NaN in one token, path {code}")
    L = Layer(8, 256, 128, seed=505)
    g = synth.generator(506)
    x = synth.rand_x(g, (9, 256))
    x[4, 77] = float("nan")
    ids, w = synth.route_topk_fast(synth.normal_logits(g, 9, 8), 2)
    xx = x.to(torch.bfloat16) if code == qm.QMOE_BF16 else x
    out = qm.qmoe_layer(L.dev, xx.to(DEV), ids.to(DEV), w.to(DEV), x_dtype=code).cpu().numpy()
    ref = L.oracle_layer(xx, ids, w)
    assert np.isnan(ref[4]).all()
    assert np.isnan(out[4]).all()
    keep = [t for t in range(9) if t != 4]
    assert np.isfinite(out[keep]).all()
    path = "bf16" if code == qm.QMOE_BF16 else "f32"
    check(out[keep], ref[keep], None, path, "other tokens")


@pytest.mark.parametrize("T", [8, 9, 128, 129])
def test_layer_inline_limit(T):
    """T x 8 = 64 pairs: two launches, the pass grouping derived inside the
    gate+up blocks; 72 pairs and more: the preparation kernel's plan records.
    16 experts, so most experts have several pairs (four tokens per pass)."""
    say(f"layer f32 E=16 H=256 F=128 T={T} k=8")
    L = Layer(16, 256, 128, seed=507)
    g = synth.generator(508 + T)
    x = synth.rand_x(g, (T, 256))
    ids, w = synth.route_topk_fast(synth.normal_logits(g, T, 16), 8)
    ids[3, 0] = -1
    ids[7, 2] = ids[7, 1]
    out = qm.qmoe_layer(L.dev, x.to(DEV), ids.to(DEV), w.to(DEV)).cpu().numpy()
    ref, mag = L.oracle_layer(x, ids, w, mag=True)
    check(out, ref, mag, "f32", "layer")


@pytest.mark.parametrize("counts_e", [16, 64, 128, 1024])
def test_layer_pass_grouping(counts_e):
    """Experts with 1..17 pairs (duplicates in one token included; 206 pairs,
    past the inline limit) at expert counts that select four tokens per pass
    in both launches, four in gate+up and two in down, two in both, and one."""
    counts = [1, 2, 3, 4, 5, 6, 7, 8, 9, 12, 13, 16, 17]
    T = sum(counts)
    E = counts_e
    say(f"layer f32 E={E} H=192 F=320 T={T} k=2, fixed pairs per expert")
    L = Layer(E, 192, 320, seed=509)
    perm = torch.randperm(2 * T, generator=torch.Generator().manual_seed(509))
    assign = torch.repeat_interleave(torch.arange(len(counts)), torch.tensor(counts) * 2)[perm]
    ids = (assign * (E // 16)).to(torch.int32).view(T, 2)
    g = synth.generator(510)
    x = synth.rand_x(g, (T, 192))
    w = torch.rand((T, 2), generator=g)
    out = qm.qmoe_layer(L.dev, x.to(DEV), ids.to(DEV), w.to(DEV)).cpu().numpy()
    ref, mag = L.oracle_layer(x, ids, w, mag=True)
    check(out, ref, mag, "f32", "layer")


@pytest.mark.parametrize("counts_e", [8, 48, 1024])
def test_layer_pass_grouping_inline(counts_e):
    """At most 64 pairs (the gate+up launch groups them itself): experts with
    1..7 pairs at expert counts that select four, two and one tokens per
    weight pass."""
    counts = [1, 2, 3, 4, 5, 6, 7]
    T = sum(counts)
    E = counts_e
    say(f"layer f32 E={E} H=192 F=320 T={T} k=2 (inline), fixed pairs per expert")
    L = Layer(E, 192, 320, seed=513)
    perm = torch.randperm(2 * T, generator=torch.Generator().manual_seed(513))
    assign = torch.repeat_interleave(torch.arange(len(counts)), torch.tensor(counts) * 2)[perm]
    ids = (assign * (E // 8)).to(torch.int32).view(T, 2)
    g = synth.generator(514)
    x = synth.rand_x(g, (T, 192))
    w = torch.rand((T, 2), generator=g)
    out = qm.qmoe_layer(L.dev, x.to(DEV), ids.to(DEV), w.to(DEV)).cpu().numpy()
    ref, mag = L.oracle_layer(x, ids, w, mag=True)
    check(out, ref, mag, "f32", "layer")


@pytest.mark.parametrize("E,H,F,T", [(16, 256, 128, 37), (128, 4096, 1536, 16)])
def test_digit_variant_layer(E, H, F, T):
    say(f"digit variant layer E={E} H={H} F={F} T={T}")
    L = Layer(E, H, F, seed=511, gen_device=DEV if E > 16 else "cpu")
    g = synth.generator(512)
    x = synth.rand_x(g, (T, H))
    ids, w = synth.route_topk_fast(synth.normal_logits(g, T, E), 8 if E > 16 else 4)
    out = qm.qmoe_layer(L.dev, x.to(DEV), ids.to(DEV), w.to(DEV),
                        x_dtype=qm.QMOE_F32_DIGITS).cpu().numpy()
    ref = L.oracle_layer(x, ids, w)
    err = rel_l2(out, ref)
    say(f"  rel_l2 = {err:.3e}")
    assert err <= F32_TOL


def test_digit_variant_expert_ffn():
    say("digit variant expert ffn H=4096 F=1536 batch 3")
    L = Layer(1, 4096, 1536, seed=513)
    x = synth.rand_x(synth.generator(514), (3, 4096))
    out = qm.qmoe_expert_ffn(L.packed["qg"][0], L.s_dev["sg"][0], L.packed["qu"][0],
                             L.s_dev["su"][0], L.packed["qd"][0], L.s_dev["sd"][0], 4096, 1536,
                             x.to(DEV), x_dtype=qm.QMOE_F32_DIGITS).cpu().numpy()
    ref = L.oracle_layer(x, torch.zeros(3, 1, dtype=torch.int32), torch.ones(3, 1))
    assert rel_l2(out, ref) <= F32_TOL


# ---------------------------------------------------------------------------
# Past 64 pairs, with input widths that are multiples of 512, the passes run
# on the matrix cores: x and h carried as three exact f16 parts each, codes as
# exact f16, products accumulated in f32, the f32 group scale per 64 inputs.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("H,F", [(1024, 512), (512, 1536), (1536, 1024), (1024, 320)])
def test_matrix_core_layer_outlier_groups(H, F):
    """Every 64-input group of x holds one element 1e4 times the others; the
    widths give one, two, three and four waves per block (H or F = 512,
    1024, 1536) and, at F = 320, a gate+up that writes f32 h for the VALU
    down projection."""
    E, T, k = 16, 24, 4
    say(f"matrix-core layer E={E} H={H} F={F} T={T} k={k}, outlier groups")
    L = Layer(E, H, F, seed=520)
    g = synth.generator(521)
    x = _outlier_x(g, T, H)
    ids, w = synth.route_topk_fast(synth.normal_logits(g, T, E), k)
    ref, mag = L.oracle_layer(x, ids, w, mag=True)
    out = qm.qmoe_layer(L.dev, x.to(DEV), ids.to(DEV), w.to(DEV)).cpu().numpy()
    err, _ = check(out, ref, mag, "f32", "layer")
    assert err <= 1e-6


@pytest.mark.parametrize("bad", [float("nan"), float("inf"), -float("inf")])
def test_matrix_core_layer_nonfinite_reaches_its_token_only(bad):
    """A NaN or infinity in one token's x: that token's outputs follow the
    oracle's NaN / infinity pattern (an infinity stays in the first f16 part
    of the split), every other token stays finite and within the bar."""
    say(f"matrix-core layer E=8 H=512 F=512 T=20 k=4, {bad} in one token")
    L = Layer(8, 512, 512, seed=522)
    g = synth.generator(523)
    x = synth.rand_x(g, (20, 512))
    x[7, 300] = bad
    ids, w = synth.route_topk_fast(synth.normal_logits(g, 20, 8), 4)
    out = qm.qmoe_layer(L.dev, x.to(DEV), ids.to(DEV), w.to(DEV)).cpu().numpy()
    ref = L.oracle_layer(x, ids, w)
    assert not np.isfinite(ref[7]).any() and not np.isfinite(out[7]).any()
    keep = [t for t in range(20) if t != 7]
    assert np.isfinite(out[keep]).all()
    check(out, ref, None, "f32", "all tokens")


@pytest.mark.parametrize("counts_e", [16, 64, 1024])
def test_matrix_core_layer_pass_grouping(counts_e):
    """Experts with 1..17 pairs (passes of four tokens, the last one short;
    duplicate experts in one token)."""
    counts = [1, 2, 3, 4, 5, 6, 7, 8, 9, 12, 13, 16, 17]
    T = sum(counts)
    E = counts_e
    say(f"matrix-core layer E={E} H=512 F=512 T={T} k=2, fixed pairs per expert")
    L = Layer(E, 512, 512, seed=524)
    perm = torch.randperm(2 * T, generator=torch.Generator().manual_seed(524))
    assign = torch.repeat_interleave(torch.arange(len(counts)), torch.tensor(counts) * 2)[perm]
    ids = (assign * (E // 16)).to(torch.int32).view(T, 2)
    g = synth.generator(525)
    x = synth.rand_x(g, (T, 512))
    w = torch.rand((T, 2), generator=g)
    out = qm.qmoe_layer(L.dev, x.to(DEV), ids.to(DEV), w.to(DEV)).cpu().numpy()
    ref, mag = L.oracle_layer(x, ids, w, mag=True)
    check(out, ref, mag, "f32", "layer")


@pytest.mark.parametrize("group", [128, 1024])
def test_matrix_core_layer_wider_groups(group):
    """Groups of 128 and one scale per row (1024 = the width of gate and up):
    the general scale path of the matrix-core kernels."""
    say(f"matrix-core layer E=16 H=1024 F=1024 T=24 k=4 group {group}")
    L = Layer(16, 1024, 1024, seed=526, group=group)
    g = synth.generator(527)
    x = synth.rand_x(g, (24, 1024))
    ids, w = synth.route_topk_fast(synth.normal_logits(g, 24, 16), 4)
    out = qm.qmoe_layer(L.dev, x.to(DEV), ids.to(DEV), w.to(DEV)).cpu().numpy()
    ref, mag = L.oracle_layer(x, ids, w, mag=True)
    check(out, ref, mag, "f32", "layer")


def test_matrix_core_layer_many_tokens_per_expert():
    """129 tokens x top-8 over 16 experts: about 65 pairs per expert, 17
    passes each, one short."""
    say("matrix-core layer E=16 H=512 F=512 T=129 k=8")
    L = Layer(16, 512, 512, seed=528)
    g = synth.generator(529)
    x = synth.rand_x(g, (129, 512))
    ids, w = synth.route_topk_fast(synth.normal_logits(g, 129, 16), 8)
    out = qm.qmoe_layer(L.dev, x.to(DEV), ids.to(DEV), w.to(DEV)).cpu().numpy()
    ref, mag = L.oracle_layer(x, ids, w, mag=True)
    check(out, ref, mag, "f32", "layer")
