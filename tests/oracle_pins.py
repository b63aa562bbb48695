"""Pins for the CPU oracle: checks against values and laws fixed by the pages
and by mathematics, never against the oracle's own formula retyped.

Each pin is a function taking an ``oracle.Oracle`` and raising
AssertionError on a mismatch, so that ``test_oracle_mutants.py`` can run the
same pins against deliberately broken builds of the oracle and show that
every planted mistake is caught by at least one of them.

Sources: the colibri pull request "cuda+engine: full fmt=4 (grouped int4
gs=64) support + diagnostic harness" (Summary; comments "implementation
complete but system-instability", "blocked by GPU driver instability",
"Here's the oracle you're missing", "fmt=4 CUDA attention crash - root cause,
fix"), and the pxq_llama.cpp release notes, section "Device-side MoE row map".
The router pins follow the same pull request's quoted issue (list of CPU
work: router top-K with a taken flag per expert).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rng(seed):
    return np.random.default_rng(seed)


def _rand_layer(orc, rng, E, H, F, gs=64):
    qg = rng.integers(-8, 8, size=(E, F, H), dtype=np.int8)
    qu = rng.integers(-8, 8, size=(E, F, H), dtype=np.int8)
    qd = rng.integers(-8, 8, size=(E, H, F), dtype=np.int8)
    sg = rng.uniform(0.005, 0.02, size=(E, F, -(-H // gs))).astype(np.float32)
    su = rng.uniform(0.005, 0.02, size=(E, F, -(-H // gs))).astype(np.float32)
    sd = rng.uniform(0.005, 0.02, size=(E, H, -(-F // gs))).astype(np.float32)
    pg, _ = orc.pack(qg)
    pu, _ = orc.pack(qu)
    pd, _ = orc.pack(qd)
    return dict(qg=qg, qu=qu, qd=qd, sg=sg, su=su, sd=sd, pg=pg, pu=pu, pd=pd)


def _close(a, b, rtol, atol=0.0, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    err = np.abs(a - b)
    lim = atol + rtol * np.abs(b)
    assert np.all(err <= lim), (what, float(err.max()))


# ---------------------------------------------------------------- format ---

def pin_sizes_kv_b_header(orc):
    """kv_b header: 28,672 rows x 256 B, 229,376 f32 scales = 8 per row."""
    g = _golden("format_sizes.json")["kv_b_header"]
    cols = 512  # I that gives 256 B per row and 8 groups of 64
    assert orc.row_bytes(cols) == g["row_bytes"]
    assert orc.groups(cols, g["group_size"]) == g["groups_per_row"]
    assert orc.packed_bytes(g["rows"], cols) == g["weight_bytes"]
    assert orc.scale_count(g["rows"], cols, 64) == g["scale_floats"]
    assert 4 * orc.scale_count(g["rows"], cols, 64) == g["scale_bytes"]


def pin_sizes_odd_and_partial(orc):
    """(I+1)/2 bytes per row and ceil(I/gs) groups, odd I and gs > I."""
    assert orc.row_bytes(5) == 3 and orc.row_bytes(1) == 1
    assert orc.groups(5, 2) == 3 and orc.groups(3, 4) == 1
    assert orc.groups(64, 64) == 1 and orc.groups(65, 64) == 2


def pin_sizes_footprint_ratio(orc):
    """g64 scales cost 1/8 of the packed bytes: 0.9 GB over 7.4 GB."""
    g = _golden("format_sizes.json")["dense_footprint"]
    rows, cols = 1024, 4096
    ratio = 4 * orc.scale_count(rows, cols, 64) / orc.packed_bytes(rows, cols)
    d = g["printed_precision_gb"]
    lo = (g["scales_gb"] - d) / (g["packed_gb"] + d)
    hi = (g["scales_gb"] + d) / (g["packed_gb"] - d)
    assert lo <= ratio <= hi, ratio


def pin_sizes_expert(orc):
    """~19 MB -> ~21-22 MB per expert, +2.2 MB, at hidden 6144 / inter 2048."""
    g = _golden("format_sizes.json")["expert_size"]
    H, F, tol = g["hidden"], g["inter"], g["tolerance_mb"]
    packed = 2 * orc.packed_bytes(F, H) + orc.packed_bytes(H, F)
    scales = 4 * (2 * orc.scale_count(F, H, 64) + orc.scale_count(H, F, 64))
    mb = 1e6
    assert abs(packed / mb - g["packed_mb_approx"]) <= tol
    lo, hi = g["grouped_mb_approx"]
    assert lo - tol <= (packed + scales) / mb <= hi + tol
    assert abs(scales / mb - g["delta_mb_approx"]) <= tol


def pin_pack_hand(orc):
    """Hand-packed bytes of the tiny matrices."""
    for case in _golden("hand_cases.json")["matvec"]:
        q = np.array(case["q"], dtype=np.int8)
        packed, bad = orc.pack(q)
        assert bad == 0
        assert packed.tolist() == case["packed"], case["name"]
        assert orc.unpack(packed, q.shape[1]).tolist() == case["q"]


def pin_pack_exhaustive(orc):
    """All 256 code pairs round-trip; all 256 bytes round-trip."""
    a, b = np.meshgrid(np.arange(-8, 8), np.arange(-8, 8), indexing="ij")
    q = np.stack([a.ravel(), b.ravel()], axis=1).astype(np.int8)   # 256 x 2
    packed, bad = orc.pack(q)
    assert bad == 0
    assert sorted(packed.ravel().tolist()) == list(range(256))
    assert np.array_equal(orc.unpack(packed, 2), q)
    allbytes = np.arange(256, dtype=np.uint8).reshape(256, 1)
    q2 = orc.unpack(allbytes, 2)
    re, _ = orc.pack(q2)
    assert np.array_equal(re, allbytes)


def pin_pack_xor_0x88(orc):
    """Offset nibble u (0..15) XOR 8 is the two's-complement nibble of u-8:
    for every byte, sign-extending the nibbles of byte ^ 0x88 gives the codes
    the oracle decodes (even element = low nibble)."""
    x = _golden("format_sizes.json")["offset_to_twos_complement"]["xor_byte"]
    allbytes = np.arange(256, dtype=np.uint8).reshape(256, 1)
    codes = orc.unpack(allbytes, 2).astype(int)
    for byte in range(256):
        t = byte ^ x
        lo, hi = t & 15, t >> 4
        lo = lo - 16 if lo >= 8 else lo
        hi = hi - 16 if hi >= 8 else hi
        assert codes[byte, 0] == lo and codes[byte, 1] == hi, byte


def pin_pack_out_of_range_counted(orc):
    q = np.array([[8, -9, 0, 7]], dtype=np.int8)
    _, bad = orc.pack(q)
    assert bad == 2


# ---------------------------------------------------------------- matvec ---

def pin_matvec_hand(orc):
    for case in _golden("hand_cases.json")["matvec"]:
        q = np.array(case["q"], dtype=np.int8)
        packed, _ = orc.pack(q)
        s = np.array(case["scales"], dtype=np.float32)
        y = orc.matvec(packed, s, q.shape[1], np.array(case["x"]), case["gs"])
        _close(y, case["y"], 1e-15, 0, case["name"])


def pin_matvec_one_hot(orc):
    """x = e_j gives y[o] = s[o, j//gs] * q[o, j] exactly."""
    rng = _rng(11)
    O, I, gs = 7, 200, 64           # 200 = 3 full groups + a partial one
    q = rng.integers(-8, 8, size=(O, I), dtype=np.int8)
    s = rng.uniform(0.005, 0.02, size=(O, -(-I // gs))).astype(np.float32)
    packed, _ = orc.pack(q)
    for j in (0, 1, 63, 64, 127, 130, 191, 192, 199):
        x = np.zeros((1, I))
        x[0, j] = 1.0
        y = orc.matvec(packed, s, I, x, gs)[0]
        want = s[:, j // gs].astype(np.float64) * q[:, j]
        assert np.array_equal(y, want), j


def pin_matvec_equal_scales(orc):
    """All scales equal c: y = c * (Q x), Q the integer code matrix."""
    rng = _rng(12)
    O, I = 5, 256
    q = rng.integers(-8, 8, size=(O, I), dtype=np.int8)
    c = np.float32(0.0078125)
    s = np.full((O, I // 64), c, dtype=np.float32)
    x = rng.standard_normal((3, I))
    packed, _ = orc.pack(q)
    y = orc.matvec(packed, s, I, x)
    want = float(c) * (x @ q.astype(np.float64).T)
    _close(y, want, 1e-12, 1e-14)


def pin_matvec_ones(orc):
    """x = 1: y[o] = sum_g s[o,g] * (sum of the codes of group g)."""
    rng = _rng(13)
    O, I, gs = 4, 160, 64
    q = rng.integers(-8, 8, size=(O, I), dtype=np.int8)
    s = rng.uniform(0.005, 0.02, size=(O, 3)).astype(np.float32)
    packed, _ = orc.pack(q)
    y = orc.matvec(packed, s, I, np.ones((1, I)), gs)[0]
    gsum = np.stack([q[:, 0:64].sum(1), q[:, 64:128].sum(1),
                     q[:, 128:160].sum(1)], axis=1).astype(np.float64)
    _close(y, (gsum * s.astype(np.float64)).sum(1), 1e-13)


def pin_matvec_group_wider_than_row(orc):
    """gs >= I: one scale per row (the per-row int4 case, ng = 1)."""
    rng = _rng(14)
    O, I = 6, 48
    q = rng.integers(-8, 8, size=(O, I), dtype=np.int8)
    s = rng.uniform(0.005, 0.02, size=(O, 1)).astype(np.float32)
    x = rng.standard_normal((2, I))
    packed, _ = orc.pack(q)
    y = orc.matvec(packed, s, I, x, 64)
    want = (x @ q.astype(np.float64).T) * s[:, 0].astype(np.float64)[None, :]
    _close(y, want, 1e-12, 1e-14)


def pin_matvec_linear(orc):
    rng = _rng(15)
    O, I = 9, 192
    q = rng.integers(-8, 8, size=(O, I), dtype=np.int8)
    s = rng.uniform(0.005, 0.02, size=(O, 3)).astype(np.float32)
    packed, _ = orc.pack(q)
    x1, x2 = rng.standard_normal(I), rng.standard_normal(I)
    y = orc.matvec(packed, s, I, np.stack([x1, x2, 2.5 * x1 - 0.5 * x2,
                                           np.zeros(I)]))
    _close(y[2], 2.5 * y[0] - 0.5 * y[1], 1e-12, 1e-14)
    assert np.all(y[3] == 0.0)


def pin_matvec_dense_library(orc):
    """Random shapes against numpy: dequantise, then a library matmul."""
    rng = _rng(16)
    for O, I in ((33, 320), (17, 100), (64, 64)):
        q = rng.integers(-8, 8, size=(O, I), dtype=np.int8)
        ng = -(-I // 64)
        s = rng.uniform(0.005, 0.02, size=(O, ng)).astype(np.float32)
        x = rng.standard_normal((4, I))
        packed, _ = orc.pack(q)
        y = orc.matvec(packed, s, I, x)
        gidx = np.arange(I) // 64
        W = q.astype(np.float64) * s.astype(np.float64)[:, gidx]
        _close(y, x @ W.T, 1e-12, 1e-14)


def pin_pair_is_two_passes(orc):
    """Fused pair == two single passes, element by element (bit-exact)."""
    rng = _rng(17)
    O, I = 20, 192
    qg = rng.integers(-8, 8, size=(O, I), dtype=np.int8)
    qu = rng.integers(-8, 8, size=(O, I), dtype=np.int8)
    sg = rng.uniform(0.005, 0.02, size=(O, 3)).astype(np.float32)
    su = rng.uniform(0.005, 0.02, size=(O, 3)).astype(np.float32)
    x = rng.standard_normal((3, I))
    pg, _ = orc.pack(qg)
    pu, _ = orc.pack(qu)
    yg, yu = orc.pair(pg, sg, pu, su, I, x)
    assert np.array_equal(yg, orc.matvec(pg, sg, I, x))
    assert np.array_equal(yu, orc.matvec(pu, su, I, x))
    assert not np.array_equal(yg, yu)


# ------------------------------------------------------------------- ffn ---

def pin_silu_values(orc):
    """silu(0) = 0, silu(1) = logistic(1), silu(-1) = -logistic(-1),
    limits at +-large."""
    assert orc.silu(0.0) == 0.0
    assert abs(orc.silu(1.0) - 0.7310585786300049) <= 1e-16
    assert abs(orc.silu(-1.0) + 0.2689414213699951) <= 1e-16
    assert orc.silu(1000.0) == 1000.0
    v = orc.silu(-1000.0)
    assert v == 0.0 and math.copysign(1.0, v) < 0


def pin_ffn_hand(orc):
    c = _golden("hand_cases.json")["ffn"]
    pg, _ = orc.pack(np.array(c["gate_q"], np.int8))
    pu, _ = orc.pack(np.array(c["up_q"], np.int8))
    pd, _ = orc.pack(np.array(c["down_q"], np.int8))
    out = orc.ffn(pg, np.array(c["gate_s"], np.float32), pu,
                  np.array(c["up_s"], np.float32), pd,
                  np.array(c["down_s"], np.float32), 2, 2,
                  np.array(c["x"]), c["gs"])
    _close(out, c["out"], 4e-16, 1e-16)


def pin_ffn_dense_library(orc):
    """down(silu(gate x) * (up x)) with numpy dense dequantised matrices."""
    rng = _rng(18)
    H, F = 192, 128
    L = _rand_layer(orc, rng, 1, H, F)
    x = rng.standard_normal((2, H))
    out = orc.ffn(L["pg"][0], L["sg"][0], L["pu"][0], L["su"][0], L["pd"][0],
                  L["sd"][0], H, F, x)

    def deq(q, s):
        return q.astype(np.float64) * s.astype(np.float64)[:, np.arange(
            q.shape[1]) // 64]
    g = x @ deq(L["qg"][0], L["sg"][0]).T
    u = x @ deq(L["qu"][0], L["su"][0]).T
    h = g / (1.0 + np.exp(-g)) * u
    _close(out, h @ deq(L["qd"][0], L["sd"][0]).T, 1e-11, 1e-13)


# -------------------------------------------------------------- worklist ---

def pin_worklist_hand(orc):
    c = _golden("hand_cases.json")["worklist"]
    r = orc.worklist(np.array(c["ids"], np.int32), c["experts"])
    for key in ("counts", "offsets", "pairs", "inv"):
        assert r[key].tolist() == c[key], key
    assert r["n_invalid"] == c["n_invalid"]


def _brute_worklist(ids, E):
    flat = ids.ravel().tolist()
    pairs = []
    counts = []
    for e in range(E):
        mine = [p for p, v in enumerate(flat) if v == e]
        counts.append(len(mine))
        pairs += mine
    return counts, pairs


def pin_worklist_brute_force(orc):
    """64 seeded cases (with invalid ids) against a per-expert scan."""
    rng = _rng(19)
    for case in range(64):
        T = int(rng.integers(1, 40))
        K = int(rng.integers(1, 9))
        E = int(rng.integers(1, 70))
        ids = rng.integers(-2, E + 2, size=(T, K)).astype(np.int32)
        r = orc.worklist(ids, E)
        counts, pairs = _brute_worklist(ids, E)
        nvalid = len(pairs)
        assert r["counts"].tolist() == counts, case
        assert r["pairs"][:nvalid].tolist() == pairs, case
        assert np.all(r["pairs"][nvalid:] == -1)
        assert r["n_invalid"] == T * K - nvalid
        assert r["offsets"][0] == 0 and r["offsets"][-1] == nvalid
        assert np.all(np.diff(r["offsets"]) == np.array(counts))
        for pos, p in enumerate(pairs):
            assert r["inv"][p] == pos
        bad = [p for p, v in enumerate(ids.ravel()) if not (0 <= v < E)]
        assert all(r["inv"][p] == -1 for p in bad)


# ----------------------------------------------------------------- layer ---

def pin_layer_hand(orc):
    """Two experts; expert 1 = expert 0 with its down scales doubled, so
    ffn_1 = 2 ffn_0; weights (0.25 on e1, 0.75 on e0) give 1.25 ffn_0."""
    c = _golden("hand_cases.json")["ffn"]
    gq = np.array([c["gate_q"]] * 2, np.int8)
    uq = np.array([c["up_q"]] * 2, np.int8)
    dq = np.array([c["down_q"]] * 2, np.int8)
    gs_ = np.array([c["gate_s"]] * 2, np.float32)
    us_ = np.array([c["up_s"]] * 2, np.float32)
    ds_ = np.array([c["down_s"], [[2.0], [1.0]]], np.float32)
    pg, _ = orc.pack(gq)
    pu, _ = orc.pack(uq)
    pd, _ = orc.pack(dq)
    x = np.array([c["x"][0]])
    ids = np.array([[1, 0]], np.int32)
    w = np.array([[0.25, 0.75]], np.float32)
    out, bad = orc.layer(pg, gs_, pu, us_, pd, ds_, 2, 2, x, ids, w, 2)
    assert bad == 0
    _close(out[0], 1.25 * np.array(c["out"][0]), 4e-16, 1e-16)


def pin_layer_weighted_sum(orc):
    """out[t] = sum_k w[t,k] * ffn_{e[t,k]}(x_t), slots in order."""
    rng = _rng(20)
    E, H, F, T, K = 5, 128, 64, 4, 3
    L = _rand_layer(orc, rng, E, H, F)
    x = rng.standard_normal((T, H))
    ids = rng.integers(0, E, size=(T, K)).astype(np.int32)
    w = rng.uniform(0, 1, size=(T, K)).astype(np.float32)
    out, bad = orc.layer(L["pg"], L["sg"], L["pu"], L["su"], L["pd"], L["sd"],
                         H, F, x, ids, w)
    assert bad == 0
    for t in range(T):
        acc = np.zeros(H)
        for k in range(K):
            e = ids[t, k]
            acc = acc + float(w[t, k]) * orc.ffn(
                L["pg"][e], L["sg"][e], L["pu"][e], L["su"][e], L["pd"][e],
                L["sd"][e], H, F, x[t:t + 1])[0]
        _close(out[t], acc, 1e-13, 1e-15)


def pin_layer_k1_is_ffn(orc):
    rng = _rng(21)
    E, H, F = 3, 128, 64
    L = _rand_layer(orc, rng, E, H, F)
    x = rng.standard_normal((2, H))
    ids = np.array([[2], [2]], np.int32)
    w = np.ones((2, 1), np.float32)
    out, _ = orc.layer(L["pg"], L["sg"], L["pu"], L["su"], L["pd"], L["sd"],
                       H, F, x, ids, w)
    ref = orc.ffn(L["pg"][2], L["sg"][2], L["pu"][2], L["su"][2], L["pd"][2],
                  L["sd"][2], H, F, x)
    assert np.array_equal(out, ref)


def pin_layer_permutation(orc):
    """Permuting tokens permutes outputs; equal rows give equal outputs."""
    rng = _rng(22)
    E, H, F, T, K = 4, 64, 64, 5, 2
    L = _rand_layer(orc, rng, E, H, F)
    x = rng.standard_normal((T, H))
    x[3] = x[1]
    ids = rng.integers(0, E, size=(T, K)).astype(np.int32)
    ids[3] = ids[1]
    w = rng.uniform(0, 1, size=(T, K)).astype(np.float32)
    w[3] = w[1]
    args = (L["pg"], L["sg"], L["pu"], L["su"], L["pd"], L["sd"], H, F)
    out, _ = orc.layer(*args, x, ids, w)
    perm = np.array([4, 2, 0, 1, 3])
    outp, _ = orc.layer(*args, x[perm], ids[perm], w[perm])
    assert np.array_equal(outp, out[perm])
    assert np.array_equal(out[3], out[1])
    assert not np.array_equal(out[0], out[1])


def pin_layer_invalid_ids(orc):
    """Ids outside [0, E) contribute nothing and are counted."""
    rng = _rng(23)
    E, H, F = 3, 64, 64
    L = _rand_layer(orc, rng, E, H, F)
    x = rng.standard_normal((1, H))
    args = (L["pg"], L["sg"], L["pu"], L["su"], L["pd"], L["sd"], H, F)
    good, _ = orc.layer(*args, x, np.array([[1, 2]], np.int32),
                        np.array([[0.5, 0.25]], np.float32))
    mixed, bad = orc.layer(*args, x, np.array([[1, -1, 2, 3]], np.int32),
                           np.array([[0.5, 9.0, 0.25, 7.0]], np.float32))
    assert bad == 2
    assert np.array_equal(good, mixed)



# ---------------------------------------------------------------- router ---

def _route_case_logits(case):
    return np.array([[float(v) for v in row] for row in case["logits"]], dtype=np.float32)


def pin_route_hand(orc):
    """Hand-evaluated picks and weights (ties, NaN / -inf ranking, k = 1)."""
    for case in _golden("hand_cases.json")["route"]:
        ids, w = orc.route(_route_case_logits(case), case["k"])
        assert ids.tolist() == case["ids"], (case["name"], ids.tolist())
        if "w" in case:
            _close(w, case["w"], rtol=1e-7, what=case["name"])


def pin_route_sort_and_softmax_library(orc):
    """Distinct logits: the picks are numpy's descending argsort, the weights
    scipy's softmax over the picked logits (library routines)."""
    from scipy.special import softmax
    rng = _rng(40)
    for (T, E, k) in [(5, 16, 4), (3, 128, 8), (2, 7, 7), (4, 256, 8)]:
        logits = rng.standard_normal((T, E)).astype(np.float32)
        ids, w = orc.route(logits, k)
        ref_ids = np.argsort(-logits.astype(np.float64), axis=1, kind="stable")[:, :k]
        assert np.array_equal(ids, ref_ids)
        picked = np.take_along_axis(logits.astype(np.float64), ref_ids, axis=1)
        ref_w = softmax(picked, axis=1).astype(np.float32)
        _close(w, ref_w, rtol=2e-7, what="softmax")


def pin_route_all_equal(orc):
    """All logits equal: ids 0..k-1 in order, every weight 1/k."""
    logits = np.full((3, 12), 0.75, dtype=np.float32)
    for k in (1, 4, 12):
        ids, w = orc.route(logits, k)
        assert ids.tolist() == [list(range(k))] * 3
        _close(w, np.full((3, k), 1.0 / k), rtol=1e-7, what="uniform")


def pin_route_shift_invariant(orc):
    """Adding a constant to a token's logits changes neither picks nor weights
    (beyond the f32 rounding of the shifted logits)."""
    rng = _rng(41)
    logits = (rng.standard_normal((6, 64)) * 2).astype(np.float32)
    ids0, w0 = orc.route(logits, 8)
    ids1, w1 = orc.route(logits + np.float32(16.0), 8)
    assert np.array_equal(ids0, ids1)
    _close(w1, w0, rtol=2e-5, what="shift")


def pin_route_weights_sum_to_one(orc):
    rng = _rng(42)
    logits = (rng.standard_normal((32, 128)) * 3).astype(np.float32)
    _, w = orc.route(logits, 8)
    _close(w.astype(np.float64).sum(axis=1), np.ones(32), rtol=1e-6, what="sum")
    assert np.all(np.diff(w, axis=1) <= 0), "slot order is descending logit"


# ------------------------------------------------ import / group detection ---

def pin_import_twos_exhaustive(orc):
    """Every byte of a two's-complement container: after import, each nibble
    decodes (offset - 8) to the signed value the two's-complement nibble
    held (n - 16 for n >= 8)."""
    twos = np.arange(256, dtype=np.uint8).reshape(1, 256)
    packed = orc.import_twos(twos, 512)
    q = orc.unpack(packed, 512)[0]
    for b in range(256):
        lo, hi = b & 15, b >> 4
        assert q[2 * b] == (lo - 16 if lo >= 8 else lo), b
        assert q[2 * b + 1] == (hi - 16 if hi >= 8 else hi), b


def pin_import_twos_pad_nibble(orc):
    """Odd I: a two's-complement zero pad nibble imports as the offset pad 8."""
    twos = np.array([[0x07]], dtype=np.uint8)    # element 0 = 7, pad nibble 0
    packed = orc.import_twos(twos, 1)
    assert packed.tolist() == [[0x8F]]


def pin_detect_group_pages(orc):
    """kv_b header: 28,672 rows of 512 inputs with 917,504 scale bytes is gs
    64; the 6144 x 2048 expert matrices (786,432 B of g64 scales) likewise;
    one scale per row (4 B a row) of 512 inputs matches no candidate (the
    widest, 256, still needs two scales per row)."""
    assert orc.detect_group(28672, 512, 917504) == 64
    assert orc.detect_group(2048, 6144, 786432) == 64
    assert orc.detect_group(6144, 2048, 786432) == 64
    assert orc.detect_group(28672, 512, 28672 * 4) == 0


def pin_detect_group_brute(orc):
    """For every candidate and a few shapes, the detected size reproduces the
    byte count, and no smaller candidate does."""
    cands = [16, 32, 48, 64, 96, 128, 192, 256]
    for rows, cols in [(7, 512), (3, 4096), (5, 100), (2, 1536)]:
        for gs in cands:
            nbytes = rows * (-(-cols // gs)) * 4
            got = orc.detect_group(rows, cols, nbytes)
            assert got != 0 and rows * (-(-cols // got)) * 4 == nbytes
            assert all(rows * (-(-cols // c)) * 4 != nbytes for c in cands if c < got)


# ------------------------------------------- per-element error scales ---
# The maintainer comment "Here's the oracle you're missing": a float result is
# judged against the sum of the magnitudes of its terms.

def pin_dsilu_values(orc):
    """silu'(0) = 1/2, silu' -> 1 and 0 at the far ends, silu' = 0 at the
    minimum of silu (z = -1.2784645427610738), and a central difference of the
    oracle's own silu elsewhere."""
    assert orc.dsilu(0.0) == 0.5
    assert abs(orc.dsilu(40.0) - 1.0) <= 1e-15
    assert abs(orc.dsilu(-40.0)) <= 1e-15
    assert abs(orc.dsilu(-1.2784645427610738)) <= 1e-15
    for z in (-3.0, -0.7, 0.3, 1.0, 2.5):
        h = 1e-5
        fd = (orc.silu(z + h) - orc.silu(z - h)) / (2 * h)
        assert abs(orc.dsilu(z) - fd) <= 1e-9, z


def pin_matvec_abs_library(orc):
    """A = |deq(W)| @ |x| (numpy dense); equals y when every term is >= 0;
    never below |y|."""
    rng = _rng(40)
    O, I = 19, 200
    q = rng.integers(-8, 8, size=(O, I), dtype=np.int8)
    s = rng.uniform(0.005, 0.02, size=(O, -(-I // 64))).astype(np.float32)
    x = rng.standard_normal((3, I))
    packed, _ = orc.pack(q)
    a = orc.matvec_abs(packed, s, I, x)
    W = q.astype(np.float64) * s.astype(np.float64)[:, np.arange(I) // 64]
    _close(a, np.abs(x) @ np.abs(W).T, 1e-13, 0, "abs")
    assert np.all(a >= np.abs(orc.matvec(packed, s, I, x)) * (1 - 1e-15))
    qp = np.abs(q).astype(np.int8) % 8
    pp, _ = orc.pack(qp)
    xp = np.abs(x)
    _close(orc.matvec_abs(pp, s, I, xp), orc.matvec(pp, s, I, xp), 1e-15, 0, "nonneg")


def _layer_sensitivity(L, x, ids, w, t, o, H, F):
    """Sum over all gate/up products, h values and down products of
    |d out[t, o] / d(relative error of that quantity)|, by float64 autograd of
    a dense evaluation of the layer (independent of the oracle's C code)."""
    import torch

    def deq(q, s):
        q = torch.as_tensor(q.astype(np.float64))
        s = torch.as_tensor(s.astype(np.float64))
        return q * s[:, torch.arange(q.shape[1]) // 64]
    xt = torch.as_tensor(x[t], dtype=torch.float64)
    total = 0.0
    for j in range(ids.shape[1]):
        e = int(ids[t, j])
        G, U, D = deq(L["qg"][e], L["sg"][e]), deq(L["qu"][e], L["su"][e]), deq(L["qd"][e], L["sd"][e])
        fg = torch.ones(F, H, dtype=torch.float64, requires_grad=True)
        fu = torch.ones(F, H, dtype=torch.float64, requires_grad=True)
        fh = torch.ones(F, dtype=torch.float64, requires_grad=True)
        fd = torch.ones(F, dtype=torch.float64, requires_grad=True)
        g = (G * xt * fg).sum(1)
        u = (U * xt * fu).sum(1)
        h = g * torch.sigmoid(g) * u * fh
        y = (D[o] * h * fd).sum()
        out = float(w[t, j]) * y
        out.backward()
        total += sum(float(v.grad.abs().sum()) for v in (fg, fu, fh, fd))
    return total


def pin_layer_mag_autograd(orc):
    """layer_mag[t, o] = the first-order sensitivity of out[t, o] to unit
    relative errors of all its rounded quantities (float64 autograd)."""
    rng = _rng(41)
    E, H, F, T, K = 3, 128, 64, 2, 2
    L = _rand_layer(orc, rng, E, H, F)
    x = rng.standard_normal((T, H))
    ids = np.array([[2, 0], [1, 2]], np.int32)
    w = np.array([[0.7, -0.3], [0.55, 0.45]], np.float32)     # any sign is accepted
    mag = orc.layer_mag(L["pg"], L["sg"], L["pu"], L["su"], L["pd"], L["sd"], H, F, x, ids, w)
    for t, o in ((0, 0), (0, 77), (1, 5), (1, 127)):
        ref = _layer_sensitivity(L, x, ids, w, t, o, H, F)
        assert abs(mag[t, o] - ref) <= 1e-10 * ref, (t, o, mag[t, o], ref)
    out, _ = orc.layer(L["pg"], L["sg"], L["pu"], L["su"], L["pd"], L["sd"], H, F, x, ids, w)
    assert np.all(mag >= np.abs(out))


def pin_layer_mag_dropped_ids(orc):
    """Dropped ids add nothing; a token with only dropped ids has M = 0."""
    rng = _rng(42)
    E, H, F = 2, 64, 64
    L = _rand_layer(orc, rng, E, H, F)
    x = rng.standard_normal((2, H))
    ids = np.array([[1, -1], [5, -3]], np.int32)
    w = np.ones((2, 2), np.float32)
    mag = orc.layer_mag(L["pg"], L["sg"], L["pu"], L["su"], L["pd"], L["sd"], H, F, x, ids, w)
    one = orc.layer_mag(L["pg"], L["sg"], L["pu"], L["su"], L["pd"], L["sd"], H, F, x[:1],
                        ids[:1, :1], w[:1, :1])
    assert np.array_equal(mag[0], one[0])
    assert np.all(mag[1] == 0.0)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
