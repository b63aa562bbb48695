"""The C-ABI library on a host without a GPU: it loads, exports every entry
point include/qmoe.h declares, reports its ABI version and size formulas, and
rejects bad arguments before any HIP call (no kernel is ever launched here:
every call below fails validation, which runs first)."""
import ctypes
import os
import re

import pytest

import grouped_int4_expert_amd as q
from grouped_int4_expert_amd import qmoe_layer_desc, qmoe_qmat

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qmoe.h")


@pytest.fixture(scope="module")
def lib():
    return q.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qmoe_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(names) == sorted(q.EXPORTS)


def test_abi_version_and_status(lib):
    assert lib.qmoe_abi_version() == q.ABI_VERSION == 1
    for s in range(10):
        assert q.qmoe_status_str(s)
    assert q.qmoe_status_str(999) == "unknown status"


def test_size_formulas(lib):
    # kv_b header of the pull request: 28,672 rows x 256 B, 8 scales per row
    assert q.qmoe_packed_bytes(28672, 512) == 7340032
    assert q.qmoe_scale_count(28672, 512, 64) == 229376
    assert q.qmoe_packed_bytes(3, 5) == 9
    assert q.qmoe_scale_count(3, 5, 2) == 9
    assert q.qmoe_packed_bytes(-1, 4) == 0
    assert q.qmoe_scale_count(4, 4, 0) == 0


FAKE = 1 << 40   # a 16-byte aligned address that is never dereferenced


def qmat(rows, cols, group=64, q_=FAKE, s_=FAKE + (1 << 30), qs=0, ss=0, size=None):
    m = qmoe_qmat()
    m.struct_size = ctypes.sizeof(qmoe_qmat) if size is None else size
    m.rows, m.cols, m.group = rows, cols, group
    m.q, m.s = q_, s_
    m.q_expert_stride, m.s_expert_stride = qs, ss
    return m


def layer_desc(E=4, H=256, F=128, group=64, size=None):
    d = qmoe_layer_desc()
    d.struct_size = ctypes.sizeof(qmoe_layer_desc) if size is None else size
    d.experts, d.hidden, d.inter, d.group = E, H, F, group
    step = 1 << 32
    d.gate = qmat(F, H, group, FAKE, FAKE + step, F * H // 2, F * H // 64)
    d.up = qmat(F, H, group, FAKE + 2 * step, FAKE + 3 * step, F * H // 2, F * H // 64)
    d.down = qmat(H, F, group, FAKE + 4 * step, FAKE + 5 * step, H * F // 2, H * F // 64)
    return d


def call_layer(lib, d, dtype=0, x=FAKE + (6 << 32), T=2, ids=FAKE + (7 << 32),
               w=FAKE + (8 << 32), k=2, out=FAKE + (9 << 32), ws=FAKE + (10 << 32),
               ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = lib.qmoe_layer_workspace_bytes(ctypes.byref(d), T, k, dtype)
    return lib.qmoe_layer(ctypes.byref(d), dtype, x, T, ids, w, k, out, ws, ws_bytes, None)


def test_layer_rejections(lib):
    d = layer_desc()
    assert call_layer(lib, layer_desc(size=8)) == 7                     # ABI
    d2 = layer_desc()
    d2.gate.struct_size = 4
    assert call_layer(lib, d2) == 7
    assert call_layer(lib, layer_desc(group=96)) == 4                   # UNSUPPORTED
    assert call_layer(lib, layer_desc(group=48)) == 4
    d3 = layer_desc(group=128)
    d3.down.group = 64                                                  # groups differ
    assert call_layer(lib, d3) == 2
    d4 = layer_desc(group=32)
    d4.gate.s_expert_stride = 128 * 256 // 64                           # too few scales for 32
    assert call_layer(lib, d4) == 2
    assert call_layer(lib, layer_desc(H=200)) == 4
    assert call_layer(lib, layer_desc(E=0)) == 2                        # SHAPE
    assert call_layer(lib, layer_desc(E=2000)) == 2
    assert call_layer(lib, d, dtype=7) == 4
    assert call_layer(lib, d, k=0) == 2
    assert call_layer(lib, d, x=None) == 1                              # NULL
    assert call_layer(lib, d, out=None) == 1
    assert call_layer(lib, d, x=FAKE + 4) == 3                          # ALIGN
    assert call_layer(lib, d, ids=FAKE + 2) == 3
    assert call_layer(lib, d, ws=None) == 5                             # WORKSPACE
    assert call_layer(lib, d, ws_bytes=16) == 5
    assert call_layer(lib, d, out=FAKE + (6 << 32)) == 6                # ALIAS out == x
    assert call_layer(lib, d, ws=FAKE + (9 << 32)) == 6                 # ws == out
    assert call_layer(lib, d, T=0) == 0                                 # nothing to do
    d3 = layer_desc()
    d3.down.rows = 128
    assert call_layer(lib, d3) == 2
    d4 = layer_desc()
    d4.up.q = FAKE + 8
    assert call_layer(lib, d4) == 3
    d5 = layer_desc()
    d5.gate.q_expert_stride = 16
    assert call_layer(lib, d5) == 2
    d6 = layer_desc()
    d6.gate.s = None
    assert call_layer(lib, d6) == 1
    # bf16 path: a tile's h and Y rows go through one descriptor each, so
    # hidden and inter stay below 2^22
    assert call_layer(lib, layer_desc(H=1 << 22, F=64), dtype=1) == 2
    assert call_layer(lib, layer_desc(H=64, F=1 << 22), dtype=1) == 2


def test_matvec_and_pack_rejections(lib):
    W = qmat(256, 1024)
    nb = lib.qmoe_matvec_workspace_bytes(ctypes.byref(W), 1)
    assert nb == 0                       # f32 activations are read as they are
    ws = FAKE + (20 << 32)
    # a width that is not a multiple of 64 (partial last group) is taken, with
    # a re-laid copy of W in the workspace: rows * 1024/2 bytes + 16 scales
    Wp = qmat(256, 1000)
    nbp = lib.qmoe_matvec_workspace_bytes(ctypes.byref(Wp), 1)
    assert nbp >= 256 * 512 + 256 * 16 * 4
    assert lib.qmoe_matvec(ctypes.byref(Wp), FAKE, 1, FAKE + (30 << 32), ws, nb, None) == 5
    assert lib.qmoe_matvec(ctypes.byref(qmat(256, 1000, q_=ws + 4096)), FAKE + (40 << 32), 1,
                           FAKE + (30 << 32), ws, nbp, None) == 6      # workspace overlaps W
    assert lib.qmoe_matvec(ctypes.byref(qmat(256, 1000, group=96)), FAKE, 1, FAKE + (30 << 32),
                           ws, nbp, None) == 4
    assert lib.qmoe_matvec(ctypes.byref(qmat(4, 20000)), FAKE, 1, FAKE + (30 << 32), ws,
                           1 << 30, None) == 4                            # wider than any shape
    assert lib.qmoe_matvec(ctypes.byref(qmat(1 << 20, 4096)), FAKE, 1, FAKE + (30 << 32), ws,
                           1 << 40, None) == 4                            # 2 GB of codes
    assert lib.qmoe_matvec(ctypes.byref(qmat(256, 1024, size=3)), FAKE, 1, FAKE, ws, nb,
                           None) == 7
    assert lib.qmoe_matvec(ctypes.byref(W), None, 1, FAKE + (30 << 32), ws, nb, None) == 1
    assert lib.qmoe_matvec(ctypes.byref(W), FAKE + 8, 1, FAKE + (30 << 32), ws, nb, None) == 3
    assert lib.qmoe_matvec(ctypes.byref(Wp), FAKE + (40 << 32), 1, FAKE + (30 << 32), ws, 8,
                           None) == 5
    assert lib.qmoe_matvec(ctypes.byref(Wp), FAKE + (40 << 32), 1, FAKE + (30 << 32), None,
                           nbp, None) == 5
    assert lib.qmoe_matvec(ctypes.byref(W), FAKE + (40 << 32), 1, FAKE + (40 << 32), ws, nb,
                           None) == 6
    assert lib.qmoe_matvec(ctypes.byref(W), FAKE, 0, FAKE, ws, nb, None) == 0
    assert lib.qmoe_pack(None, 4, 4, FAKE, None, None) == 1
    assert lib.qmoe_pack(FAKE, -1, 4, FAKE, None, None) == 2
    assert lib.qmoe_pack(FAKE, 4, 64, FAKE + 8, None, None) == 6       # packed overlaps q
    assert lib.qmoe_pack(FAKE, 0, 4, FAKE, None, None) == 0
    assert lib.qmoe_worklist(FAKE, 4, 0, 8, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None) == 2
    assert lib.qmoe_worklist(FAKE, 4, 2, 8, None, FAKE, FAKE, FAKE, FAKE, None, 0, None) == 1
    a = FAKE + (50 << 32)
    assert lib.qmoe_worklist(FAKE, 4, 2, 8, a, a, a + 4096, a + 8192, a + 12288, None, 0,
                             None) == 6


def test_expert_ffn_rejections(lib):
    G, U, D = qmat(128, 256), qmat(128, 256), qmat(256, 128)
    nb = lib.qmoe_expert_ffn_workspace_bytes(ctypes.byref(G), ctypes.byref(U), ctypes.byref(D),
                                             0, 2)
    ws = FAKE + (20 << 32)
    args = lambda x_dtype, x, out: lib.qmoe_expert_ffn(  # noqa: E731
        ctypes.byref(G), ctypes.byref(U), ctypes.byref(D), x_dtype, x, 2, out, ws, nb, None)
    assert args(3, FAKE, FAKE + (30 << 32)) == 4
    assert args(0, None, FAKE + (30 << 32)) == 1
    assert args(0, FAKE + (30 << 32), FAKE + (30 << 32)) == 6
    D2 = qmat(256, 192)
    assert lib.qmoe_expert_ffn(ctypes.byref(G), ctypes.byref(U), ctypes.byref(D2), 0, FAKE, 2,
                               FAKE + (30 << 32), ws, nb, None) == 2


def test_route_rejections(lib):
    L, I, W = FAKE, FAKE + (50 << 32), FAKE + (51 << 32)
    assert lib.qmoe_route(L, 4, 128, 0, I, W, None) == 2          # k < 1
    assert lib.qmoe_route(L, 4, 8, 9, I, W, None) == 2            # k > experts
    assert lib.qmoe_route(L, -1, 128, 8, I, W, None) == 2         # tokens < 0
    assert lib.qmoe_route(L, 4, 0, 1, I, W, None) == 2            # no experts
    assert lib.qmoe_route(L, 4, 128, 17, I, W, None) == 4         # k beyond 16
    assert lib.qmoe_route(L, 4, 2048, 8, I, W, None) == 4         # experts beyond 1024
    assert lib.qmoe_route(None, 4, 128, 8, I, W, None) == 1
    assert lib.qmoe_route(L, 4, 128, 8, None, W, None) == 1
    assert lib.qmoe_route(L + 2, 4, 128, 8, I, W, None) == 3      # misaligned logits
    assert lib.qmoe_route(L, 4, 128, 8, L + 64, W, None) == 6     # ids inside the logits
    assert lib.qmoe_route(L, 4, 128, 8, I, I + 16, None) == 6     # ids and weights overlap
    assert lib.qmoe_route(L, 0, 128, 8, None, None, None) == 0    # nothing to do


def test_import_twos_rejections(lib):
    assert lib.qmoe_import_twos(None, 4, 64, FAKE, None) == 1
    assert lib.qmoe_import_twos(FAKE, -1, 64, FAKE, None) == 2
    assert lib.qmoe_import_twos(FAKE, 4, 64, FAKE + 16, None) == 6   # partial overlap
    assert lib.qmoe_import_twos(FAKE, 0, 64, FAKE, None) == 0        # nothing to do


def test_detect_group_matches_oracle(lib):
    # host-only entry point: the library and the oracle agree everywhere
    import oracle
    orc = oracle.Oracle()
    for rows in (1, 3, 7, 2048):
        for cols in (1, 31, 64, 100, 512, 1536, 4096, 6144):
            for gs in (8, 16, 32, 48, 64, 96, 128, 192, 256, 512, 100000):
                nb = rows * (-(-cols // gs)) * 4
                for b in (nb, nb + 4, nb - 4):
                    assert lib.qmoe_detect_group(rows, cols, b) == orc.detect_group(rows, cols, b)
    assert lib.qmoe_detect_group(28672, 512, 917504) == 64


def test_cache_create_validation(lib):
    host, dev = layer_desc(E=16), layer_desc(E=4)
    h = ctypes.c_void_p()
    assert lib.qmoe_cache_create(ctypes.byref(host), ctypes.byref(dev), ctypes.byref(h)) == 0
    assert h.value
    assert lib.qmoe_cache_resident(h, 3) == -1          # nothing resident yet
    assert lib.qmoe_cache_resident(h, 99) == -1
    # prepare with no pairs enqueues nothing
    n = ctypes.c_int64(7)
    assert lib.qmoe_cache_prepare(h, None, 0, 2, None, ctypes.byref(n), None) == 0
    assert n.value == 0
    assert lib.qmoe_cache_prepare(h, None, 2, 2, None, None, None) == 1
    assert lib.qmoe_cache_prepare(h, FAKE, 2, 0, FAKE, None, None) == 2
    lib.qmoe_cache_destroy(h)
    bad = layer_desc(E=4, H=512)                         # other shape
    assert lib.qmoe_cache_create(ctypes.byref(host), ctypes.byref(bad), ctypes.byref(h)) == 2
    bad = layer_desc(E=4, size=8)
    assert lib.qmoe_cache_create(ctypes.byref(host), ctypes.byref(bad), ctypes.byref(h)) == 7
    nul = layer_desc(E=16)
    nul.up.q = None
    assert lib.qmoe_cache_create(ctypes.byref(nul), ctypes.byref(dev), ctypes.byref(h)) == 1
    assert lib.qmoe_cache_create(None, ctypes.byref(dev), ctypes.byref(h)) == 1


def test_cache_device_validation(lib):
    host, dev = layer_desc(E=16), layer_desc(E=4)
    h = ctypes.c_void_p()
    assert lib.qmoe_cache_create(ctypes.byref(host), ctypes.byref(dev), ctypes.byref(h)) == 0
    nb = lib.qmoe_cache_device_state_bytes(16, 4)
    assert nb == 4 * (4 + 16 + 5 * 4)
    assert lib.qmoe_cache_device_state_bytes(0, 4) == 0
    assert lib.qmoe_cache_device_state_bytes(16, 0) == 0
    # rejections happen before anything is enqueued
    assert lib.qmoe_cache_device_init(None, FAKE, nb, None) == 1
    assert lib.qmoe_cache_device_init(h, None, nb, None) == 1
    assert lib.qmoe_cache_device_init(h, FAKE, nb - 4, None) == 5
    assert lib.qmoe_cache_device_init(h, FAKE + 2, nb, None) == 3
    assert lib.qmoe_cache_prepare_device(h, FAKE, nb, None, 2, 2, None, None) == 1
    assert lib.qmoe_cache_prepare_device(h, FAKE, nb, FAKE, 2, 0, FAKE, None) == 2
    assert lib.qmoe_cache_prepare_device(h, FAKE, nb, FAKE, -1, 2, FAKE, None) == 2
    assert lib.qmoe_cache_prepare_device(h, FAKE, nb - 4, FAKE, 2, 2, FAKE, None) == 5
    assert lib.qmoe_cache_prepare_device(h, None, nb, FAKE, 2, 2, FAKE, None) == 1
    lib.qmoe_cache_destroy(h)
    # more slots than the device tables hold
    big = layer_desc(E=2000)
    assert lib.qmoe_cache_create(ctypes.byref(layer_desc(E=3000)), ctypes.byref(big),
                                 ctypes.byref(h)) == 0
    nb = lib.qmoe_cache_device_state_bytes(3000, 2000)
    assert lib.qmoe_cache_device_init(h, FAKE, nb, None) == 4
    assert lib.qmoe_cache_prepare_device(h, FAKE, nb, FAKE, 2, 2, FAKE, None) == 4
    lib.qmoe_cache_destroy(h)


def test_layer_logits_validation(lib):
    d = layer_desc()
    T, k = 2, 2
    nb = lib.qmoe_layer_logits_workspace_bytes(ctypes.byref(d), T, k, 0)
    assert nb >= lib.qmoe_layer_workspace_bytes(ctypes.byref(d), T, k, 0) + 2 * 256
    X, L, O, W = FAKE + (60 << 32), FAKE + (61 << 32), FAKE + (62 << 32), FAKE + (63 << 32)
    assert lib.qmoe_layer_logits(ctypes.byref(d), 0, X, T, L, 0, O, W, nb, None) == 2
    assert lib.qmoe_layer_logits(ctypes.byref(d), 0, X, T, L, 17, O, W, nb, None) == 4
    assert lib.qmoe_layer_logits(ctypes.byref(d), 0, X, T, None, k, O, W, nb, None) == 1
    assert lib.qmoe_layer_logits(ctypes.byref(d), 0, X, T, L + 2, k, O, W, nb, None) == 3
    assert lib.qmoe_layer_logits(ctypes.byref(d), 0, X, T, L, k, O, W, nb - 16, None) == 5
    assert lib.qmoe_layer_logits(ctypes.byref(d), 0, X, T, W + 64, k, O, W, nb, None) == 6
    # a bad layer argument is caught before the router would run
    assert lib.qmoe_layer_logits(ctypes.byref(d), 0, None, T, L, k, O, W, nb, None) == 1
    assert lib.qmoe_layer_logits(ctypes.byref(d), 0, X, T, L, k, X, W, nb, None) == 6
    assert lib.qmoe_layer_logits(ctypes.byref(d), 0, X, 0, None, k, None, None, 0, None) == 0


def test_layer_noalloc_rejections(lib):
    """The allocation-free layer refuses, before touching any device, a stale
    descriptor, bad sizes and a call whose workspace exceeds its fixed scratch."""
    def call(d, dtype=0, T=2, k=2):
        return lib.qmoe_layer_noalloc(ctypes.byref(d), dtype, FAKE + (6 << 32), T,
                                      FAKE + (7 << 32), FAKE + (8 << 32), k,
                                      FAKE + (9 << 32), None)
    assert call(layer_desc(size=8)) == 7
    assert call(layer_desc(), k=0) == 2
    assert call(layer_desc(), T=-1) == 2
    assert call(layer_desc(), dtype=7) == 4
    big = layer_desc(E=4, H=4096, F=1536)
    need = lib.qmoe_layer_workspace_bytes(ctypes.byref(big), 4096, 8, 1)
    assert need > q.NOALLOC_SCRATCH_BYTES
    assert call(big, dtype=1, T=4096, k=8) == 9
    assert q.qmoe_status_str(9).startswith("needs more workspace")


def test_stream_probe_validation(lib):
    # every case fails before a launch
    S = FAKE + (4 << 30)   # sink far from the buffer
    assert lib.qmoe_stream_probe(None, 1024, 0, S, None) == 1   # NULL
    assert lib.qmoe_stream_probe(FAKE, 1024, 0, None, None) == 1   # NULL
    assert lib.qmoe_stream_probe(FAKE, 1024, 2, S, None) == 4   # UNSUPPORTED
    assert lib.qmoe_stream_probe(FAKE, 0, 0, S, None) == 2   # SHAPE
    assert lib.qmoe_stream_probe(FAKE, (1 << 30) + 16, 0, S, None) == 2   # SHAPE
    assert lib.qmoe_stream_probe(FAKE, 4096 + 16, 1, S, None) == 2   # SHAPE
    assert lib.qmoe_stream_probe(FAKE + 8, 1024, 0, S, None) == 3   # ALIGN
    assert lib.qmoe_stream_probe(FAKE, 1024, 0, S + 2, None) == 3   # ALIGN
    assert lib.qmoe_stream_probe(FAKE, 1 << 20, 0, FAKE + 4096, None) == 6   # ALIAS
