"""CPU oracle for the grouped-int4 (gs=64) MoE expert path -- TEST
INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  The product library never loads it, and it
never loads the product library.

The arithmetic lives in ``qmoe_oracle.c`` (plain scalar C, fp64); this file
only builds it with gcc and marshals numpy arrays through ctypes.  Every
floating input is widened exactly to float64 before the call (f32 and bf16
are exact in double), so the oracle sees the same numbers the GPU sees.

Parity status of each function (what pins it is in ``tests/test_oracle_*``):
pack/unpack, import_twos, detect_group, matvec, pair, silu, ffn, worklist,
layer and route are all pinned by hand-written values, closed forms or brute
force; dsilu, matvec_abs and layer_mag (the scales of the per-element error
check) by closed forms and by perturbing a separate float64 evaluation of
the layer; none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qmoe_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(cflags=None, out=None) -> str:
    """Compile the oracle with gcc (no OpenMP, -O2, strict IEEE double)."""
    out = out or _LIB
    flags = cflags if cflags is not None else []
    cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC",
           "-shared", "-std=c99", "-Wall", "-Werror", *flags, _SRC, "-o",
           out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


_OMP_SRC = os.path.join(_HERE, "baseline_omp.c")
_OMP_LIB = os.path.join(_HERE, "liboracle_omp.so")
_omp = None


def build_omp(out=None) -> str:
    """The same oracle source plus the all-cores baseline driver (an OpenMP
    parallel for over tokens around the unchanged orc_layer), in a library
    of its own: used only by the benchmark's CPU-baseline leg."""
    out = out or _OMP_LIB
    cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared",
           "-std=c99", "-Wall", "-Werror", "-fopenmp", _SRC, _OMP_SRC, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def load_omp():
    global _omp
    if _omp is not None:
        return _omp
    if not os.path.exists(_OMP_LIB):
        build_omp()
    lib = ctypes.CDLL(_OMP_LIB)
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    lib.orc_layer_omp.restype = i64
    lib.orc_layer_omp.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, vp, i64, vp, vp,
                                  i64, vp]
    lib.orc_omp_threads.restype = ctypes.c_int
    lib.orc_omp_threads.argtypes = []
    _omp = lib
    return lib


def layer_omp(pg, sg, pu, su, pd, sd, hidden, inter, x, ids, w, gs=64):
    """orc_layer over all tokens on all host cores (OpenMP over tokens).
    Returns (out, n_invalid, threads)."""
    lib = load_omp()
    pg, pu, pd = (_c(_np(a), np.uint8) for a in (pg, pu, pd))
    sg, su, sd = (_c(_np(a), np.float32) for a in (sg, su, sd))
    experts = pg.shape[0]
    x = _c(_np(x), np.float64).reshape(-1, hidden)
    ids = _c(_np(ids), np.int32)
    w = _c(_np(w), np.float32)
    tokens, k = ids.shape
    out = np.empty((tokens, hidden), dtype=np.float64)
    bad = lib.orc_layer_omp(_p(pg), _p(sg), _p(pu), _p(su), _p(pd), _p(sd), experts, hidden,
                            inter, gs, _p(x), tokens, _p(ids), _p(w), k, _p(out))
    return out, int(bad), int(lib.orc_omp_threads())


def load(path=None):
    """Load (building once if missing) and declare the C signatures."""
    global _lib
    if path is None and _lib is not None:
        return _lib
    p = path or _LIB
    if not os.path.exists(p):
        build(out=p)
    lib = ctypes.CDLL(p)
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    lib.orc_row_bytes.restype = i64
    lib.orc_row_bytes.argtypes = [i64]
    lib.orc_groups.restype = i64
    lib.orc_groups.argtypes = [i64, i64]
    lib.orc_packed_bytes.restype = i64
    lib.orc_packed_bytes.argtypes = [i64, i64]
    lib.orc_scale_count.restype = i64
    lib.orc_scale_count.argtypes = [i64, i64, i64]
    lib.orc_pack.restype = i64
    lib.orc_pack.argtypes = [vp, i64, i64, vp]
    lib.orc_unpack.restype = None
    lib.orc_unpack.argtypes = [vp, i64, i64, vp]
    lib.orc_code.restype = ctypes.c_int
    lib.orc_code.argtypes = [vp, i64, i64, i64]
    lib.orc_weight.restype = ctypes.c_double
    lib.orc_weight.argtypes = [vp, vp, i64, i64, i64, i64]
    lib.orc_matvec.restype = None
    lib.orc_matvec.argtypes = [vp, vp, i64, i64, i64, vp, i64, vp]
    lib.orc_pair.restype = None
    lib.orc_pair.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp, i64, vp, vp]
    lib.orc_silu.restype = ctypes.c_double
    lib.orc_silu.argtypes = [ctypes.c_double]
    lib.orc_ffn.restype = None
    lib.orc_ffn.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, vp, i64, vp]
    lib.orc_worklist.restype = i64
    lib.orc_worklist.argtypes = [vp, i64, i64, i64, vp, vp, vp, vp]
    lib.orc_layer.restype = i64
    lib.orc_layer.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, vp,
                              i64, vp, vp, i64, vp]
    lib.orc_route.restype = None
    lib.orc_route.argtypes = [vp, i64, i64, i64, vp, vp]
    lib.orc_import_twos.restype = None
    lib.orc_import_twos.argtypes = [vp, i64, i64, vp]
    lib.orc_detect_group.restype = i64
    lib.orc_detect_group.argtypes = [i64, i64, i64]
    lib.orc_dsilu.restype = ctypes.c_double
    lib.orc_dsilu.argtypes = [ctypes.c_double]
    lib.orc_matvec_abs.restype = None
    lib.orc_matvec_abs.argtypes = [vp, vp, i64, i64, i64, vp, i64, vp]
    lib.orc_layer_mag.restype = None
    lib.orc_layer_mag.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, vp,
                                  i64, vp, vp, i64, vp]
    if path is None:
        _lib = lib
    return lib


def _c(a, dtype):
    a = np.ascontiguousarray(np.asarray(a), dtype=dtype)
    return a


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _np(t):
    """torch tensor or array -> numpy (bf16 widened exactly to f32)."""
    try:
        import torch
        if isinstance(t, torch.Tensor):
            t = t.detach().cpu()
            if t.dtype == torch.bfloat16:
                t = t.to(torch.float32)
            return t.numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(t)


class Oracle:
    """numpy-facing wrapper; ``lib`` may be a mutant build for pin tests."""

    def __init__(self, lib=None):
        self.lib = lib or load()

    # sizes
    def packed_bytes(self, rows, cols):
        return int(self.lib.orc_packed_bytes(rows, cols))

    def scale_count(self, rows, cols, gs=64):
        return int(self.lib.orc_scale_count(rows, cols, gs))

    def row_bytes(self, cols):
        return int(self.lib.orc_row_bytes(cols))

    def groups(self, cols, gs=64):
        return int(self.lib.orc_groups(cols, gs))

    # format
    def pack(self, q):
        q = _c(_np(q), np.int8)
        rows, cols = q.shape[-2], q.shape[-1]
        lead = q.shape[:-2]
        nmat = int(np.prod(lead)) if lead else 1
        q2 = q.reshape(nmat * rows, cols)
        out = np.empty((nmat * rows, self.row_bytes(cols)), dtype=np.uint8)
        bad = self.lib.orc_pack(_p(q2), nmat * rows, cols, _p(out))
        return out.reshape(*lead, rows, self.row_bytes(cols)), int(bad)

    def unpack(self, packed, cols):
        packed = _c(_np(packed), np.uint8)
        rows = int(np.prod(packed.shape[:-1]))
        out = np.empty((rows, cols), dtype=np.int8)
        self.lib.orc_unpack(_p(packed), rows, cols, _p(out))
        return out.reshape(*packed.shape[:-1], cols)

    def weight(self, packed, scales, cols, gs, o, i):
        packed = _c(_np(packed), np.uint8)
        scales = _c(_np(scales), np.float32)
        return float(self.lib.orc_weight(_p(packed), _p(scales), cols, gs, o, i))

    # float ops
    def matvec(self, packed, scales, cols, x, gs=64):
        packed = _c(_np(packed), np.uint8)
        scales = _c(_np(scales), np.float32)
        x = _c(_np(x), np.float64)
        rows = packed.shape[0]
        xb = x.reshape(-1, cols)
        y = np.empty((xb.shape[0], rows), dtype=np.float64)
        self.lib.orc_matvec(_p(packed), _p(scales), rows, cols, gs, _p(xb),
                            xb.shape[0], _p(y))
        return y

    def pair(self, pg, sg, pu, su, cols, x, gs=64):
        pg, pu = _c(_np(pg), np.uint8), _c(_np(pu), np.uint8)
        sg, su = _c(_np(sg), np.float32), _c(_np(su), np.float32)
        x = _c(_np(x), np.float64)
        rows = pg.shape[0]
        xb = x.reshape(-1, cols)
        yg = np.empty((xb.shape[0], rows), dtype=np.float64)
        yu = np.empty_like(yg)
        self.lib.orc_pair(_p(pg), _p(sg), _p(pu), _p(su), rows, cols, gs,
                          _p(xb), xb.shape[0], _p(yg), _p(yu))
        return yg, yu

    def silu(self, z):
        return float(self.lib.orc_silu(float(z)))

    def ffn(self, pg, sg, pu, su, pd, sd, hidden, inter, x, gs=64):
        arrs = [_c(_np(a), np.uint8) if i % 2 == 0 else _c(_np(a), np.float32)
                for i, a in enumerate((pg, sg, pu, su, pd, sd))]
        x = _c(_np(x), np.float64).reshape(-1, hidden)
        out = np.empty((x.shape[0], hidden), dtype=np.float64)
        self.lib.orc_ffn(*[_p(a) for a in arrs], hidden, inter, gs, _p(x),
                         x.shape[0], _p(out))
        return out

    def worklist(self, ids, experts):
        ids = _c(_np(ids), np.int32)
        tokens, k = ids.shape
        n = tokens * k
        counts = np.empty(experts, np.int32)
        offsets = np.empty(experts + 1, np.int32)
        pairs = np.empty(n, np.int32)
        inv = np.empty(n, np.int32)
        bad = self.lib.orc_worklist(_p(ids), tokens, k, experts, _p(counts),
                                    _p(offsets), _p(pairs), _p(inv))
        return dict(counts=counts, offsets=offsets, pairs=pairs, inv=inv,
                    n_invalid=int(bad))

    def layer(self, pg, sg, pu, su, pd, sd, hidden, inter, x, ids, w, gs=64):
        pg, pu, pd = (_c(_np(a), np.uint8) for a in (pg, pu, pd))
        sg, su, sd = (_c(_np(a), np.float32) for a in (sg, su, sd))
        experts = pg.shape[0]
        x = _c(_np(x), np.float64).reshape(-1, hidden)
        ids = _c(_np(ids), np.int32)
        w = _c(_np(w), np.float32)
        tokens, k = ids.shape
        out = np.empty((tokens, hidden), dtype=np.float64)
        bad = self.lib.orc_layer(_p(pg), _p(sg), _p(pu), _p(su), _p(pd),
                                 _p(sd), experts, hidden, inter, gs, _p(x),
                                 tokens, _p(ids), _p(w), k, _p(out))
        return out, int(bad)

    def dsilu(self, z):
        return float(self.lib.orc_dsilu(float(z)))

    def matvec_abs(self, packed, scales, cols, x, gs=64):
        """A[b, o] = sum_i |deq(W)[o, i] x[b, i]| (per-element error scale)."""
        packed = _c(_np(packed), np.uint8)
        scales = _c(_np(scales), np.float32)
        x = _c(_np(x), np.float64)
        rows = packed.shape[0]
        xb = x.reshape(-1, cols)
        a = np.empty((xb.shape[0], rows), dtype=np.float64)
        self.lib.orc_matvec_abs(_p(packed), _p(scales), rows, cols, gs, _p(xb),
                                xb.shape[0], _p(a))
        return a

    def layer_mag(self, pg, sg, pu, su, pd, sd, hidden, inter, x, ids, w, gs=64):
        """M[t, o]: first-order change of out[t, o] under a unit relative error
        of every gate/up product, every h and every down product."""
        pg, pu, pd = (_c(_np(a), np.uint8) for a in (pg, pu, pd))
        sg, su, sd = (_c(_np(a), np.float32) for a in (sg, su, sd))
        experts = pg.shape[0]
        x = _c(_np(x), np.float64).reshape(-1, hidden)
        ids = _c(_np(ids), np.int32)
        w = _c(_np(w), np.float32)
        tokens, k = ids.shape
        mag = np.empty((tokens, hidden), dtype=np.float64)
        self.lib.orc_layer_mag(_p(pg), _p(sg), _p(pu), _p(su), _p(pd), _p(sd), experts,
                               hidden, inter, gs, _p(x), tokens, _p(ids), _p(w), k, _p(mag))
        return mag

    def route(self, logits, k):
        """Top-k ids (pick order) and f32 softmax weights over the picked."""
        logits = _c(_np(logits), np.float32)
        tokens, experts = logits.shape
        ids = np.empty((tokens, k), np.int32)
        w = np.empty((tokens, k), np.float32)
        self.lib.orc_route(_p(logits), tokens, experts, k, _p(ids), _p(w))
        return ids, w

    def import_twos(self, twos, cols):
        """Two's-complement nibble container -> offset container."""
        twos = _c(_np(twos), np.uint8)
        rows = int(np.prod(twos.shape[:-1]))
        out = np.empty_like(twos)
        self.lib.orc_import_twos(_p(twos), rows, cols, _p(out))
        return out

    def detect_group(self, rows, cols, scale_bytes):
        return int(self.lib.orc_detect_group(rows, cols, scale_bytes))
