"""Python binding of libqmoe.so (grouped int4, gs = 64, MoE expert matmul on
MI355X).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/qmoe.h``.  PyTorch provides
device memory and the current stream.  There is no CPU fallback: if the
library is missing or a call fails, an exception is raised.

Names mirror the C entry points (``qmoe_pack``, ``qmoe_matvec``,
``qmoe_expert_ffn``, ``qmoe_worklist``, ``qmoe_layer`` ...).
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqmoe.so")
ABI_VERSION = 1

QMOE_OK = 0
QMOE_F32 = 0
QMOE_BF16 = 1
QMOE_F32_DIGITS = 2      # f32 x, activations rounded to 18-bit block fixed point
STATUS = {0: "QMOE_OK", 1: "QMOE_ERR_NULL", 2: "QMOE_ERR_SHAPE", 3: "QMOE_ERR_ALIGN",
          4: "QMOE_ERR_UNSUPPORTED", 5: "QMOE_ERR_WORKSPACE", 6: "QMOE_ERR_ALIAS",
          7: "QMOE_ERR_ABI", 8: "QMOE_ERR_HIP", 9: "QMOE_ERR_SCRATCH"}
NOALLOC_SCRATCH_BYTES = 64 << 20


class QmoeError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({_lib_status_str(status)})")


class qmoe_qmat(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("rows", ctypes.c_int32),
                ("cols", ctypes.c_int32), ("group", ctypes.c_int32),
                ("q", ctypes.c_void_p), ("s", ctypes.c_void_p),
                ("q_expert_stride", ctypes.c_int64), ("s_expert_stride", ctypes.c_int64)]


class qmoe_layer_desc(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("experts", ctypes.c_int32),
                ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("group", ctypes.c_int32), ("gate", qmoe_qmat), ("up", qmoe_qmat),
                ("down", qmoe_qmat)]


class qmoe_layer_ws_view(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("counts", ctypes.c_int64),
                ("offsets", ctypes.c_int64), ("pairs", ctypes.c_int64),
                ("inv", ctypes.c_int64), ("n_invalid", ctypes.c_int64)]


EXPORTS = ["qmoe_abi_version", "qmoe_status_str", "qmoe_packed_bytes", "qmoe_scale_count",
           "qmoe_pack", "qmoe_unpack", "qmoe_matvec_workspace_bytes", "qmoe_matvec",
           "qmoe_expert_ffn_workspace_bytes", "qmoe_expert_ffn",
           "qmoe_worklist_workspace_bytes", "qmoe_worklist", "qmoe_layer_workspace_bytes",
           "qmoe_layer", "qmoe_layer_ex", "qmoe_layer_ws_layout", "qmoe_route",
           "qmoe_import_twos", "qmoe_detect_group", "qmoe_cache_create", "qmoe_cache_destroy",
           "qmoe_cache_prepare", "qmoe_cache_resident", "qmoe_cache_device_state_bytes",
           "qmoe_cache_device_init", "qmoe_cache_prepare_device", "qmoe_layer_logits_workspace_bytes",
           "qmoe_layer_logits", "qmoe_layer_noalloc", "qmoe_prefill_pass_rows",
           "qmoe_stream_probe"]

_lib = None


def load(path: str | None = None):
    """Load libqmoe.so and declare signatures.  Raises if it is missing or
    was built from another ABI version."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"libqmoe.so not built ({p}); run __graft_entry__.build()")
    lib = ctypes.CDLL(p)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    sig = {
        "qmoe_abi_version": (ctypes.c_int, []),
        "qmoe_status_str": (ctypes.c_char_p, [ctypes.c_int]),
        "qmoe_packed_bytes": (sz, [i64, i64]),
        "qmoe_scale_count": (sz, [i64, i64, i64]),
        "qmoe_pack": (ctypes.c_int, [vp, i64, i64, vp, vp, vp]),
        "qmoe_unpack": (ctypes.c_int, [vp, i64, i64, vp, vp]),
        "qmoe_matvec_workspace_bytes": (sz, [ctypes.POINTER(qmoe_qmat), i32]),
        "qmoe_matvec": (ctypes.c_int, [ctypes.POINTER(qmoe_qmat), vp, i32, vp, vp, sz, vp]),
        "qmoe_expert_ffn_workspace_bytes": (sz, [ctypes.POINTER(qmoe_qmat)] * 3 + [i32, i32]),
        "qmoe_expert_ffn": (ctypes.c_int, [ctypes.POINTER(qmoe_qmat)] * 3 +
                            [i32, vp, i32, vp, vp, sz, vp]),
        "qmoe_worklist_workspace_bytes": (sz, [i32, i32, i32]),
        "qmoe_worklist": (ctypes.c_int, [vp, i32, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp]),
        "qmoe_layer_workspace_bytes": (sz, [ctypes.POINTER(qmoe_layer_desc), i32, i32, i32]),
        "qmoe_layer": (ctypes.c_int, [ctypes.POINTER(qmoe_layer_desc), i32, vp, i32, vp, vp,
                                      i32, vp, vp, sz, vp]),
        "qmoe_layer_ex": (ctypes.c_int, [ctypes.POINTER(qmoe_layer_desc), i32, vp, i32, vp, vp,
                                         i32, vp, vp, sz, vp, ctypes.POINTER(ctypes.c_void_p),
                                         i32]),
        "qmoe_layer_ws_layout": (ctypes.c_int, [ctypes.POINTER(qmoe_layer_desc), i32, i32, i32,
                                                ctypes.POINTER(qmoe_layer_ws_view)]),
        "qmoe_route": (ctypes.c_int, [vp, i32, i32, i32, vp, vp, vp]),
        "qmoe_import_twos": (ctypes.c_int, [vp, i64, i64, vp, vp]),
        "qmoe_detect_group": (i32, [i64, i64, i64]),
        "qmoe_cache_create": (ctypes.c_int, [ctypes.POINTER(qmoe_layer_desc),
                                             ctypes.POINTER(qmoe_layer_desc),
                                             ctypes.POINTER(ctypes.c_void_p)]),
        "qmoe_cache_destroy": (None, [vp]),
        "qmoe_cache_prepare": (ctypes.c_int, [vp, vp, i32, i32, vp, ctypes.POINTER(i64), vp]),
        "qmoe_cache_resident": (i32, [vp, i32]),
        "qmoe_cache_device_state_bytes": (sz, [i32, i32]),
        "qmoe_cache_device_init": (ctypes.c_int, [vp, vp, sz, vp]),
        "qmoe_cache_prepare_device": (ctypes.c_int, [vp, vp, sz, vp, i32, i32, vp, vp]),
        "qmoe_layer_logits_workspace_bytes": (sz, [ctypes.POINTER(qmoe_layer_desc), i32, i32, i32]),
        "qmoe_layer_logits": (ctypes.c_int, [ctypes.POINTER(qmoe_layer_desc), i32, vp, i32, vp, i32,
                                             vp, vp, sz, vp]),
        "qmoe_layer_noalloc": (ctypes.c_int, [ctypes.POINTER(qmoe_layer_desc), i32, vp, i32, vp,
                                              vp, i32, vp, vp]),
        "qmoe_prefill_pass_rows": (i32, []),
        "qmoe_stream_probe": (ctypes.c_int, [vp, i64, i32, vp, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    v = lib.qmoe_abi_version()
    if v != ABI_VERSION:
        raise ImportError(f"libqmoe.so ABI {v}, binding expects {ABI_VERSION}")
    if path is None:
        _lib = lib
    return lib


def _lib_status_str(status):
    try:
        return load().qmoe_status_str(int(status)).decode()
    except Exception:  # pragma: no cover
        return "?"


def _check(status, what):
    if status != QMOE_OK:
        raise QmoeError(status, what)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _dev(t, name, dtype=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


# ------------------------------------------------------------------ sizes ---

def qmoe_abi_version() -> int:
    return int(load().qmoe_abi_version())


QMOE_PROBE_LINEAR, QMOE_PROBE_ROWS, QMOE_PROBE_SINK = 0, 1, 2048


def qmoe_stream_probe(buf, pattern=QMOE_PROBE_LINEAR, sink=None, stream=None):
    """Read `buf` (a device tensor) once with the probe's load shape; returns
    the uint32 sink (per-block dword sums, as int32 storage)."""
    _dev(buf, "buf")
    s = sink if sink is not None else torch.empty(QMOE_PROBE_SINK, dtype=torch.int32,
                                                  device=buf.device)
    _check(load().qmoe_stream_probe(_ptr(buf), buf.numel() * buf.element_size(), pattern,
                                    _ptr(s), _stream(stream)), "qmoe_stream_probe")
    return s


def qmoe_prefill_pass_rows() -> int:
    """Experts with at most this many pairs take the bf16 prefill passes."""
    return int(load().qmoe_prefill_pass_rows())


def qmoe_status_str(status: int) -> str:
    return load().qmoe_status_str(int(status)).decode()


def qmoe_packed_bytes(rows: int, cols: int) -> int:
    return int(load().qmoe_packed_bytes(rows, cols))


def qmoe_scale_count(rows: int, cols: int, group: int = 64) -> int:
    return int(load().qmoe_scale_count(rows, cols, group))


# ----------------------------------------------------------------- format ---

def qmoe_pack(q: torch.Tensor, out: torch.Tensor | None = None, count_bad: bool = False,
              stream=None):
    """int8 codes [..., rows, cols] -> packed uint8 [..., rows, ceil(cols/2)].
    Returns packed (and the device count of out-of-range codes if asked)."""
    _dev(q, "q", torch.int8)
    cols = q.shape[-1]
    rows = q.numel() // cols if cols else 0
    if out is None:
        out = torch.empty(*q.shape[:-1], (cols + 1) // 2, dtype=torch.uint8, device=q.device)
    nbad = torch.empty(4, dtype=torch.int32, device=q.device) if count_bad else None
    _check(load().qmoe_pack(_ptr(q), rows, cols, _ptr(out), _ptr(nbad), _stream(stream)),
           "qmoe_pack")
    return (out, nbad[:1]) if count_bad else out


def qmoe_unpack(packed: torch.Tensor, cols: int, stream=None):
    _dev(packed, "packed", torch.uint8)
    rows = packed.numel() // packed.shape[-1] if packed.numel() else 0
    out = torch.empty(*packed.shape[:-1], cols, dtype=torch.int8, device=packed.device)
    _check(load().qmoe_unpack(_ptr(packed), rows, cols, _ptr(out), _stream(stream)),
           "qmoe_unpack")
    return out


# ------------------------------------------------------------ descriptors ---

def make_qmat(q: torch.Tensor, s: torch.Tensor, cols: int, group: int = 64) -> qmoe_qmat:
    """Descriptor of packed codes q [E?, rows, ceil(cols/2)] and scales
    s [E?, rows, ceil(cols/group)]."""
    rows = q.shape[-2]
    m = qmoe_qmat()
    m.struct_size = ctypes.sizeof(qmoe_qmat)
    m.rows, m.cols, m.group = rows, cols, group
    m.q = q.data_ptr()
    m.s = s.data_ptr()
    m.q_expert_stride = q.stride(0) if q.dim() == 3 else 0
    m.s_expert_stride = s.stride(0) if s.dim() == 3 else 0
    return m


class QLayer:
    """Stacked grouped-int4 weights of one MoE layer resident on the device.

    gate/up packed [E, F, H/2] + scales [E, F, ceil(H/group)]; down packed
    [E, H, F/2] + scales [E, H, ceil(F/group)]."""

    def __init__(self, pg, sg, pu, su, pd, sd, hidden, inter, group=64):
        self.tensors = [pg, sg, pu, su, pd, sd]
        for t, n in zip(self.tensors, ("pg", "sg", "pu", "su", "pd", "sd")):
            _dev(t, n)
        self.experts = pg.shape[0]
        self.hidden, self.inter, self.group = hidden, inter, group
        d = qmoe_layer_desc()
        d.struct_size = ctypes.sizeof(qmoe_layer_desc)
        d.experts, d.hidden, d.inter, d.group = self.experts, hidden, inter, group
        d.gate = make_qmat(pg, sg, hidden, group)
        d.up = make_qmat(pu, su, hidden, group)
        d.down = make_qmat(pd, sd, inter, group)
        self.desc = d

    def workspace_bytes(self, tokens, k, x_dtype):
        return int(load().qmoe_layer_workspace_bytes(ctypes.byref(self.desc), tokens, k,
                                                     x_dtype))

    def ws_view(self, tokens, k, x_dtype):
        v = qmoe_layer_ws_view()
        v.struct_size = ctypes.sizeof(qmoe_layer_ws_view)
        _check(load().qmoe_layer_ws_layout(ctypes.byref(self.desc), tokens, k, x_dtype,
                                           ctypes.byref(v)), "qmoe_layer_ws_layout")
        return v


class HostLayer:
    """Stacked weights of one MoE layer in host memory (pinned CPU tensors:
    gate/up packed [E, F, H/2] + scales, down packed [E, H, F/2] + scales),
    the backing store of an ExpertCache."""

    def __init__(self, pg, sg, pu, su, pd, sd, hidden, inter, group=64):
        self.tensors = [pg, sg, pu, su, pd, sd]
        for t, n in zip(self.tensors, ("pg", "sg", "pu", "su", "pd", "sd")):
            if not isinstance(t, torch.Tensor) or t.is_cuda or not t.is_contiguous():
                raise TypeError(f"{n} must be a contiguous CPU tensor (pinned for async copies)")
        self.experts = pg.shape[0]
        self.hidden, self.inter, self.group = hidden, inter, group
        d = qmoe_layer_desc()
        d.struct_size = ctypes.sizeof(qmoe_layer_desc)
        d.experts, d.hidden, d.inter, d.group = self.experts, hidden, inter, group
        d.gate = make_qmat(pg, sg, hidden, group)
        d.up = make_qmat(pu, su, hidden, group)
        d.down = make_qmat(pd, sd, inter, group)
        self.desc = d


class ExpertCache:
    """S expert slots in HBM (a device QLayer with S experts) in front of a
    HostLayer; prepare() copies the routed experts that are missing."""

    def __init__(self, host: HostLayer, slots: QLayer):
        self.host, self.slots = host, slots
        h = ctypes.c_void_p()
        _check(load().qmoe_cache_create(ctypes.byref(host.desc), ctypes.byref(slots.desc),
                                        ctypes.byref(h)), "qmoe_cache_create")
        self.handle = h
        self._lib = load()

    def prepare(self, host_ids, slot_ids=None, stream=None):
        """host_ids int32 CPU [T, k] -> (slot_ids int32 CPU [T, k], bytes copied)."""
        if host_ids.is_cuda or host_ids.dtype != torch.int32 or not host_ids.is_contiguous():
            raise TypeError("host_ids must be a contiguous int32 CPU tensor")
        T, k = host_ids.shape
        out = slot_ids if slot_ids is not None else torch.empty(T, k, dtype=torch.int32)
        nb = ctypes.c_int64(0)
        _check(self._lib.qmoe_cache_prepare(self.handle, _ptr(host_ids), T, k, _ptr(out),
                                            ctypes.byref(nb), _stream(stream)),
               "qmoe_cache_prepare")
        return out, nb.value

    def resident(self, expert):
        return int(self._lib.qmoe_cache_resident(self.handle, expert))

    def device_state(self, stream=None):
        """A fresh device state for prepare_device (int32 device tensor),
        initialised on `stream` to an empty cache."""
        nb = int(self._lib.qmoe_cache_device_state_bytes(self.host.experts,
                                                         self.slots.desc.experts))
        st = torch.empty(nb // 4, dtype=torch.int32, device=self.slots.tensors[0].device)
        _check(self._lib.qmoe_cache_device_init(self.handle, _ptr(st), nb, _stream(stream)),
               "qmoe_cache_device_init")
        return st

    def prepare_device(self, state, dev_ids, slot_ids=None, stream=None):
        """dev_ids int32 device [T, k] -> slot_ids int32 device [T, k]; the
        missing experts are chosen and copied on the device (no host sync)."""
        _dev(dev_ids, "dev_ids", torch.int32)
        T, k = dev_ids.shape
        out = slot_ids if slot_ids is not None else torch.empty(T, k, dtype=torch.int32,
                                                                device=dev_ids.device)
        _check(self._lib.qmoe_cache_prepare_device(self.handle, _ptr(state), state.numel() * 4,
                                                   _ptr(dev_ids), T, k, _ptr(out),
                                                   _stream(stream)),
               "qmoe_cache_prepare_device")
        return out

    def close(self):
        if self.handle:
            self._lib.qmoe_cache_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # pragma: no cover
            pass


def _dtype_code(x, x_dtype=None):
    """Path code from x's dtype: float32 -> QMOE_F32 (f32 arithmetic), bfloat16
    -> QMOE_BF16.  x_dtype=QMOE_F32_DIGITS selects the digit variant of the
    f32 path (x still float32)."""
    if x_dtype is not None:
        want = torch.bfloat16 if x_dtype == QMOE_BF16 else torch.float32
        if x.dtype != want:
            raise TypeError(f"x_dtype {x_dtype} needs x of {want}, got {x.dtype}")
        return int(x_dtype)
    if x.dtype == torch.float32:
        return QMOE_F32
    if x.dtype == torch.bfloat16:
        return QMOE_BF16
    raise TypeError("x must be float32 (decode path) or bfloat16 (prefill path)")


def _workspace(nbytes, device, ws, stream=None):
    """The caller's workspace, or a new one.  A new one is allocated by
    torch's caching allocator; when the call runs on a stream other than the
    current one, the block is marked as used by that stream so that it is not
    handed out again before the call's kernels have finished with it."""
    if ws is not None:
        if ws.numel() < nbytes:
            raise ValueError(f"workspace of {ws.numel()} bytes < {nbytes}")
        return ws
    t = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)
    if stream is not None:
        st = stream if isinstance(stream, torch.cuda.Stream) else \
            torch.cuda.ExternalStream(int(stream), device=device)
        if st != torch.cuda.current_stream(device):
            t.record_stream(st)
    return t


# ------------------------------------------------------------------ calls ---

def qmoe_matvec(pq, s, cols, x, group=64, out=None, ws=None, stream=None):
    """y = W x; W packed [rows, ceil(cols/2)] + scales [rows, ceil(cols/group)];
    x f32 [B, cols].  Any cols (a partial last group is re-laid on the device)."""
    _dev(x, "x", torch.float32)
    W = make_qmat(pq, s, cols, group)
    batch = x.shape[0] if x.dim() == 2 else 1
    y = out if out is not None else torch.empty(batch, W.rows, dtype=torch.float32,
                                                device=x.device)
    nb = int(load().qmoe_matvec_workspace_bytes(ctypes.byref(W), batch))
    ws = _workspace(nb, x.device, ws, stream)
    _check(load().qmoe_matvec(ctypes.byref(W), _ptr(x), batch, _ptr(y), _ptr(ws), ws.numel(),
                              _stream(stream)), "qmoe_matvec")
    return y


def qmoe_expert_ffn(pg, sg, pu, su, pd, sd, hidden, inter, x, group=64, out=None, ws=None,
                    stream=None, x_dtype=None):
    """out = down(silu(gate x) * (up x)) for one expert; x f32 or bf16 [B, H]."""
    _dev(x, "x")
    code = _dtype_code(x, x_dtype)
    G = make_qmat(pg, sg, hidden, group)
    U = make_qmat(pu, su, hidden, group)
    D = make_qmat(pd, sd, inter, group)
    batch = x.shape[0]
    o = out if out is not None else torch.empty(batch, hidden, dtype=torch.float32,
                                                device=x.device)
    nb = int(load().qmoe_expert_ffn_workspace_bytes(ctypes.byref(G), ctypes.byref(U),
                                                    ctypes.byref(D), code, batch))
    ws = _workspace(nb, x.device, ws, stream)
    _check(load().qmoe_expert_ffn(ctypes.byref(G), ctypes.byref(U), ctypes.byref(D), code,
                                  _ptr(x), batch, _ptr(o), _ptr(ws), ws.numel(),
                                  _stream(stream)), "qmoe_expert_ffn")
    return o


def qmoe_worklist(topk_ids, experts, ws=None, stream=None):
    """Device worklist for int32 ids [T, k]; returns a dict of device tensors."""
    _dev(topk_ids, "topk_ids", torch.int32)
    T, k = topk_ids.shape
    n = T * k
    dev = topk_ids.device
    out = dict(counts=torch.empty(experts, dtype=torch.int32, device=dev),
               offsets=torch.empty(experts + 1, dtype=torch.int32, device=dev),
               pairs=torch.empty(max(n, 1), dtype=torch.int32, device=dev),
               inv=torch.empty(max(n, 1), dtype=torch.int32, device=dev),
               n_invalid=torch.empty(1, dtype=torch.int32, device=dev))
    nb = int(load().qmoe_worklist_workspace_bytes(T, k, experts))
    ws = _workspace(nb, dev, ws, stream)
    _check(load().qmoe_worklist(_ptr(topk_ids), T, k, experts, _ptr(out["counts"]),
                                _ptr(out["offsets"]), _ptr(out["pairs"]), _ptr(out["inv"]),
                                _ptr(out["n_invalid"]), _ptr(ws), ws.numel(),
                                _stream(stream)), "qmoe_worklist")
    out["pairs"] = out["pairs"][:n]
    out["inv"] = out["inv"][:n]
    return out


def qmoe_import_twos(twos, cols, out=None, stream=None):
    """Two's-complement nibble container (uint8 [rows, ceil(cols/2)]) ->
    offset container (what qmoe_pack writes); out may be twos itself."""
    _dev(twos, "twos", torch.uint8)
    rows = twos.shape[0]
    out = out if out is not None else torch.empty_like(twos)
    _check(load().qmoe_import_twos(_ptr(twos), rows, cols, _ptr(out), _stream(stream)),
           "qmoe_import_twos")
    return out


def qmoe_detect_group(rows: int, cols: int, scale_bytes: int) -> int:
    """Group size from a scale array's byte count (0: no candidate fits)."""
    return int(load().qmoe_detect_group(rows, cols, scale_bytes))


def qmoe_route(logits, k, ids=None, w=None, stream=None):
    """Device router: top-k ids (pick order) and softmax weights over the
    picked logits, for f32 logits [T, E]."""
    _dev(logits, "logits", torch.float32)
    T, E = logits.shape
    dev = logits.device
    ids = ids if ids is not None else torch.empty(T, k, dtype=torch.int32, device=dev)
    w = w if w is not None else torch.empty(T, k, dtype=torch.float32, device=dev)
    _check(load().qmoe_route(_ptr(logits), T, E, k, _ptr(ids), _ptr(w), _stream(stream)),
           "qmoe_route")
    return ids, w


def qmoe_layer(layer: QLayer, x, topk_ids, topk_w, out=None, ws=None, stream=None,
               x_dtype=None):
    """Routed MoE layer: out[t] = sum_j w[t,j] * ffn_{ids[t,j]}(x_t)."""
    _dev(x, "x")
    _dev(topk_ids, "topk_ids", torch.int32)
    _dev(topk_w, "topk_w", torch.float32)
    code = _dtype_code(x, x_dtype)
    T, k = topk_ids.shape
    o = out if out is not None else torch.empty(T, layer.hidden, dtype=torch.float32,
                                                device=x.device)
    nb = layer.workspace_bytes(T, k, code)
    ws = _workspace(nb, x.device, ws, stream)
    _check(load().qmoe_layer(ctypes.byref(layer.desc), code, _ptr(x), T, _ptr(topk_ids),
                             _ptr(topk_w), k, _ptr(o), _ptr(ws), ws.numel(), _stream(stream)),
           "qmoe_layer")
    return o


def qmoe_layer_noalloc(layer: QLayer, x, topk_ids, topk_w, out=None, stream=None,
                       x_dtype=None):
    """qmoe_layer without a workspace argument: the library's fixed device
    scratch (NOALLOC_SCRATCH_BYTES per GPU) serves as the workspace, so the
    call allocates nothing beyond `out` (pass `out` to allocate nothing)."""
    _dev(x, "x")
    _dev(topk_ids, "topk_ids", torch.int32)
    _dev(topk_w, "topk_w", torch.float32)
    code = _dtype_code(x, x_dtype)
    T, k = topk_ids.shape
    o = out if out is not None else torch.empty(T, layer.hidden, dtype=torch.float32,
                                                device=x.device)
    _check(load().qmoe_layer_noalloc(ctypes.byref(layer.desc), code, _ptr(x), T,
                                     _ptr(topk_ids), _ptr(topk_w), k, _ptr(o),
                                     _stream(stream)), "qmoe_layer_noalloc")
    return o


def qmoe_layer_logits(layer: QLayer, x, logits, k, out=None, ws=None, stream=None,
                      x_dtype=None):
    """Router + layer in one call: route f32 logits [T, E] on the device, then
    out[t] = sum_j w[t,j] * ffn_{ids[t,j]}(x_t)."""
    _dev(x, "x")
    _dev(logits, "logits", torch.float32)
    code = _dtype_code(x, x_dtype)
    T = x.shape[0]
    o = out if out is not None else torch.empty(T, layer.hidden, dtype=torch.float32,
                                                device=x.device)
    nb = int(load().qmoe_layer_logits_workspace_bytes(ctypes.byref(layer.desc), T, k, code))
    ws = _workspace(nb, x.device, ws, stream)
    _check(load().qmoe_layer_logits(ctypes.byref(layer.desc), code, _ptr(x), T, _ptr(logits), k,
                                    _ptr(o), _ptr(ws), ws.numel(), _stream(stream)),
           "qmoe_layer_logits")
    return o


def qmoe_layer_ex(layer: QLayer, x, topk_ids, topk_w, events, out=None, ws=None,
                  stream=None, x_dtype=None):
    """qmoe_layer that records the given torch.cuda.Event objects between its
    phases (events[0] before the first kernel)."""
    _dev(x, "x")
    code = _dtype_code(x, x_dtype)
    T, k = topk_ids.shape
    o = out if out is not None else torch.empty(T, layer.hidden, dtype=torch.float32,
                                                device=x.device)
    nb = layer.workspace_bytes(T, k, code)
    ws = _workspace(nb, x.device, ws, stream)
    handles = (ctypes.c_void_p * len(events))(*[ctypes.c_void_p(ev.cuda_event)
                                                  for ev in events])
    _check(load().qmoe_layer_ex(ctypes.byref(layer.desc), code, _ptr(x), T, _ptr(topk_ids),
                                _ptr(topk_w), k, _ptr(o), _ptr(ws), ws.numel(),
                                _stream(stream), handles, len(events)), "qmoe_layer_ex")
    return o


def layer_worklist_from_ws(layer: QLayer, ws, tokens, k, x_dtype):
    """Views of the worklist a qmoe_layer call left in its workspace."""
    v = layer.ws_view(tokens, k, x_dtype)
    n = tokens * k
    b = ws

    def i32(off, cnt):
        return b[off:off + 4 * cnt].view(torch.int32)
    E = layer.experts
    return dict(counts=i32(v.counts, E), offsets=i32(v.offsets, E + 1), pairs=i32(v.pairs, n),
                inv=i32(v.inv, n), n_invalid=i32(v.n_invalid, 1))
