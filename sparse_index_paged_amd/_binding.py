"""ctypes marshalling for libqsa.so (see include/qsa.h for the contract)."""
from __future__ import annotations

import ctypes
import os
import struct

PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(PKG, "libqsa.so")

ABI_VERSION = 5

# qsa_dtype
BF16, F16, F32, I32, FP8_E4M3FN, I8, U4X2, I64 = 1, 2, 3, 4, 5, 6, 7, 8
STATUS = {0: "QSA_OK", 1: "QSA_ERR_CONTRACT", 2: "QSA_ERR_ARG", 3: "QSA_ERR_WORKSPACE",
          4: "QSA_ERR_HIP"}

EXPORTS = (
    "qsa_decode", "qsa_decode_noalloc", "qsa_kv_store", "qsa_decode_tiered", "qsa_kv_store_tiered", "qsa_index",
    "qsa_index_reserve", "qsa_workspace_reserve", "qsa_workspace_attach", "qsa_workspace_detach",
    "qsa_workspace_reset",
    "qsa_workspace_release", "qsa_workspace_bytes", "qsa_last_error", "qsa_plan", "qsa_set_option", "qsa_get_option",
    "qsa_debug_counters", "qsa_debug_read_counters", "qsa_debug_audit_counters",
    "qsa_debug_device_error", "qsa_abi_version",
)


class QsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status
        self.message = message


class QsaTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 4), ("stride", ctypes.c_int64 * 4)]


class QsaKvScales(ctypes.Structure):
    _fields_ = [("k_scale", QsaTensor), ("v_scale", QsaTensor), ("group_size", ctypes.c_int32)]


class QsaTieredPool(ctypes.Structure):
    _fields_ = [("ring_k", QsaTensor), ("ring_v", QsaTensor), ("ring_k_scale", QsaTensor),
                ("ring_v_scale", QsaTensor), ("owner", QsaTensor), ("claim", QsaTensor),
                ("cold_k", QsaTensor), ("cold_v", QsaTensor), ("cold_k_scale", QsaTensor),
                ("cold_v_scale", QsaTensor)]


TIERED_FIELDS = ("ring_k", "ring_v", "ring_k_scale", "ring_v_scale", "owner", "claim",
                 "cold_k", "cold_v", "cold_k_scale", "cold_v_scale")


_lib = None


def lib_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libqsa.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with "
                          "`python -m sparse_index_paged_amd.build` (hipcc, gfx950)")
    _lib = _configure(ctypes.CDLL(_LIB_PATH))
    return _lib


_stamps_lib = None


def load_stamps_library():
    """The measurement build libqsa_stamps.so (include/qsa_stamps.h): the
    same API with per-workgroup phase stamps in the decode kernel, loaded
    beside libqsa.so with its own library state."""
    global _stamps_lib
    if _stamps_lib is None:
        path = os.path.join(os.path.dirname(_LIB_PATH), "libqsa_stamps.so")
        if not os.path.exists(path):
            raise ImportError(f"{path} is missing: build it with `python -m sparse_index_paged_amd.build`")
        lib = _configure(ctypes.CDLL(path))
        lib.qsa_debug_set_phase_stamps.restype = ctypes.c_int
        lib.qsa_debug_set_phase_stamps.argtypes = [ctypes.c_void_p, ctypes.c_int64]
        _stamps_lib = lib
    return _stamps_lib


def _configure(lib):
    """Argument and result types of every qsa.h call."""
    P = ctypes.POINTER
    T = P(QsaTensor)
    lib.qsa_decode.restype = ctypes.c_int
    lib.qsa_decode.argtypes = [T, T, T, P(QsaKvScales), T, T, T, T, ctypes.c_void_p]
    lib.qsa_decode_noalloc.restype = ctypes.c_int
    lib.qsa_decode_noalloc.argtypes = [T, T, T, P(QsaKvScales), T, T, T, T, ctypes.c_void_p]
    lib.qsa_kv_store.restype = ctypes.c_int
    lib.qsa_kv_store.argtypes = [T, T, T, T, T, P(QsaKvScales), ctypes.c_void_p]
    lib.qsa_decode_tiered.restype = ctypes.c_int
    lib.qsa_decode_tiered.argtypes = [T, P(QsaTieredPool), T, T, T, T, ctypes.c_void_p]
    lib.qsa_kv_store_tiered.restype = ctypes.c_int
    lib.qsa_kv_store_tiered.argtypes = [T, T, T, P(QsaTieredPool), ctypes.c_void_p]
    lib.qsa_index.restype = ctypes.c_int
    lib.qsa_index.argtypes = [T, T, T, T, T, T, ctypes.c_int, ctypes.c_int, T, T, ctypes.c_void_p]
    lib.qsa_index_reserve.restype = ctypes.c_int
    lib.qsa_index_reserve.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.qsa_workspace_reserve.restype = ctypes.c_int
    lib.qsa_workspace_reserve.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.qsa_workspace_attach.restype = ctypes.c_int
    lib.qsa_workspace_attach.argtypes = [ctypes.c_void_p]
    lib.qsa_workspace_detach.restype = ctypes.c_int
    lib.qsa_workspace_detach.argtypes = [ctypes.c_void_p]
    lib.qsa_workspace_reset.restype = ctypes.c_int
    lib.qsa_workspace_reset.argtypes = [ctypes.c_void_p]
    lib.qsa_workspace_release.restype = ctypes.c_int
    lib.qsa_workspace_release.argtypes = []
    lib.qsa_workspace_bytes.restype = ctypes.c_int64
    lib.qsa_workspace_bytes.argtypes = []
    lib.qsa_last_error.restype = ctypes.c_char_p
    lib.qsa_last_error.argtypes = []
    lib.qsa_plan.restype = ctypes.c_int
    lib.qsa_plan.argtypes = [ctypes.c_int, ctypes.c_int, P(ctypes.c_int), P(ctypes.c_int)]
    lib.qsa_set_option.restype = ctypes.c_int
    lib.qsa_set_option.argtypes = [ctypes.c_char_p, ctypes.c_int64]
    lib.qsa_get_option.restype = ctypes.c_int
    lib.qsa_get_option.argtypes = [ctypes.c_char_p, P(ctypes.c_int64)]
    lib.qsa_debug_counters.restype = ctypes.c_int
    lib.qsa_debug_counters.argtypes = [P(ctypes.c_void_p), P(ctypes.c_int), ctypes.c_void_p]
    lib.qsa_debug_read_counters.restype = ctypes.c_int
    lib.qsa_debug_read_counters.argtypes = [P(ctypes.c_uint32), ctypes.c_int, ctypes.c_void_p]
    lib.qsa_debug_audit_counters.restype = ctypes.c_int
    lib.qsa_debug_audit_counters.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    lib.qsa_debug_device_error.restype = ctypes.c_int
    lib.qsa_debug_device_error.argtypes = [P(ctypes.c_uint32), ctypes.c_void_p]
    lib.qsa_abi_version.restype = ctypes.c_int
    lib.qsa_abi_version.argtypes = []
    return lib


def _check(status: int):
    if status != 0:
        msg = load_library().qsa_last_error().decode()
        raise QsaError(status, msg)


_FORMAT_CODES = {"bf16": BF16, "fp8": FP8_E4M3FN, "int8": I8, "int4": U4X2}
_DTYPE_CODES = None
_TENSOR_LAYOUT = struct.Struct("<Qii4q4q")  # qsa_tensor: data, dtype, ndim, shape[4], stride[4]
_PAD = (0, 0, 0, 0)
assert _TENSOR_LAYOUT.size == ctypes.sizeof(QsaTensor)


def _dtype_codes() -> dict:
    global _DTYPE_CODES
    import torch
    m = {torch.bfloat16: BF16, torch.float16: F16, torch.float32: F32, torch.int32: I32,
         torch.int8: I8, torch.int64: I64}
    fp8 = getattr(torch, "float8_e4m3fn", None)
    if fp8 is not None:
        m[fp8] = FP8_E4M3FN
    _DTYPE_CODES = m
    return m


def describe(t, kv_format: str | None = None, dtype_code: int | None = None) -> QsaTensor:
    """qsa_tensor for a torch tensor (strides in elements).  A tensor without
    storage (data pointer 0, only possible when it is empty) gets a non-null
    placeholder pointer, which the library never dereferences."""
    shape = t.shape
    nd = len(shape)
    if nd > 4:
        raise ValueError("at most 4 dimensions")
    ptr = t.data_ptr() or 16
    if dtype_code is not None:
        code = dtype_code
    elif kv_format is not None:
        code = _FORMAT_CODES[kv_format]
    else:
        code = (_DTYPE_CODES or _dtype_codes()).get(t.dtype)
        if code is None:
            raise TypeError(f"no qsa dtype for {t.dtype}")
    pad = _PAD[nd:]
    return QsaTensor.from_buffer_copy(_TENSOR_LAYOUT.pack(ptr, code, nd, *shape, *pad, *t.stride(), *pad))


_RAW_STREAM = None


def _stream_handle(stream):
    """hipStream_t of `stream`, or of torch's current stream on the current
    device when None (read through torch's raw-stream accessor where it has
    one: about 0.4 us instead of 3 us for building a Stream object)."""
    global _RAW_STREAM
    import torch
    if stream is None:
        if _RAW_STREAM is None:
            raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
            _RAW_STREAM = (lambda: raw(torch.cuda.current_device())) if raw is not None else (
                lambda: torch.cuda.current_stream().cuda_stream)
        return ctypes.c_void_p(_RAW_STREAM())
    return ctypes.c_void_p(stream.cuda_stream)


def decode(q, k_pool, v_pool, sel, cu_seqlens, *, out=None, lse=None, kv_format: str = "bf16",
           k_scale=None, v_scale=None, group_size: int | None = None, stream=None,
           _noalloc: bool = False):
    """Packed QSA decode (one kernel launch on `stream`, default torch's
    current stream).  Returns (out [bs, Hq, 256] bf16, lse [bs, Hq] fp32).

    kv_format: "bf16" | "fp8" (e4m3fn bytes, torch.uint8 or float8_e4m3fn)
    | "int8" (torch.int8) | "int4" (torch.uint8 [slots, Hkv, 128]).
    Quantized formats take k_scale / v_scale [slots, Hkv, 256 // group_size]
    float32 or float16."""
    import torch
    lib = load_library()
    bs, hq = q.shape[0], q.shape[1]
    if out is None:
        out = torch.empty((bs, hq, 256), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((bs, hq), dtype=torch.float32, device=q.device)
    qd, od, ld = describe(q), describe(out), describe(lse)
    kd = describe(k_pool, kv_format)
    vd = describe(v_pool, kv_format)
    sd, cd = describe(sel), describe(cu_seqlens)
    scales = _scales(kv_format, k_scale, v_scale, group_size)
    entry = lib.qsa_decode_noalloc if _noalloc else lib.qsa_decode
    st = entry(ctypes.byref(qd), ctypes.byref(kd), ctypes.byref(vd),
               ctypes.byref(scales) if scales is not None else None,
               ctypes.byref(sd), ctypes.byref(cd), ctypes.byref(od), ctypes.byref(ld),
               _stream_handle(stream))
    _check(st)
    return out, lse


def decode_noalloc(q, k_pool, v_pool, sel, cu_seqlens, *, out, lse, kv_format: str = "bf16",
                   k_scale=None, v_scale=None, group_size: int | None = None, stream=None):
    """qsa_decode_noalloc: the same decode with the split scratch in the
    library's fixed per-device array (nothing is allocated, by the library
    or here: out and lse must be given)."""
    return decode(q, k_pool, v_pool, sel, cu_seqlens, out=out, lse=lse, kv_format=kv_format,
                  k_scale=k_scale, v_scale=v_scale, group_size=group_size, stream=stream,
                  _noalloc=True)


class KvPool:
    """A single-tier K/V pool (and its scales) whose descriptors are built
    once: decode / decode_noalloc / store through it skip rebuilding them on
    every call.  The tensors are held here, so they stay alive; they must
    not be reallocated or reshaped while the KvPool is in use."""

    def __init__(self, k_pool, v_pool, *, kv_format: str = "bf16", k_scale=None, v_scale=None,
                 group_size: int | None = None):
        self.k_pool, self.v_pool, self.k_scale, self.v_scale = k_pool, v_pool, k_scale, v_scale
        self.kv_format = kv_format
        self._kd = describe(k_pool, kv_format)
        self._vd = describe(v_pool, kv_format)
        self._scales = _scales(kv_format, k_scale, v_scale, group_size)
        self._held = [(k_pool, self._kd.data), (v_pool, self._vd.data)]
        if self._scales is not None:
            self._held += [(k_scale, self._scales.k_scale.data), (v_scale, self._scales.v_scale.data)]

    def check(self):
        """Raise if a held tensor no longer has the storage its descriptor
        names (reallocated by resize_ or set_): a stale descriptor would send
        the kernels to freed memory."""
        for t, ptr in self._held:
            if (t.data_ptr() or 16) != ptr:
                raise ValueError("KvPool: a pool tensor was reallocated; build a new KvPool")

    def decode(self, q, sel, cu_seqlens, *, out=None, lse=None, stream=None, noalloc: bool = False):
        """qsa_decode (qsa_decode_noalloc with noalloc=True, which needs out
        and lse) over this pool; returns (out, lse)."""
        import torch
        lib = load_library()
        if out is None or lse is None:
            if noalloc:
                raise ValueError("decode with noalloc=True needs out and lse")
            bs, hq = q.shape[0], q.shape[1]
            if out is None:
                out = torch.empty((bs, hq, 256), dtype=torch.bfloat16, device=q.device)
            if lse is None:
                lse = torch.empty((bs, hq), dtype=torch.float32, device=q.device)
        self.check()
        qd, od, ld = describe(q), describe(out), describe(lse)
        sd, cd = describe(sel), describe(cu_seqlens)
        entry = lib.qsa_decode_noalloc if noalloc else lib.qsa_decode
        _check(entry(ctypes.byref(qd), ctypes.byref(self._kd), ctypes.byref(self._vd),
                     ctypes.byref(self._scales) if self._scales is not None else None,
                     ctypes.byref(sd), ctypes.byref(cd), ctypes.byref(od), ctypes.byref(ld),
                     _stream_handle(stream)))
        return out, lse

    def store(self, k_new, v_new, loc, *, stream=None):
        """qsa_kv_store of k_new / v_new [n, Hkv, 256] bf16 into this pool."""
        lib = load_library()
        self.check()
        kd, vd, ld = describe(k_new), describe(v_new), describe(loc)
        _check(lib.qsa_kv_store(ctypes.byref(kd), ctypes.byref(vd), ctypes.byref(ld), ctypes.byref(self._kd),
                                ctypes.byref(self._vd),
                                ctypes.byref(self._scales) if self._scales is not None else None,
                                _stream_handle(stream)))


def _scales(kv_format, k_scale, v_scale, group_size):
    if kv_format == "bf16":
        return None
    if k_scale is None or v_scale is None:
        raise ValueError(f"{kv_format} pools need k_scale and v_scale")
    g = group_size if group_size is not None else 256 // k_scale.shape[-1]
    return QsaKvScales(describe(k_scale), describe(v_scale), g)


def kv_store(k_new, v_new, loc, k_pool, v_pool, *, kv_format: str = "bf16", k_scale=None,
             v_scale=None, group_size: int | None = None, stream=None):
    """Quantize k_new / v_new [n, Hkv, 256] bf16 and scatter row t to pool
    slot loc[t] (int32 or int64, distinct ids), writing codes and scales in
    place (one kernel launch on `stream`)."""
    lib = load_library()
    kd, vd, ld = describe(k_new), describe(v_new), describe(loc)
    kpd = describe(k_pool, kv_format)
    vpd = describe(v_pool, kv_format)
    scales = _scales(kv_format, k_scale, v_scale, group_size)
    st = lib.qsa_kv_store(ctypes.byref(kd), ctypes.byref(vd), ctypes.byref(ld), ctypes.byref(kpd),
                          ctypes.byref(vpd), ctypes.byref(scales) if scales is not None else None,
                          _stream_handle(stream))
    _check(st)


def tiered_pool(*, ring_k, ring_v, ring_k_scale, ring_v_scale, owner, claim, cold_k, cold_v,
                cold_k_scale, cold_v_scale) -> QsaTieredPool:
    """qsa_tiered_pool for torch tensors: ring_k / ring_v int8 [R, Hkv, 256],
    ring scales float16 [R, Hkv, 4], owner / claim int32 [R], cold_k /
    cold_v uint8 [slots, Hkv, 128] (two int4 codes per byte), cold scales
    float16 [slots, Hkv, 8]."""
    tp = QsaTieredPool()
    tp.ring_k, tp.ring_v = describe(ring_k), describe(ring_v)
    tp.ring_k_scale, tp.ring_v_scale = describe(ring_k_scale), describe(ring_v_scale)
    tp.owner, tp.claim = describe(owner), describe(claim)
    tp.cold_k, tp.cold_v = describe(cold_k, "int4"), describe(cold_v, "int4")
    tp.cold_k_scale, tp.cold_v_scale = describe(cold_k_scale), describe(cold_v_scale)
    return tp


class TieredPool:
    """A tiered pool's qsa_tiered_pool descriptor, built once from its
    tensors (held here, so they stay alive) and passed to decode_tiered /
    kv_store_tiered in place of the dict, which saves rebuilding the ten
    tensor descriptors on every call."""

    def __init__(self, pool: dict):
        self.tensors = {name: pool[name] for name in TIERED_FIELDS}
        self.desc = tiered_pool(**self.tensors)
        self._held = [(t, getattr(self.desc, name).data) for name, t in self.tensors.items()]

    def check(self):
        """Raise if a held tensor no longer has the storage its descriptor
        names (reallocated by resize_ or set_): a stale descriptor would send
        the kernels to freed memory."""
        for t, ptr in self._held:
            if (t.data_ptr() or 16) != ptr:
                raise ValueError("TieredPool: a pool tensor was reallocated; build a new TieredPool")


def _tiered_desc(pool) -> QsaTieredPool:
    if isinstance(pool, TieredPool):
        pool.check()
        return pool.desc
    return tiered_pool(**{name: pool[name] for name in TIERED_FIELDS})


def decode_tiered(q, pool, sel, cu_seqlens, *, out=None, lse=None, stream=None):
    """Packed QSA decode over a tiered pool (a dict with the qsa_tiered_pool
    fields as torch tensors, or a TieredPool).  One kernel launch; returns
    (out, lse)."""
    import torch
    lib = load_library()
    bs, hq = q.shape[0], q.shape[1]
    if out is None:
        out = torch.empty((bs, hq, 256), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((bs, hq), dtype=torch.float32, device=q.device)
    tp = _tiered_desc(pool)
    qd, od, ld = describe(q), describe(out), describe(lse)
    sd, cd = describe(sel), describe(cu_seqlens)
    _check(lib.qsa_decode_tiered(ctypes.byref(qd), ctypes.byref(tp), ctypes.byref(sd),
                                 ctypes.byref(cd), ctypes.byref(od), ctypes.byref(ld),
                                 _stream_handle(stream)))
    return out, lse


def kv_store_tiered(k_new, v_new, loc, pool, *, stream=None):
    """Write k_new / v_new [n, Hkv, 256] bf16 into a tiered pool (dict or
    TieredPool): int4 into slot loc[t], int8 into ring row loc[t] & (R-1)
    with its owner stamp (three kernel launches on `stream`)."""
    lib = load_library()
    tp = _tiered_desc(pool)
    kd, vd, ld = describe(k_new), describe(v_new), describe(loc)
    _check(lib.qsa_kv_store_tiered(ctypes.byref(kd), ctypes.byref(vd), ctypes.byref(ld),
                                   ctypes.byref(tp), _stream_handle(stream)))


def index(q_index, k_index_pool, block_table, req_to_token, context_lens, *, budget: int,
          compress_ratio: int, head_weights=None, sel_out=None, cu_out=None, stream=None):
    """The indexer step (two kernel launches on `stream`): per row, the
    top budget / compress_ratio blocks by MQA score, expanded to KV slots.
    Returns (sel [bs * (budget + compress_ratio - 1)] int32, whose first
    cu[-1] entries are the packed lists, cu [bs + 1] int32)."""
    import torch
    lib = load_library()
    bs = q_index.shape[0]
    dev = q_index.device
    if sel_out is None:
        sel_out = torch.empty(bs * (budget + compress_ratio - 1), dtype=torch.int32, device=dev)
    if cu_out is None:
        cu_out = torch.empty(bs + 1, dtype=torch.int32, device=dev)
    qd, kd = describe(q_index), describe(k_index_pool)
    wd = describe(head_weights) if head_weights is not None else None
    bd, rd, cd = describe(block_table), describe(req_to_token), describe(context_lens)
    sd, ud = describe(sel_out), describe(cu_out)
    _check(lib.qsa_index(ctypes.byref(qd), ctypes.byref(wd) if wd is not None else None,
                         ctypes.byref(kd), ctypes.byref(bd), ctypes.byref(rd), ctypes.byref(cd),
                         int(budget), int(compress_ratio), ctypes.byref(sd), ctypes.byref(ud),
                         _stream_handle(stream)))
    return sel_out, cu_out


def index_reserve(max_bs: int, max_blocks: int, stream=None):
    _check(load_library().qsa_index_reserve(max_bs, max_blocks, _stream_handle(stream)))


def workspace_reserve(max_bs: int, hq: int, hkv: int, stream=None):
    _check(load_library().qsa_workspace_reserve(max_bs, hq, hkv, _stream_handle(stream)))


def workspace_attach(stream=None):
    """Give `stream` (default: torch's current stream) a private workspace,
    so that its calls may run concurrently with calls on other streams."""
    _check(load_library().qsa_workspace_attach(_stream_handle(stream)))


def workspace_detach(stream=None):
    """Free the private workspace of `stream` (synchronises it); its later
    calls use the device's shared workspace."""
    _check(load_library().qsa_workspace_detach(_stream_handle(stream)))


def workspace_reset(stream=None):
    _check(load_library().qsa_workspace_reset(_stream_handle(stream)))


def workspace_release():
    _check(load_library().qsa_workspace_release())


def workspace_bytes() -> int:
    return int(load_library().qsa_workspace_bytes())


def plan(bs: int, hkv: int) -> tuple[int, int]:
    s, w = ctypes.c_int(), ctypes.c_int()
    _check(load_library().qsa_plan(bs, hkv, ctypes.byref(s), ctypes.byref(w)))
    return s.value, w.value


def set_option(name: str, value: int):
    _check(load_library().qsa_set_option(name.encode(), int(value)))


def get_option(name: str) -> int:
    v = ctypes.c_int64()
    _check(load_library().qsa_get_option(name.encode(), ctypes.byref(v)))
    return v.value


def debug_counters(stream=None) -> list[int]:
    """Current values of the split counters of the workspace `stream` uses
    (synchronises `stream`); they read zero between calls."""
    ptr, n = ctypes.c_void_p(), ctypes.c_int()
    lib = load_library()
    h = _stream_handle(stream)
    _check(lib.qsa_debug_counters(ctypes.byref(ptr), ctypes.byref(n), h))
    buf = (ctypes.c_uint32 * n.value)()
    _check(lib.qsa_debug_read_counters(buf, n.value, h))
    return list(buf)


def debug_counter_ptr(stream=None) -> tuple[int, int]:
    """(device address, count) of the split counters of the workspace
    `stream` uses."""
    ptr, n = ctypes.c_void_p(), ctypes.c_int()
    _check(load_library().qsa_debug_counters(ctypes.byref(ptr), ctypes.byref(n),
                                             _stream_handle(stream)))
    return int(ptr.value or 0), n.value


def debug_audit_counters(accum, stream=None):
    """Enqueue: accum[0] += sum(counters).  accum is a 1-element int32 /
    uint32 device tensor."""
    _check(load_library().qsa_debug_audit_counters(ctypes.c_void_p(accum.data_ptr()),
                                                   _stream_handle(stream)))


def debug_device_error(stream=None) -> int:
    w = ctypes.c_uint32()
    _check(load_library().qsa_debug_device_error(ctypes.byref(w), _stream_handle(stream)))
    return w.value


def abi_version() -> int:
    return int(load_library().qsa_abi_version())
