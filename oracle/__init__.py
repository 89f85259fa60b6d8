"""Reference (oracle) implementation of packed QSA decode -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports it, and this package imports nothing from
the product.

Contents
  * ``decode``      -- ctypes front end of ``qsa_oracle.c`` (double precision,
                       two-pass softmax, list order, duplicates kept).
  * ``dequant_row`` -- one pool row dequantized to float64.
  * ``fp8_e4m3fn_to_double`` -- decode of one e4m3fn byte from the format's
                       definition.
  * ``quant``       -- the write-side quantizers (int8 / int4 / fp8) following
                       the rules of the page "feat(qsa): quantized KV pools
                       with dequant-on-gather (fp8/int8/int4)".
  * ``layout``      -- bytes per token of each pool layout.

Each function cites the passage it follows; the pins that tie it to the pages
and to mathematics live in ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from . import layout, quant  # noqa: F401  (re-exported)

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qsa_oracle.c")
_SRC_INDEX = os.path.join(_HERE, "qsa_index_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

FMT_BF16, FMT_FP8, FMT_INT8, FMT_INT4 = 0, 1, 2, 3
FMT_BY_NAME = {"bf16": FMT_BF16, "fp8": FMT_FP8, "int8": FMT_INT8, "int4": FMT_INT4}
CAPACITY = 2055
HEAD_DIM = 256
GQA = 12
ERRORS = {1: "bad arguments", 2: "bad cu_seqlens", 3: "row longer than 2055",
          4: "slot index out of range", 5: "context length out of range",
          6: "block table entry out of range"}


def build(sanitize: bool = False) -> str:
    """Compile qsa_oracle.c and qsa_index_oracle.c with gcc (-O2, no
    fast-math, no floating-point contraction, OpenMP) into liboracle.so.
    With sanitize=True compile them instead into one object file with
    AddressSanitizer and UndefinedBehaviorSanitizer (for a checking driver
    to link) and return its path."""
    if sanitize:
        out_dir = os.path.join(os.path.dirname(_HERE), "_build", "sanitize")
        os.makedirs(out_dir, exist_ok=True)
        obj = os.path.join(out_dir, "oracle_asan.o")
        cmd = ["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
               "-fno-sanitize-recover=undefined", "-fopenmp", "-std=c11", "-ffp-contract=off",
               "-r", "-nostdlib", "-o", obj, _SRC, _SRC_INDEX]
        subprocess.run(cmd, check=True)
        return obj
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c11", "-ffp-contract=off",
           "-o", _LIB + ".tmp", _SRC, _SRC_INDEX, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        lib.oracle_qsa_decode.restype = ctypes.c_int
        lib.oracle_qsa_decode.argtypes = [
            ctypes.c_int, ctypes.c_int, ctypes.c_int, P, ctypes.c_int,
            ctypes.c_int, ctypes.c_int64, P, P, P, P, P, ctypes.c_int64, P,
            ctypes.c_double, P, P, ctypes.c_int]
        lib.oracle_qsa_decode_tiered.restype = ctypes.c_int
        lib.oracle_qsa_decode_tiered.argtypes = [
            ctypes.c_int, ctypes.c_int, ctypes.c_int, P, ctypes.c_int64, P, P, P, P, P,
            ctypes.c_int64, P, P, P, P, P, ctypes.c_int64, P, ctypes.c_double, P, P,
            ctypes.c_int]
        lib.oracle_dequant_row.restype = None
        lib.oracle_dequant_row.argtypes = [
            ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P, ctypes.c_int64,
            ctypes.c_int, P]
        lib.oracle_fp8_e4m3fn_to_double.restype = ctypes.c_double
        lib.oracle_fp8_e4m3fn_to_double.argtypes = [ctypes.c_uint8]
        lib.oracle_qsa_index.restype = ctypes.c_int
        lib.oracle_qsa_index.argtypes = [
            ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P, P, ctypes.c_int64, P, ctypes.c_int,
            P, ctypes.c_int, P, ctypes.c_int, ctypes.c_int, P, P, P]
        lib.oracle_threads_used.restype = ctypes.c_int
        lib.oracle_threads_used.argtypes = [ctypes.c_int]
        _lib = lib
    return _lib


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _as_u16(x) -> np.ndarray:
    """bf16 data (torch bf16 tensor or uint16 array of bf16 bits) -> uint16."""
    if isinstance(x, np.ndarray):
        assert x.dtype == np.uint16
        return np.ascontiguousarray(x)
    import torch
    assert x.dtype == torch.bfloat16
    return np.ascontiguousarray(x.contiguous().view(torch.int16).numpy().view(np.uint16))


def _as_bytes(x) -> np.ndarray:
    if isinstance(x, np.ndarray):
        return np.ascontiguousarray(x).view(np.uint8)
    import torch
    t = x.contiguous()
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    elif t.dtype != torch.uint8 and t.dtype != torch.int8:
        t = t.view(torch.uint8)
    return np.ascontiguousarray(t.numpy()).view(np.uint8)


def _as_f32(x) -> np.ndarray | None:
    if x is None:
        return None
    if not isinstance(x, np.ndarray):
        x = x.contiguous().float().numpy()
    return np.ascontiguousarray(x, dtype=np.float32)


def decode(q, k_pool, v_pool, sel, cu, *, fmt: str = "bf16", group: int = 256,
           k_scale=None, v_scale=None, sm_scale: float = 1.0 / 16.0,
           nthreads: int = 1):
    """Packed QSA decode on the CPU, in float64.

    Follows the page "fix(qsa): restore SM121 correctness with Humanize and
    Kernel Design Agent", section "Changes" (the packed one-query decode
    contract), computed as plain two-pass softmax attention.

    q        [bs, hq, 256] bf16 (torch tensor or uint16 bits)
    k_pool   [slots, hkv, 256] bf16 / [slots, hkv, 256] uint8 codes (fp8,
             int8) / [slots, hkv, 128] uint8 (int4, two per byte)
    k_scale  [slots, hkv, 256 // group] float32 (quantized formats only)
    sel      [n_sel] int32 slot ids;  cu [bs + 1] int32
    Returns (out [bs, hq, 256] float64, lse [bs, hq] float64).
    """
    lib = _load()
    qb = _as_u16(q)
    bs, hq, d = qb.shape
    assert d == HEAD_DIM
    kb, vb = _as_bytes(k_pool), _as_bytes(v_pool)
    slots, hkv = kb.shape[0], kb.shape[1]
    sel_np = np.ascontiguousarray(np.asarray(sel, dtype=np.int32))
    cu_np = np.ascontiguousarray(np.asarray(cu, dtype=np.int32))
    assert cu_np.shape == (bs + 1,)
    ks, vs = _as_f32(k_scale), _as_f32(v_scale)
    out = np.empty((bs, hq, HEAD_DIM), dtype=np.float64)
    lse = np.empty((bs, hq), dtype=np.float64)
    rc = lib.oracle_qsa_decode(
        bs, hq, hkv, _ptr(qb), FMT_BY_NAME[fmt], group, slots, _ptr(kb),
        _ptr(vb), _ptr(ks), _ptr(vs), _ptr(sel_np), sel_np.size, _ptr(cu_np),
        sm_scale, _ptr(out), _ptr(lse), nthreads)
    if rc != 0:
        raise ValueError(f"oracle rejected the call: {ERRORS.get(rc, rc)}")
    return out, lse


def decode_tiered(q, owner, ring_k, ring_v, ring_k_scale, ring_v_scale, cold_k, cold_v,
                  cold_k_scale, cold_v_scale, sel, cu, *, sm_scale: float = 1.0 / 16.0,
                  nthreads: int = 1):
    """Packed QSA decode over a tiered pool, in float64.

    Follows the page "feat(qsa): quantized KV pools with dequant-on-gather
    (fp8/int8/int4)", part 4 "Modifications", tiered pool bullet: listed
    slot s reads ring row r = s & (R - 1) (int8 codes, one scale per 64
    channels) when owner[r] == s, else its int4 row (one scale per 32
    channels).

    owner [R] int32 (R a power of two); ring_k / ring_v [R, hkv, 256] int8;
    ring scales [R, hkv, 4]; cold_k / cold_v [slots, hkv, 128] uint8 (two
    int4 codes per byte); cold scales [slots, hkv, 8]; scales as float32 or
    float16 (their values are used).  Returns (out, lse) like decode().
    """
    lib = _load()
    qb = _as_u16(q)
    bs, hq, d = qb.shape
    assert d == HEAD_DIM
    own = np.ascontiguousarray(np.asarray(owner, dtype=np.int32))
    rk, rv = _as_bytes(ring_k), _as_bytes(ring_v)
    ck, cv = _as_bytes(cold_k), _as_bytes(cold_v)
    ring_rows, hkv = rk.shape[0], rk.shape[1]
    slots = ck.shape[0]
    rks, rvs = _as_f32(ring_k_scale), _as_f32(ring_v_scale)
    cks, cvs = _as_f32(cold_k_scale), _as_f32(cold_v_scale)
    assert own.shape == (ring_rows,) and rks.shape == (ring_rows, hkv, 4)
    assert ck.shape == (slots, hkv, 128) and cks.shape == (slots, hkv, 8)
    sel_np = np.ascontiguousarray(np.asarray(sel, dtype=np.int32))
    cu_np = np.ascontiguousarray(np.asarray(cu, dtype=np.int32))
    out = np.empty((bs, hq, HEAD_DIM), dtype=np.float64)
    lse = np.empty((bs, hq), dtype=np.float64)
    rc = lib.oracle_qsa_decode_tiered(
        bs, hq, hkv, _ptr(qb), ring_rows, _ptr(own), _ptr(rk), _ptr(rv), _ptr(rks), _ptr(rvs),
        slots, _ptr(ck), _ptr(cv), _ptr(cks), _ptr(cvs), _ptr(sel_np), sel_np.size,
        _ptr(cu_np), sm_scale, _ptr(out), _ptr(lse), nthreads)
    if rc != 0:
        raise ValueError(f"oracle rejected the call: {ERRORS.get(rc, rc)}")
    return out, lse


def index(q, k_pool, block_table, req_to_token, ctx_len, *, budget: int, compress_ratio: int,
          weights=None, return_scores: bool = False):
    """The QSA indexer step (MQA block scores, exact top-k, expansion to
    KV slots) as read in qsa_index_oracle.c.

    q [bs, hi, di] bf16 (index query heads); k_pool [n, di] bf16 (one
    compressed index key per block row); block_table [bs, max_blocks] int32;
    req_to_token [bs, max_tokens] int32; ctx_len [bs] int32; weights
    [bs, hi] float32 or None (all 1).  Returns (sel int32 packed, cu
    [bs + 1] int32) and, with return_scores, the [bs, max_blocks] float32
    block scores (NaN past each row's blocks)."""
    lib = _load()
    qb = _as_u16(q)
    bs, hi, di = qb.shape
    kb = _as_u16(k_pool)
    assert kb.ndim == 2 and kb.shape[1] == di
    bt = np.ascontiguousarray(np.asarray(block_table, dtype=np.int32))
    r2t = np.ascontiguousarray(np.asarray(req_to_token, dtype=np.int32))
    cl = np.ascontiguousarray(np.asarray(ctx_len, dtype=np.int32))
    assert bt.shape[0] == bs and r2t.shape[0] == bs and cl.shape == (bs,)
    w = None if weights is None else _as_f32(weights)
    if w is not None:
        assert w.shape == (bs, hi)
    c = int(compress_ratio)
    sel = np.empty(bs * (budget + c - 1) + 1, dtype=np.int32)
    cu = np.empty(bs + 1, dtype=np.int32)
    scores = np.full((bs, bt.shape[1]), np.nan, dtype=np.float32)
    rc = lib.oracle_qsa_index(bs, hi, di, _ptr(qb), _ptr(w), _ptr(kb), kb.shape[0], _ptr(bt),
                              bt.shape[1], _ptr(r2t), r2t.shape[1], _ptr(cl), int(budget), c,
                              _ptr(sel), _ptr(cu), _ptr(scores))
    if rc != 0:
        raise ValueError(f"oracle rejected the call: {ERRORS.get(rc, rc)}")
    out = (sel[: cu[-1]].copy(), cu)
    return out + (scores,) if return_scores else out


def dequant_row(pool, scale, slot: int, g: int, *, fmt: str, group: int = 256):
    """One (slot, kv-head) row of a pool dequantized to float64 [256]."""
    lib = _load()
    pb = _as_bytes(pool)
    hkv = pb.shape[1]
    sc = _as_f32(scale)
    out = np.empty(HEAD_DIM, dtype=np.float64)
    lib.oracle_dequant_row(FMT_BY_NAME[fmt], group, hkv, _ptr(pb), _ptr(sc),
                           slot, g, _ptr(out))
    return out


def fp8_e4m3fn_to_double(code: int) -> float:
    """Value of one OCP e4m3fn byte (sign, 4-bit exponent bias 7, 3-bit
    mantissa, subnormals at exponent 0, NaN only at S.1111.111)."""
    return _load().oracle_fp8_e4m3fn_to_double(code)


def threads_used(nthreads: int) -> int:
    return _load().oracle_threads_used(nthreads)
