"""Write-side KV quantizers -- TEST INFRASTRUCTURE (part of the oracle).

They turn float K/V rows into the code + scale pools that the decode path
reads, following the page "feat(qsa): quantized KV pools with
dequant-on-gather (fp8/int8/int4)":

  * part 4, "Modifications", int8 pool bullet: signed 8-bit codes with one
    absmax/127 scale per (token, kv-head, channel group); the pages use
    64-channel groups with fp16 scales.
  * same section, int4 pool bullet: codes q in [-7, 7] stored offset-binary
    as q + 8, two per byte with the even channel in the low nibble, one
    absmax/7 scale per 32-channel group; rounding by ``rint`` (ties to even,
    named in the int4 unit-test bullet); fp16 scales are clamped to 65504
    (the write-kernel bullet of the same section).
  * part 4 also relies on the fp8 write path of part 2 (``memory_pool.py``
    bullet): values are saturated to +-448 before the cast to e4m3fn because
    the cast yields NaN beyond that range.

Readings where the pages are silent:
  * The measured configuration uses fp32 scales (per row for fp8 / int8,
    per 32 channels for int4); fp16 scales are supported as the pages' own
    storage.  Codes are computed from the stored (possibly fp16-rounded)
    scale, so dequantization reproduces what was quantized against.
  * fp8 gets a per-row scale absmax/448 so that the largest element lands on
    the top of the e4m3fn range.
  * An all-zero group gets scale 0 and all-zero codes (no NaN).

Arithmetic is float32 (numpy), the precision the pages' kernels use for the
division; the fp8 rounding itself is torch's float8_e4m3fn cast (a library
routine, round-to-nearest-even).
"""
from __future__ import annotations

import numpy as np

FP16_MAX = 65504.0
E4M3_MAX = 448.0


def _as_f32(x) -> np.ndarray:
    if isinstance(x, np.ndarray):
        return np.ascontiguousarray(x, dtype=np.float32)
    return np.ascontiguousarray(x.float().numpy(), dtype=np.float32)


def _group_absmax(x: np.ndarray, group: int) -> np.ndarray:
    *lead, d = x.shape
    assert d % group == 0
    return np.abs(x.reshape(*lead, d // group, group)).max(axis=-1)


def _store_scale(raw: np.ndarray, scale_dtype: str) -> np.ndarray:
    """Scale as stored (fp32 or fp16 with the 65504 clamp), returned as the
    float32 value the reader will use."""
    raw = raw.astype(np.float32)
    if scale_dtype == "f32":
        return raw
    if scale_dtype == "f16":
        return np.minimum(raw, np.float32(FP16_MAX)).astype(np.float16).astype(np.float32)
    raise ValueError(scale_dtype)


def _scaled(x: np.ndarray, scale: np.ndarray, group: int) -> np.ndarray:
    """x / scale per group in float32; a zero scale gives 0."""
    *lead, d = x.shape
    xg = x.reshape(*lead, d // group, group)
    s = scale[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        y = np.where(s > 0, xg / np.where(s > 0, s, np.float32(1)), np.float32(0))
    return y.astype(np.float32).reshape(x.shape)


def quantize_int8(x, group: int = 256, scale_dtype: str = "f32"):
    """int8 symmetric: scale = absmax / 127, code = clip(rint(x / scale), -127, 127).

    x: [..., 256] float.  Returns (codes int8 [..., 256], scales float32
    [..., 256 // group])."""
    x = _as_f32(x)
    scale = _store_scale(_group_absmax(x, group) / np.float32(127.0), scale_dtype)
    y = _scaled(x, scale, group)
    codes = np.clip(np.rint(y), -127, 127).astype(np.int8)
    return codes, scale


def quantize_int4(x, group: int = 32, scale_dtype: str = "f32"):
    """int4 symmetric: scale = absmax / 7, q = clip(rint(x / scale), -7, 7),
    stored as the nibble q + 8, channel 2i in the low nibble of byte i and
    channel 2i+1 in the high nibble.

    Returns (packed uint8 [..., 128], scales float32 [..., 256 // group])."""
    x = _as_f32(x)
    scale = _store_scale(_group_absmax(x, group) / np.float32(7.0), scale_dtype)
    y = _scaled(x, scale, group)
    q = np.clip(np.rint(y), -7, 7).astype(np.int16)
    nib = (q + 8).astype(np.uint8)
    packed = (nib[..., 0::2] & 0xF) | (nib[..., 1::2] << 4)
    return packed.astype(np.uint8), scale


def unpack_int4(packed: np.ndarray) -> np.ndarray:
    """uint8 [..., 128] -> signed codes int8 [..., 256] (nibble - 8)."""
    lo = (packed & 0xF).astype(np.int16) - 8
    hi = (packed >> 4).astype(np.int16) - 8
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def quantize_fp8(x, group: int = 256, scale_dtype: str = "f32"):
    """fp8 e4m3fn with a scale: scale = absmax / 448,
    code = e4m3fn(clamp(x / scale, -448, 448)) rounded to nearest even.

    Returns (codes uint8 [..., 256], scales float32 [..., 256 // group])."""
    import torch
    x = _as_f32(x)
    scale = _store_scale(_group_absmax(x, group) / np.float32(E4M3_MAX), scale_dtype)
    y = np.clip(_scaled(x, scale, group), -E4M3_MAX, E4M3_MAX).astype(np.float32)
    codes = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes.copy(), scale


def quantize(x, fmt: str, group: int, scale_dtype: str = "f32"):
    if fmt == "int8":
        return quantize_int8(x, group, scale_dtype)
    if fmt == "int4":
        return quantize_int4(x, group, scale_dtype)
    if fmt == "fp8":
        return quantize_fp8(x, group, scale_dtype)
    raise ValueError(fmt)


def dequantize(codes: np.ndarray, scale: np.ndarray, fmt: str, group: int) -> np.ndarray:
    """Float64 values of a whole pool (vectorised twin of the C row decoder,
    used only for error-band checks)."""
    if fmt == "int8":
        c = codes.astype(np.float64)
    elif fmt == "int4":
        c = unpack_int4(codes).astype(np.float64)
    elif fmt == "fp8":
        from . import fp8_e4m3fn_to_double
        table = np.array([fp8_e4m3fn_to_double(i) for i in range(256)])
        c = table[codes]
    else:
        raise ValueError(fmt)
    *lead, d = c.shape
    cg = c.reshape(*lead, d // group, group)
    return (cg * scale.astype(np.float64)[..., None]).reshape(c.shape)


def rel_rms(x, xq) -> float:
    x = np.asarray(x, dtype=np.float64)
    xq = np.asarray(xq, dtype=np.float64)
    return float(np.sqrt(np.mean((x - xq) ** 2) / np.mean(x ** 2)))


def store_tiered(k_new, v_new, loc, ring, cold):
    """Write side of the tiered pool (page "feat(qsa): quantized KV pools
    with dequant-on-gather (fp8/int8/int4)", part 4 "Modifications", tiered
    pool bullet): every token is written as int8 with one fp16 scale per 64
    channels into ring row loc & (R - 1), whose owner entry is stamped with
    loc, and as int4 with one fp16 scale per 32 channels into its own slot
    of the full pool.

    Reading where the pages are silent: when several tokens of one call map
    to the same ring row, the token with the largest index wins (row and
    owner both come from it).

    ring = dict(k, v, k_scale, v_scale, owner) numpy arrays ([R, hkv, 256]
    int8, [R, hkv, 4] float32 values of fp16 scales, [R] int32);
    cold = dict(k, v, k_scale, v_scale) ([slots, hkv, 128] uint8,
    [slots, hkv, 8]).  Returns updated copies (ring, cold)."""
    loc = np.asarray(loc, dtype=np.int64)
    ring = {name: np.array(a, copy=True) for name, a in ring.items()}
    cold = {name: np.array(a, copy=True) for name, a in cold.items()}
    r_rows = ring["owner"].shape[0]
    assert r_rows & (r_rows - 1) == 0
    k8, ks8 = quantize_int8(k_new, 64, "f16")
    v8, vs8 = quantize_int8(v_new, 64, "f16")
    k4, ks4 = quantize_int4(k_new, 32, "f16")
    v4, vs4 = quantize_int4(v_new, 32, "f16")
    cold["k"][loc] = k4
    cold["v"][loc] = v4
    cold["k_scale"][loc] = ks4
    cold["v_scale"][loc] = vs4
    for t in range(loc.shape[0]):          # in token order: a later token overwrites
        r = int(loc[t]) & (r_rows - 1)
        ring["k"][r] = k8[t]
        ring["v"][r] = v8[t]
        ring["k_scale"][r] = ks8[t]
        ring["v_scale"][r] = vs8[t]
        ring["owner"][r] = int(loc[t])
    return ring, cold

