"""Bytes of the KV pool layouts -- TEST INFRASTRUCTURE (part of the oracle).

Page "feat(qsa): quantized KV pools with dequant-on-gather (fp8/int8/int4)",
part 4 "Motivation" and "Modifications": a bf16 row is 256 two-byte values;
an int8 row is 256 one-byte codes plus one scale per channel group; an int4
row is 128 bytes (two codes per byte) plus one scale per 32-channel group;
the tiered pool keeps every token in the int4 pool and the most recent R
tokens also in an int8 ring.  Bytes per token count K and V, every KV head
and every QSA layer of the model.
"""
from __future__ import annotations

HEAD_DIM = 256


def code_bytes(fmt: str) -> float:
    return {"bf16": 2.0, "fp16": 2.0, "fp8": 1.0, "int8": 1.0, "int4": 0.5}[fmt]


def row_bytes(fmt: str, group: int = HEAD_DIM, scale_bytes: int = 4) -> int:
    """Bytes of one (slot, kv-head) row of one of K or V: codes + scales."""
    codes = int(HEAD_DIM * code_bytes(fmt))
    if fmt in ("bf16", "fp16"):
        return codes
    return codes + (HEAD_DIM // group) * scale_bytes


def bytes_per_token(fmt: str, group: int = HEAD_DIM, *, kv_heads: int = 2,
                    layers: int = 12, scale_bytes: int = 2) -> int:
    """K + V bytes one token occupies over all QSA layers."""
    return 2 * kv_heads * layers * row_bytes(fmt, group, scale_bytes)


def tiered_bytes_per_token(ring_slots: int, context: int, *, kv_heads: int = 2,
                           layers: int = 12) -> float:
    """int4-g32 for every token plus an int8-g64 ring of ring_slots tokens,
    amortised over a context of ``context`` tokens (fp16 scales)."""
    cold = bytes_per_token("int4", 32, kv_heads=kv_heads, layers=layers)
    hot = bytes_per_token("int8", 64, kv_heads=kv_heads, layers=layers)
    return cold + hot * ring_slots / context


def empty_tiered(ring_rows: int, slots: int, hkv: int = 2):
    """Host arrays of an empty tiered pool: the int8 ring (codes, float32
    values of the fp16 64-channel scales, owner table with -1 = no slot) and
    the int4 pool (all codes 0, i.e. nibble 8, and zero 32-channel scales)."""
    import numpy as np
    ring = dict(k=np.zeros((ring_rows, hkv, HEAD_DIM), np.int8),
                v=np.zeros((ring_rows, hkv, HEAD_DIM), np.int8),
                k_scale=np.zeros((ring_rows, hkv, HEAD_DIM // 64), np.float32),
                v_scale=np.zeros((ring_rows, hkv, HEAD_DIM // 64), np.float32),
                owner=np.full(ring_rows, -1, np.int32))
    cold = dict(k=np.full((slots, hkv, HEAD_DIM // 2), 0x88, np.uint8),
                v=np.full((slots, hkv, HEAD_DIM // 2), 0x88, np.uint8),
                k_scale=np.zeros((slots, hkv, HEAD_DIM // 32), np.float32),
                v_scale=np.zeros((slots, hkv, HEAD_DIM // 32), np.float32))
    return ring, cold
