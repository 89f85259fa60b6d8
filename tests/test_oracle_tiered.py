"""Pins for the oracle's tiered pool (int8 ring + int4 full pool).

Source: page "feat(qsa): quantized KV pools with dequant-on-gather
(fp8/int8/int4)", part 4 "Modifications", tiered pool bullet (every token is
written as int8-g64 into a ring of R rows with an int32 owner table and as
int4-g32 into the full pool; a reader takes ring row slot & (R - 1) when its
owner is the slot, else the int4 row) and the bullet on its registered unit
test (owner stamping with R = 64 over 4096 slots and ring wrap, hot/cold
boundary, same-launch ring-row collisions, stale owner -> int4 path, fp16
clamp on the ring, all-cold / all-hot equal to the single-tier pools).

Expected values come from the token values themselves (which tier a slot
must read after a known write history) and from plain float64 softmax
attention in torch over numpy-dequantized rows, never from the tiered
oracle's own row selection.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import layout, quant

HKV = 2


def empty_tiers(ring_rows: int, slots: int, hkv: int = HKV):
    return layout.empty_tiered(ring_rows, slots, hkv)


def tiered_decode(q, ring, cold, sel, cu, **kw):
    return oracle.decode_tiered(q, ring["owner"], ring["k"], ring["v"], ring["k_scale"],
                                ring["v_scale"], cold["k"], cold["v"], cold["k_scale"],
                                cold["v_scale"], sel, cu, **kw)


def brute_force(q, krows, vrows, sel, cu):
    """softmax(q k^T / 16) v per (row, head) in float64; krows / vrows
    [slots, hkv, 256] float64 values of each slot as the reader must see it."""
    bs, hq = q.shape[0], q.shape[1]
    hkv = krows.shape[1]
    qpk = hq // hkv
    out = np.zeros((bs, hq, 256))
    lse = np.full((bs, hq), -np.inf)
    kt, vt = torch.from_numpy(krows), torch.from_numpy(vrows)
    for b in range(bs):
        idx = torch.from_numpy(sel[cu[b]:cu[b + 1]].astype(np.int64))
        if idx.numel() == 0:
            continue
        for g in range(hkv):
            qg = q[b, qpk * g:qpk * (g + 1)].double()
            logits = qg @ kt[idx, g].T / 16
            out[b, qpk * g:qpk * (g + 1)] = (torch.softmax(logits, -1) @ vt[idx, g]).numpy()
            lse[b, qpk * g:qpk * (g + 1)] = torch.logsumexp(logits, -1).numpy()
    return out, lse


def tier_values(x, hot_mask):
    """Float64 values a reader must see for token values x [slots, hkv, 256]:
    int8-g64 round trip where hot, int4-g32 round trip elsewhere (both with
    fp16 scales), quantized from the token values directly."""
    c8, s8 = quant.quantize_int8(x, 64, "f16")
    c4, s4 = quant.quantize_int4(x, 32, "f16")
    hot = quant.dequantize(c8, s8, "int8", 64)
    cold = quant.dequantize(c4, s4, "int4", 32)
    return np.where(np.asarray(hot_mask)[:, None, None], hot, cold)


def close(a, b):
    np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-12)


def test_all_cold_equals_int4_single_tier():
    rng = np.random.default_rng(31)
    slots, r = 80, 16
    x = synth.normal_bf16(rng, (slots, HKV, 256))
    y = synth.normal_bf16(rng, (slots, HKV, 256))
    q = synth.normal_bf16(rng, (3, 24, 256))
    sel, cu = synth.pack([synth.draw_indices(rng, n, slots, 0.2) for n in (40, 1, 77)])
    ring, cold = empty_tiers(r, slots)
    cold["k"], cold["k_scale"] = quant.quantize_int4(x, 32, "f16")
    cold["v"], cold["v_scale"] = quant.quantize_int4(y, 32, "f16")
    # ring rows full of other data, owners pointing at slots never listed
    ring["k"] = rng.integers(-127, 128, ring["k"].shape).astype(np.int8)
    ring["k_scale"][:] = 1.0
    ring["owner"][:] = np.arange(r) + 1000
    o, l = tiered_decode(q, ring, cold, sel, cu)
    o1, l1 = oracle.decode(q, cold["k"], cold["v"], sel, cu, fmt="int4", group=32,
                           k_scale=cold["k_scale"], v_scale=cold["v_scale"])
    np.testing.assert_array_equal(o, o1)
    np.testing.assert_array_equal(l, l1)
    ob, lb = brute_force(q, tier_values(x, np.zeros(slots, bool)),
                         tier_values(y, np.zeros(slots, bool)), sel, cu)
    close(o, ob)
    close(l, lb)


def test_all_hot_equals_int8_single_tier():
    rng = np.random.default_rng(32)
    slots = r = 64
    x = synth.normal_bf16(rng, (slots, HKV, 256))
    y = synth.normal_bf16(rng, (slots, HKV, 256))
    q = synth.normal_bf16(rng, (2, 24, 256))
    sel, cu = synth.pack([synth.draw_indices(rng, n, slots, 0.3) for n in (64, 23)])
    ring, cold = store_all(x, y, np.arange(slots), r, slots)
    assert np.array_equal(ring["owner"], np.arange(r))
    o, l = tiered_decode(q, ring, cold, sel, cu)
    o1, l1 = oracle.decode(q, ring["k"], ring["v"], sel, cu, fmt="int8", group=64,
                           k_scale=ring["k_scale"], v_scale=ring["v_scale"])
    np.testing.assert_array_equal(o, o1)
    np.testing.assert_array_equal(l, l1)
    ob, lb = brute_force(q, tier_values(x, np.ones(slots, bool)),
                         tier_values(y, np.ones(slots, bool)), sel, cu)
    close(o, ob)
    close(l, lb)


def store_all(x, y, loc, r, slots, batches=1, rng=None):
    ring, cold = empty_tiers(r, slots, x.shape[1])
    loc = np.asarray(loc)
    cuts = [0, len(loc)] if batches == 1 else \
        sorted(set([0, len(loc)] + list(rng.integers(1, len(loc), batches - 1))))
    for a, b in zip(cuts[:-1], cuts[1:]):
        ring, cold = quant.store_tiered(x[loc[a:b]], y[loc[a:b]], loc[a:b], ring, cold)
    return ring, cold


def test_ring_wrap_hot_set_is_the_most_recent_ring_rows():
    """R = 64 over 4096 slots written in order in uneven batches: afterwards
    exactly the last 64 written slots read int8; every older slot finds its
    ring row owned by a newer slot (stale owner) and reads int4."""
    rng = np.random.default_rng(33)
    slots, r, n = 4096, 64, 4000
    x = synth.normal_bf16(rng, (slots, 1, 256))
    y = synth.normal_bf16(rng, (slots, 1, 256))
    ring, cold = store_all(x, y, np.arange(n), r, slots, batches=37, rng=rng)
    np.testing.assert_array_equal(np.sort(ring["owner"]), np.arange(n - r, n))
    hot = np.zeros(slots, bool)
    hot[n - r:n] = True
    q = synth.normal_bf16(rng, (4, 12, 256))
    lists = [np.arange(n - r - 40, n - r + 40),           # across the hot/cold boundary
             rng.integers(0, n, 300),                     # mostly cold, repeats allowed
             np.arange(n - r, n)[::-1],                   # all hot
             np.arange(0, 64)]                            # oldest: ring rows owned by newer slots
    sel, cu = synth.pack([np.asarray(a, np.int32) for a in lists])
    o, l = tiered_decode(q, ring, cold, sel, cu)
    ob, lb = brute_force(q, tier_values(x, hot), tier_values(y, hot), sel, cu)
    close(o, ob)
    close(l, lb)
    # one stale-owner slot alone reads exactly the int4 single-tier result
    s = np.array([n - r - 1], np.int32)
    assert ring["owner"][s[0] & (r - 1)] == n - 1
    o1, l1 = tiered_decode(q[:1], ring, cold, s, np.array([0, 1], np.int32))
    o2, l2 = oracle.decode(q[:1], cold["k"], cold["v"], s, np.array([0, 1], np.int32),
                           fmt="int4", group=32, k_scale=cold["k_scale"],
                           v_scale=cold["v_scale"])
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_permuted_slots_hot_set_follows_write_order():
    """Slots handed out in a random order: the hot set is, per ring row, the
    slot written last among those that map to it."""
    rng = np.random.default_rng(34)
    slots, r = 4096, 64
    loc = rng.permutation(slots)[:1500]
    x = synth.normal_bf16(rng, (slots, HKV, 256))
    y = synth.normal_bf16(rng, (slots, HKV, 256))
    ring, cold = store_all(x, y, loc, r, slots, batches=9, rng=rng)
    last = {}
    for s in loc:
        last[int(s) & (r - 1)] = int(s)
    hot = np.zeros(slots, bool)
    hot[list(last.values())] = True
    assert hot.sum() == len(last)
    q = synth.normal_bf16(rng, (3, 24, 256))
    sel, cu = synth.pack([rng.choice(loc, 200), loc[-100:], rng.choice(loc, 7)])
    o, l = tiered_decode(q, ring, cold, sel.astype(np.int32), cu)
    ob, lb = brute_force(q, tier_values(x, hot), tier_values(y, hot), sel, cu)
    close(o, ob)
    close(l, lb)


def test_same_launch_ring_collisions_last_token_wins():
    """Tokens of one write that share a ring row: the ring row and its owner
    both come from the last of them; the others read int4."""
    rng = np.random.default_rng(35)
    slots, r = 256, 64
    x = synth.normal_bf16(rng, (slots, HKV, 256))
    y = synth.normal_bf16(rng, (slots, HKV, 256))
    loc = np.array([5, 69, 133, 7, 200, 71], np.int64)
    ring, cold = store_all(x, y, loc, r, slots)
    assert ring["owner"][5] == 133 and ring["owner"][7] == 71 and ring["owner"][8] == 200
    c8, s8 = quant.quantize_int8(x[133], 64, "f16")
    np.testing.assert_array_equal(ring["k"][5], c8)
    np.testing.assert_array_equal(ring["k_scale"][5], s8)
    hot = np.zeros(slots, bool)
    hot[[133, 71, 200]] = True
    q = synth.normal_bf16(rng, (2, 24, 256))
    sel, cu = synth.pack([loc.astype(np.int32), np.array([5, 5, 133, 69, 7], np.int32)])
    o, l = tiered_decode(q, ring, cold, sel, cu)
    ob, lb = brute_force(q, tier_values(x, hot), tier_values(y, hot), sel, cu)
    close(o, ob)
    close(l, lb)


def test_fp16_clamp_on_the_ring():
    x = np.zeros((1, 1, 256), np.float32)
    x[0, 0, 3] = 127.0 * 70000.0            # int8 scale 70000 > fp16 max
    x[0, 0, 100] = -2.0
    ring, cold = empty_tiers(4, 8, 1)
    ring, cold = quant.store_tiered(x, x, np.array([6]), ring, cold)
    assert ring["owner"][2] == 6
    assert ring["k_scale"][2, 0, 0] == 65504.0
    assert ring["k"][2, 0, 3] == 127
    assert ring["k_scale"][2, 0, 1] == np.float32(np.float16(2.0 / 127))
    assert cold["k_scale"][6, 0, 0] == 65504.0


def test_empty_rows_and_rejections():
    rng = np.random.default_rng(36)
    ring, cold = empty_tiers(16, 32)
    q = synth.normal_bf16(rng, (2, 24, 256))
    sel = np.array([3, 4], np.int32)
    cu = np.array([0, 0, 2], np.int32)
    o, l = tiered_decode(q, ring, cold, sel, cu)
    assert not o[0].any() and np.all(np.isneginf(l[0]))
    assert np.all(np.isfinite(o[1]))
    with pytest.raises(ValueError):
        tiered_decode(q, ring, cold, np.array([3, 32], np.int32), cu)
    bad_ring, _ = empty_tiers(12, 32)                     # ring rows not a power of two
    with pytest.raises(ValueError):
        tiered_decode(q, bad_ring, cold, sel, cu)
