"""Parity of the HIP quantize + scatter write (qsa_kv_store) with the oracle
quantizers, through the C ABI.

Page "feat(qsa): quantized KV pools with dequant-on-gather (fp8/int8/int4)",
part 4 "Modifications": writing a quantized pool is one fused quantize +
scatter launch, tested bit-exact against a reference quantizer (int8-g64
with int32 and int64 slot ids; int4-g32 including rint ties and the fp16
scale clamp at 65504).  Here every written code and scale must equal the
oracle's (oracle/quant.py) bit for bit, every slot not named in loc must
keep its previous bytes, and pools produced on the device must feed the
decode to the usual tolerance.
"""
import zlib

import numpy as np
import pytest
import torch

import synth
from oracle import quant
from qsa_testlib import run_and_compare, say

import sparse_index_paged_amd as qsa

pytestmark = pytest.mark.gpu

ROW_BYTES = {"fp8": 256, "int8": 256, "int4": 128}
QMAX = {"fp8": 448.0, "int8": 127.0, "int4": 7.0}


def _source_rows(rng, n, hkv, fmt, group):
    """bf16 [n, hkv, 256]: N(0, 1) rows plus rows that hit the edges --
    exact rounding ties, an all-zero group, tiny and huge magnitudes."""
    x = rng.standard_normal((n, hkv, 256), dtype=np.float32)
    if n >= 8:
        # a group whose absmax is QMAX makes the scale exactly 1, so values
        # k + 1/2 are exact ties for rint (int8 / int4) and e4m3fn midpoints
        # are exact ties for the fp8 rounding
        qm = QMAX[fmt]
        t = np.zeros(group, np.float32)
        t[0] = qm
        if fmt == "fp8":
            codes = torch.arange(0, 126, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
            mids = (codes[:-1] + codes[1:]) / 2
            vals = mids[rng.integers(0, len(mids), group - 1)]
        else:
            vals = rng.integers(-int(qm), int(qm), group - 1).astype(np.float32) + 0.5
        t[1:] = vals * np.where(rng.random(group - 1) < 0.5, -1, 1)
        x[0, 0, :group] = t
        x[1, hkv - 1, :group] = 0.0                           # all-zero group
        x[2] *= np.float32(2.0 ** -20)                        # tiny scales (f16 subnormal)
        x[3] *= np.float32(2.0 ** 20)                         # huge: f16 clamp at 65504
        x[4, 0, 5] = np.float32(2.0 ** 30)                    # one outlier per group
    return synth.to_bf16(x)


def _expected(pool_k, pool_v, sk, sv, xk, xv, loc, fmt, group, scale_dtype):
    """Host copies of the pools with rows at loc replaced by the oracle's
    quantization of xk / xv."""
    kc, ks = quant.quantize(xk, fmt, group, scale_dtype)
    vc, vs = quant.quantize(xv, fmt, group, scale_dtype)
    ek, ev = pool_k.copy(), pool_v.copy()
    eks, evs = sk.copy(), sv.copy()
    ek[loc] = kc.view(ek.dtype)
    ev[loc] = vc.view(ev.dtype)
    eks[loc] = ks
    evs[loc] = vs
    return ek, ev, eks, evs


def _pools(rng, slots, hkv, fmt, group, scale_dtype):
    """Device pools filled with random bytes (what was there before) and
    their host copies."""
    nb = ROW_BYTES[fmt]
    kb = rng.integers(0, 256, (slots, hkv, nb), dtype=np.uint8)
    vb = rng.integers(0, 256, (slots, hkv, nb), dtype=np.uint8)
    ng = 256 // group
    sk = rng.random((slots, hkv, ng), dtype=np.float32)
    sv = rng.random((slots, hkv, ng), dtype=np.float32)
    if scale_dtype == "f16":
        sk = sk.astype(np.float16).astype(np.float32)
        sv = sv.astype(np.float16).astype(np.float32)
    tdt = torch.float16 if scale_dtype == "f16" else torch.float32
    dk = torch.from_numpy(kb.view(np.int8) if fmt == "int8" else kb).cuda()
    dv = torch.from_numpy(vb.view(np.int8) if fmt == "int8" else vb).cuda()
    dsk = torch.from_numpy(sk).to(tdt).cuda()
    dsv = torch.from_numpy(sv).to(tdt).cuda()
    return (kb, vb, sk, sv), (dk, dv, dsk, dsv)


def _check_pools(dev, exp, label):
    dk, dv, dsk, dsv = dev
    ek, ev, eks, evs = exp
    got_k = dk.cpu().numpy().view(np.uint8)
    got_v = dv.cpu().numpy().view(np.uint8)
    for name, got, want in (("k codes", got_k, ek.view(np.uint8)), ("v codes", got_v, ev.view(np.uint8))):
        bad = np.argwhere(got != want)
        assert bad.size == 0, f"{label}: {name} differ at {len(bad)} bytes, first {bad[:3].tolist()}"
    for name, got, want in (("k scales", dsk.float().cpu().numpy(), eks),
                            ("v scales", dsv.float().cpu().numpy(), evs)):
        assert np.array_equal(got.view(np.uint32), want.astype(np.float32).view(np.uint32)), \
            f"{label}: {name} differ at {np.count_nonzero(got != want)} entries"


CASES = [("fp8", 256), ("fp8", 64), ("fp8", 32), ("int8", 256), ("int8", 64), ("int8", 32),
         ("int4", 64), ("int4", 32)]


@pytest.mark.parametrize("fmt,group", CASES)
@pytest.mark.parametrize("scale_dtype", ["f32", "f16"])
@pytest.mark.parametrize("hkv", [2, 1])
def test_store_bit_exact(fmt, group, scale_dtype, hkv):
    seed = zlib.crc32(f"{fmt}/{group}/{scale_dtype}/{hkv}".encode())
    rng = np.random.default_rng(seed)
    slots, n = 3000, 777
    label = f"store {fmt} g{group} {scale_dtype} hkv{hkv}"
    say(f"[gpu] {label}: slots={slots} n={n}")
    host, dev = _pools(rng, slots, hkv, fmt, group, scale_dtype)
    xk = _source_rows(rng, n, hkv, fmt, group)
    xv = _source_rows(rng, n, hkv, fmt, group)
    loc = rng.permutation(slots)[:n]
    loc_t = torch.from_numpy(loc.astype(np.int64 if hkv == 1 else np.int32)).cuda()
    qsa.kv_store(xk.cuda(), xv.cuda(), loc_t, dev[0], dev[1], kv_format=fmt, k_scale=dev[2],
                 v_scale=dev[3], group_size=group)
    torch.cuda.synchronize()
    exp = _expected(*host, xk, xv, loc, fmt, group, scale_dtype)
    _check_pools(dev, exp, label)


def test_store_bf16_pool_is_a_copy():
    rng = np.random.default_rng(5)
    slots, n = 500, 129
    k = torch.from_numpy(rng.standard_normal((slots, 2, 256), dtype=np.float32)).to(torch.bfloat16)
    v = torch.from_numpy(rng.standard_normal((slots, 2, 256), dtype=np.float32)).to(torch.bfloat16)
    xk = synth.normal_bf16(rng, (n, 2, 256))
    xv = synth.normal_bf16(rng, (n, 2, 256))
    loc = rng.permutation(slots)[:n].astype(np.int32)
    dk, dv = k.cuda(), v.cuda()
    qsa.kv_store(xk.cuda(), xv.cuda(), torch.from_numpy(loc).cuda(), dk, dv)
    torch.cuda.synchronize()
    k[loc] = xk
    v[loc] = xv
    assert torch.equal(dk.cpu(), k) and torch.equal(dv.cpu(), v)


def test_store_strided_views_and_empty_call():
    """Sources and pools as strided views; n = 0 writes nothing."""
    rng = np.random.default_rng(6)
    slots, n, fmt, group = 700, 200, "int8", 64
    big_src = synth.normal_bf16(rng, (n, 3, 256))
    xk, xv = big_src[:, 0:2], big_src[:, 1:3]
    dbig = big_src.cuda()
    dxk, dxv = dbig[:, 0:2], dbig[:, 1:3]   # strided device views
    kb = rng.integers(-128, 128, (slots, 4, 256), dtype=np.int8)
    vb = rng.integers(-128, 128, (slots, 3, 256), dtype=np.int8)
    sbig = rng.random((slots, 2, 8), dtype=np.float32)
    dkb, dvb, dsb = torch.from_numpy(kb).cuda(), torch.from_numpy(vb).cuda(), torch.from_numpy(sbig).cuda()
    dk, dv = dkb[:, 1:3], dvb[:, 0:2]
    dsk, dsv = dsb[:, :, 0:4], dsb[:, :, 4:8]
    loc = rng.permutation(slots)[:n].astype(np.int32)
    empty = torch.zeros(0, 2, 256, dtype=torch.bfloat16, device="cuda")
    qsa.kv_store(empty, empty, torch.zeros(0, dtype=torch.int32, device="cuda"), dk, dv,
                 kv_format=fmt, k_scale=dsk, v_scale=dsv, group_size=group)
    torch.cuda.synchronize()
    assert np.array_equal(dkb.cpu().numpy(), kb) and np.array_equal(dsb.cpu().numpy(), sbig)
    assert not dxk.is_contiguous() and not dk.is_contiguous() and not dsv.is_contiguous()
    qsa.kv_store(dxk, dxv, torch.from_numpy(loc).cuda(), dk, dv, kv_format=fmt,
                 k_scale=dsk, v_scale=dsv, group_size=group)
    torch.cuda.synchronize()
    kc, ks = quant.quantize(xk, fmt, group)
    vc, vs = quant.quantize(xv, fmt, group)
    ek, ev, es = kb.copy(), vb.copy(), sbig.copy()
    ek[loc, 1:3] = kc
    ev[loc, 0:2] = vc
    es[loc, :, 0:4] = ks
    es[loc, :, 4:8] = vs
    assert np.array_equal(dkb.cpu().numpy(), ek)
    assert np.array_equal(dvb.cpu().numpy(), ev)
    assert np.array_equal(dsb.cpu().numpy(), es)


def test_store_bad_slots_are_skipped_and_reported():
    rng = np.random.default_rng(7)
    slots, n, fmt, group = 400, 64, "int4", 32
    host, dev = _pools(rng, slots, 2, fmt, group, "f32")
    xk = _source_rows(rng, n, 2, fmt, group)
    xv = _source_rows(rng, n, 2, fmt, group)
    loc = rng.permutation(slots)[:n].astype(np.int64)
    bad = np.array([3, 17, 40])
    loc_bad = loc.copy()
    loc_bad[bad] = [slots, -1, 1 << 40]
    qsa.workspace_reset()
    qsa.kv_store(xk.cuda(), xv.cuda(), torch.from_numpy(loc_bad).cuda(), dev[0], dev[1],
                 kv_format=fmt, k_scale=dev[2], v_scale=dev[3], group_size=group)
    assert qsa.debug_device_error() == 4
    keep = np.setdiff1d(np.arange(n), bad)
    exp = _expected(*host, xk[keep], xv[keep], loc[keep], fmt, group, "f32")
    _check_pools(dev, exp, "bad slots")
    qsa.workspace_reset()
    assert qsa.debug_device_error() == 0


@pytest.mark.parametrize("fmt,group,scale_dtype", [("fp8", 256, "f32"), ("int8", 256, "f32"),
                                                   ("int4", 32, "f32"), ("int8", 64, "f16"),
                                                   ("int4", 32, "f16")])
def test_pools_written_on_device_feed_the_decode(fmt, group, scale_dtype):
    """bs=64 TP1 quantized-pool workload with the pools produced by
    qsa_kv_store from the bf16 source pools (every slot, in a shuffled
    order), checked bit-exact against the oracle quantizer and then decoded
    against the oracle."""
    case = synth.case_bs64_tp1_quantsrc(3100 + group)
    slots = case.k_pool.shape[0]
    rng = np.random.default_rng(group)
    order = rng.permutation(slots).astype(np.int32)
    nb = ROW_BYTES[fmt]
    pdt = torch.int8 if fmt == "int8" else torch.uint8
    tdt = torch.float16 if scale_dtype == "f16" else torch.float32
    dk = torch.empty((slots, 2, nb), dtype=pdt, device="cuda")
    dv = torch.empty((slots, 2, nb), dtype=pdt, device="cuda")
    dsk = torch.empty((slots, 2, 256 // group), dtype=tdt, device="cuda")
    dsv = torch.empty((slots, 2, 256 // group), dtype=tdt, device="cuda")
    say(f"[gpu] device-written {fmt} g{group} {scale_dtype} pools, bs=64 tp1")
    qsa.kv_store(case.k_pool[order].cuda(), case.v_pool[order].cuda(), torch.from_numpy(order).cuda(),
                 dk, dv, kv_format=fmt, k_scale=dsk, v_scale=dsv, group_size=group)
    torch.cuda.synchronize()
    kc, ks = quant.quantize(case.k_pool, fmt, group, scale_dtype)
    vc, vs = quant.quantize(case.v_pool, fmt, group, scale_dtype)
    assert np.array_equal(dk.cpu().numpy().view(np.uint8), kc.view(np.uint8))
    assert np.array_equal(dv.cpu().numpy().view(np.uint8), vc.view(np.uint8))
    assert np.array_equal(dsk.float().cpu().numpy(), ks) and np.array_equal(dsv.float().cpu().numpy(), vs)
    rows = sorted(np.random.default_rng(1).choice(64, 16, replace=False).tolist())
    run_and_compare(case, f"decode on device-written {fmt} g{group} {scale_dtype}", rows=rows,
                    quant=(fmt, group, kc, ks, vc, vs), scale_dtype=tdt)


def _bf16_grid():
    """Every finite non-negative bf16 value, as float32."""
    bits = np.arange(0, 0x7F80, dtype=np.uint32) << 16
    return bits.view(np.float32)


def _adversarial_rows(rng, n, hkv, fmt, group, scale_dtype):
    """bf16 rows whose quotients x / scale sit on or within a few ulp of a
    rounding boundary of the code (half-integers for int8 / int4, midpoints
    of the e4m3fn grid for fp8), so that any shortcut in computing the
    quotient would change codes."""
    grid = _bf16_grid()
    qmax = np.float32(QMAX[fmt])
    x = np.zeros((n, hkv, 256), np.float32)
    for r in range(n):
        for h in range(hkv):
            for g0 in range(0, 256, group):
                amax = np.float32(grid[rng.integers(0x3F00, 0x4080)])    # [0.5, 4)
                s = np.float32(amax / qmax)
                if scale_dtype == "f16":
                    s = np.float32(np.float16(min(s, np.float32(65504.0))))
                cand = grid[grid <= amax]
                y = (cand / s).astype(np.float32)
                if fmt == "fp8":
                    yc = np.minimum(y, np.float32(448.0))
                    bits = yc.view(np.uint32).astype(np.int64)
                    dist = np.abs((bits & 0xFFFFF) - 0x80000).astype(np.float64)
                    sub = yc < np.float32(2.0 ** -6)
                    t = yc[sub] * np.float32(512.0)
                    dist[sub] = np.abs(t - np.floor(t) - 0.5) / np.maximum(np.spacing(t), 1e-30)
                else:
                    dist = np.abs(y - np.floor(y) - 0.5) / np.spacing(np.maximum(y, 1.0))
                pick = cand[np.argsort(dist, kind="stable")[: 4 * group]]
                vals = rng.choice(pick, group - 1, replace=False)
                vals = vals * np.where(rng.random(group - 1) < 0.5, -1, 1)
                x[r, h, g0] = amax
                x[r, h, g0 + 1: g0 + group] = vals
    return synth.to_bf16(x)


@pytest.mark.parametrize("fmt,group", [("int8", 32), ("int8", 256), ("int4", 32), ("fp8", 32),
                                       ("fp8", 256)])
@pytest.mark.parametrize("scale_dtype", ["f32", "f16"])
def test_store_quotients_near_rounding_boundaries(fmt, group, scale_dtype):
    seed = zlib.crc32(f"adv/{fmt}/{group}/{scale_dtype}".encode())
    rng = np.random.default_rng(seed)
    slots, n, hkv = 256, 48, 2
    label = f"near-boundary store {fmt} g{group} {scale_dtype}"
    say(f"[gpu] {label}")
    host, dev = _pools(rng, slots, hkv, fmt, group, scale_dtype)
    xk = _adversarial_rows(rng, n, hkv, fmt, group, scale_dtype)
    xv = _adversarial_rows(rng, n, hkv, fmt, group, scale_dtype)
    loc = rng.permutation(slots)[:n].astype(np.int32)
    qsa.kv_store(xk.cuda(), xv.cuda(), torch.from_numpy(loc).cuda(), dev[0], dev[1], kv_format=fmt,
                 k_scale=dev[2], v_scale=dev[3], group_size=group)
    torch.cuda.synchronize()
    exp = _expected(*host, xk, xv, loc, fmt, group, scale_dtype)
    _check_pools(dev, exp, label)


@pytest.mark.parametrize("fmt,group", [("int8", 64), ("int4", 32), ("fp8", 256)])
def test_store_repeated_slot_leaves_every_other_slot_exact(fmt, group):
    """qsa.h: the slot ids of one call must be distinct; a repeated id leaves
    that slot holding an unspecified mix of the rows written to it.  The
    rest of the call stays exact: every other written slot equals the
    oracle's quantization, every unwritten slot keeps its bytes, and each
    scale of the repeated slot is the one of the two tokens' (a scale is a
    single store)."""
    rng = np.random.default_rng(zlib.crc32(f"dup/{fmt}/{group}".encode()))
    slots, n, hkv = 2000, 300, 2
    host, dev = _pools(rng, slots, hkv, fmt, group, "f16")
    xk = _source_rows(rng, n, hkv, fmt, group)
    xv = _source_rows(rng, n, hkv, fmt, group)
    loc = rng.permutation(slots)[:n].astype(np.int64)
    loc[200] = loc[17]                              # tokens 17 and 200 both name one slot
    dup = int(loc[17])
    say(f"[gpu] store {fmt} g{group}: slot {dup} named twice")
    qsa.kv_store(xk.cuda(), xv.cuda(), torch.from_numpy(loc.astype(np.int32)).cuda(), dev[0], dev[1],
                 kv_format=fmt, k_scale=dev[2], v_scale=dev[3], group_size=group)
    torch.cuda.synchronize()
    keep = np.ones(n, bool)
    keep[[17, 200]] = False
    kt = torch.from_numpy(keep)
    ek, ev, eks, evs = _expected(*host, xk[kt], xv[kt], loc[keep], fmt, group, "f16")
    other = np.arange(slots) != dup
    for name, got, want in (("k codes", dev[0].cpu().numpy().view(np.uint8), ek.view(np.uint8)),
                            ("v codes", dev[1].cpu().numpy().view(np.uint8), ev.view(np.uint8)),
                            ("k scales", dev[2].float().cpu().numpy().view(np.uint32),
                             eks.astype(np.float32).view(np.uint32)),
                            ("v scales", dev[3].float().cpu().numpy().view(np.uint32),
                             evs.astype(np.float32).view(np.uint32))):
        assert np.array_equal(got[other], want[other]), f"{fmt}: {name} of other slots differ"
    for name, x, d in (("k", xk, dev[2]), ("v", xv, dev[3])):
        tok = quant.quantize(x[[17, 200]], fmt, group, "f16")[1]
        s_dup = d[dup].float().cpu().numpy()
        assert np.all((s_dup == tok[0]) | (s_dup == tok[1])), f"{fmt}: {name} scale of the repeated slot"
