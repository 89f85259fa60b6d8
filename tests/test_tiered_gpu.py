"""Parity of the HIP tiered-pool path (qsa_kv_store_tiered, qsa_decode_tiered)
with the oracle, through the C ABI.

Page "feat(qsa): quantized KV pools with dequant-on-gather (fp8/int8/int4)",
part 4 "Modifications", tiered pool bullet and its registered unit test:
every token is written twice (int8-g64 into a ring of R rows with an owner
table, int4-g32 into the full pool), same-launch ring-row collisions, ring
wrap with R = 64 over 4096 slots, stale owners reading int4, and all-cold /
all-hot pools.  Writes must equal the oracle's (oracle/quant.py
store_tiered) bit for bit, with the claim table back at zero; decodes must
meet the decode tolerance against oracle.decode_tiered.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import layout, quant
from qsa_testlib import compare, oracle_threads, say

import sparse_index_paged_amd as qsa

pytestmark = pytest.mark.gpu

ARRAYS = ("k", "v", "k_scale", "v_scale")


def to_dev(ring, cold):
    """Device tiered pool (dict of qsa_tiered_pool fields) from host arrays."""
    f16 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.float16).cuda()
    return dict(ring_k=torch.from_numpy(ring["k"]).cuda(), ring_v=torch.from_numpy(ring["v"]).cuda(),
                ring_k_scale=f16(ring["k_scale"]), ring_v_scale=f16(ring["v_scale"]),
                owner=torch.from_numpy(ring["owner"]).cuda(),
                claim=torch.zeros(ring["owner"].shape[0], dtype=torch.int32, device="cuda"),
                cold_k=torch.from_numpy(cold["k"]).cuda(), cold_v=torch.from_numpy(cold["v"]).cuda(),
                cold_k_scale=f16(cold["k_scale"]), cold_v_scale=f16(cold["v_scale"]))


def check_pool(dev, ring, cold, label, slot_rows=None):
    """Every device array equals the oracle's bit for bit (scales compared
    as fp16 bit patterns); slot_rows limits the int4 pool check to rows."""
    torch.cuda.synchronize()
    def f16bits(a):
        return np.ascontiguousarray(a, np.float32).astype(np.float16).view(np.uint16)
    rows = slice(None) if slot_rows is None else slot_rows
    for name in ARRAYS:
        d = dev["ring_" + name].cpu()
        e = ring[name]
        if "scale" in name:
            assert np.array_equal(d.view(torch.int16).numpy().view(np.uint16), f16bits(e)), f"{label}: ring {name}"
        else:
            assert np.array_equal(d.numpy(), e), f"{label}: ring {name}"
        d = dev["cold_" + name].cpu()[rows]
        e = cold[name][rows]
        if "scale" in name:
            assert np.array_equal(d.view(torch.int16).numpy().view(np.uint16), f16bits(e)), f"{label}: cold {name}"
        else:
            assert np.array_equal(d.numpy(), e), f"{label}: cold {name}"
    assert np.array_equal(dev["owner"].cpu().numpy(), ring["owner"]), f"{label}: owner"
    assert not dev["claim"].any().item(), f"{label}: claim table not back at zero"


def oracle_tiered(q, ring, cold, sel, cu):
    return oracle.decode_tiered(q, ring["owner"], ring["k"], ring["v"], ring["k_scale"],
                                ring["v_scale"], cold["k"], cold["v"], cold["k_scale"],
                                cold["v_scale"], sel, cu, nthreads=oracle_threads())


def decode_and_compare(q, dev, ring, cold, sel, cu, label, rows=None):
    say(f"[gpu] tiered decode {label}: bs={q.shape[0]} hq={q.shape[1]} n_sel={sel.shape[0]} "
        f"R={ring['owner'].shape[0]} slots={cold['k'].shape[0]}")
    out, lse = qsa.decode_tiered(q.cuda(), dev, torch.from_numpy(sel).cuda(), torch.from_numpy(cu).cuda())
    torch.cuda.synchronize()
    lengths = np.diff(cu)
    if rows is None:
        o_ref, l_ref = oracle_tiered(q, ring, cold, sel, cu)
        compare(out, lse, o_ref, l_ref, lengths, label=label)
    else:
        lists = [sel[cu[b]:cu[b + 1]] for b in rows]
        sel2, cu2 = synth.pack(lists)
        o_ref, l_ref = oracle_tiered(q[rows].contiguous(), ring, cold, sel2, cu2)
        compare(out[rows], lse[rows], o_ref, l_ref, lengths[rows], label=label)
    assert all(v == 0 for v in qsa.debug_counters())
    return out, lse


def write_history(x, y, batches, ring, cold):
    for loc in batches:
        ring, cold = quant.store_tiered(x[loc], y[loc], loc, ring, cold)
    return ring, cold


@pytest.mark.parametrize("hkv", [2, 1])
@pytest.mark.parametrize("loc_dtype", [torch.int32, torch.int64])
def test_tiered_store_bit_exact(hkv, loc_dtype):
    """R = 64 over 4096 slots: 1500 slots in a shuffled order over 9 calls
    (ring wrap, stale owners), then one call whose tokens collide on ring
    rows; every array bit-exact after each call."""
    rng = np.random.default_rng(500 + hkv)
    slots, r = 4096, 64
    x = synth.normal_bf16(rng, (slots, hkv, 256))
    y = synth.normal_bf16(rng, (slots, hkv, 256))
    x[7] *= 2.0 ** 20                                    # fp16 scale clamp on both tiers
    ring, cold = layout.empty_tiered(r, slots, hkv)
    dev = to_dev(ring, cold)
    batches = synth.write_batches(rng, rng.permutation(slots)[:1500], 9)
    batches.append(np.array([5, 69, 133, 7, 200, 71, 7 + 64 * 30], np.int64))
    batches.append(np.array([], np.int64))
    for i, loc in enumerate(batches):
        say(f"[gpu] tiered store call {i}: n={len(loc)} hkv={hkv} {loc_dtype}")
        qsa.kv_store_tiered(x[loc].cuda(), y[loc].cuda(), torch.from_numpy(loc).to(loc_dtype).cuda(), dev)
        ring, cold = quant.store_tiered(x[loc], y[loc], loc, ring, cold)
        check_pool(dev, ring, cold, f"call {i}")
    assert ring["owner"][5] == 133 and ring["owner"][7] == 7 + 64 * 30


def test_tiered_store_bad_slots_are_skipped_and_reported():
    rng = np.random.default_rng(510)
    slots, r, n = 1024, 128, 200
    x = synth.normal_bf16(rng, (slots, 2, 256))
    y = synth.normal_bf16(rng, (slots, 2, 256))
    ring, cold = layout.empty_tiered(r, slots, 2)
    dev = to_dev(ring, cold)
    loc = rng.permutation(slots)[:n].astype(np.int64)
    bad = np.array([3, 50, 199])
    loc_bad = loc.copy()
    loc_bad[bad] = [slots, -1, 1 << 40]
    qsa.workspace_reset()
    qsa.kv_store_tiered(x[loc].cuda(), y[loc].cuda(), torch.from_numpy(loc_bad).cuda(), dev)
    assert qsa.debug_device_error() == 4
    keep = np.setdiff1d(np.arange(n), bad)
    ring, cold = quant.store_tiered(x[loc[keep]], y[loc[keep]], loc[keep], ring, cold)
    check_pool(dev, ring, cold, "bad slots")
    qsa.workspace_reset()
    assert qsa.debug_device_error() == 0


@pytest.mark.parametrize("hkv,r,slots,hot_frac", [(2, 1024, 8192, 0.5), (1, 1024, 8192, 0.5),
                                                  (2, 64, 4096, 0.3), (2, 8192, 16384, 0.9)])
def test_tiered_decode_mixed_tiers(hkv, r, slots, hot_frac):
    """Pools written by the oracle from a shuffled write history; lists mix
    recently written slots (hot unless their ring row was taken since) with
    uniform draws; mixed lengths incl. 0, 1 and 2055 and duplicate runs."""
    rng = np.random.default_rng(520 + r + hkv)
    x = synth.normal_bf16(rng, (slots, hkv, 256))
    y = synth.normal_bf16(rng, (slots, hkv, 256))
    order = rng.permutation(slots)
    ring, cold = write_history(x, y, synth.write_batches(rng, order, 12),
                               *layout.empty_tiered(r, slots, hkv))
    lens = synth.mixed_lengths_bs16(rng)
    lens[3], lens[9] = 0, 1
    sel, cu = synth.tiered_lists(rng, lens, slots, order[-r:], hot_frac, dup_prob=0.05)
    hot = (ring["owner"][sel & (r - 1)] == sel).mean()
    say(f"  hot entries: {hot:.2f}")
    q = synth.normal_bf16(rng, (16, 12 * hkv, 256))
    decode_and_compare(q, to_dev(ring, cold), ring, cold, sel, cu, f"hkv{hkv} R{r} hot{hot:.2f}")


@pytest.mark.parametrize("kind", ["all_cold", "all_hot"])
def test_tiered_decode_single_tier(kind):
    rng = np.random.default_rng(530)
    slots, hkv = 2048, 2
    r = 2048 if kind == "all_hot" else 256
    x = synth.normal_bf16(rng, (slots, hkv, 256))
    y = synth.normal_bf16(rng, (slots, hkv, 256))
    ring, cold = write_history(x, y, synth.write_batches(rng, rng.permutation(slots), 5),
                               *layout.empty_tiered(r, slots, hkv))
    if kind == "all_cold":
        ring["owner"][:] = -1
    else:
        assert np.array_equal(np.sort(ring["owner"]), np.arange(slots))
    sel, cu = synth.pack([synth.draw_indices(rng, n, slots, 0.1) for n in (2055, 300, 17, 2055)])
    q = synth.normal_bf16(rng, (4, 24, 256))
    decode_and_compare(q, to_dev(ring, cold), ring, cold, sel, cu, kind)


def test_tiered_pools_written_on_device_feed_the_decode():
    """kv_store_tiered writes every slot of a bs=64 workload's pools (shuffled
    order, 16 calls); the pools are checked bit-exact against the oracle's
    and then decoded against the oracle."""
    rng = np.random.default_rng(540)
    slots, hkv, r = 32768, 2, 4096
    x = synth.normal_bf16(rng, (slots, hkv, 256))
    y = synth.normal_bf16(rng, (slots, hkv, 256))
    ring, cold = layout.empty_tiered(r, slots, hkv)
    dev = to_dev(ring, cold)
    order = rng.permutation(slots)
    batches = synth.write_batches(rng, order, 16)
    for loc in batches:
        qsa.kv_store_tiered(x[loc].cuda(), y[loc].cuda(), torch.from_numpy(loc).cuda(), dev)
    ring, cold = write_history(x, y, batches, ring, cold)
    check_pool(dev, ring, cold, "device-written")
    lens = synth.quant_lengths_bs64(rng)
    sel, cu = synth.tiered_lists(rng, lens, slots, order[-r:], 0.3)
    q = synth.normal_bf16(rng, (64, 24, 256))
    decode_and_compare(q, dev, ring, cold, sel, cu, "device-written bs64")


def test_tiered_full_size_sampled_rows():
    """bs=128 rows of 2055 entries over a 262144-slot int4 pool with an
    8192-row ring, written in slot order (the ring then holds the last 8192
    slots), 25% of the entries drawn from them; the launch configuration of
    the tiered benchmark.  The oracle checks 12 sampled rows; only the slots
    those rows list are quantized on the host."""
    rng = np.random.default_rng(550)
    slots, hkv, r, bs = 262144, 2, 8192, 128
    order = np.arange(slots)
    sel, cu = synth.tiered_lists(rng, [2055] * bs, slots, order[-r:], 0.25)
    rows = sorted(rng.choice(bs, size=12, replace=False).tolist())
    need = np.unique(np.concatenate([sel[cu[b]:cu[b + 1]] for b in rows] + [order[-r:]]))
    say(f"[gpu] tiered full size: slots={slots} R={r}, {len(need)} slots checked")
    # token values: a seeded generator per block of slots, so any slot's
    # values can be made without the whole pool on the host
    x = torch.empty((slots, hkv, 256), dtype=torch.bfloat16)
    y = torch.empty((slots, hkv, 256), dtype=torch.bfloat16)
    blk = 16384
    for b0 in range(0, slots, blk):
        g = np.random.default_rng([551, b0])
        x[b0:b0 + blk] = synth.normal_bf16(g, (blk, hkv, 256))
        y[b0:b0 + blk] = synth.normal_bf16(g, (blk, hkv, 256))
    ring, cold = layout.empty_tiered(r, slots, hkv)
    dev = to_dev(ring, cold)
    for b0 in range(0, slots, 32768):
        loc = order[b0:b0 + 32768]
        qsa.kv_store_tiered(x[loc].cuda(), y[loc].cuda(), torch.from_numpy(loc).cuda(), dev)
    # host pools: int4 rows of the needed slots, the ring from the last R slots
    c4k, c4ks = quant.quantize_int4(x[need], 32, "f16")
    c4v, c4vs = quant.quantize_int4(y[need], 32, "f16")
    for name, a in zip(ARRAYS, (c4k, c4v, c4ks, c4vs)):
        cold[name][need] = a
    last = order[-r:]
    ring, cold = quant.store_tiered(x[last], y[last], last, ring, cold)
    check_pool(dev, ring, cold, "full size", slot_rows=need)
    q = synth.normal_bf16(rng, (bs, 24, 256))
    out, lse = decode_and_compare(q, dev, ring, cold, sel, cu, "bs128 tp1 full size", rows=rows)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()


def test_tiered_pools_beyond_32bit_offsets():
    """int4 pool rows 2^24 bytes apart (strided views into 4.4 GB buffers), so
    the two tiers cannot share a 32-bit offset range and the 64-bit address
    path is used; compared with the oracle on compact host copies."""
    rng = np.random.default_rng(560)
    slots, hkv, r = 260, 2, 64
    x = synth.normal_bf16(rng, (slots, hkv, 256))
    y = synth.normal_bf16(rng, (slots, hkv, 256))
    ring, cold = write_history(x, y, synth.write_batches(rng, rng.permutation(slots), 4),
                               *layout.empty_tiered(r, slots, hkv))
    dev = to_dev(ring, cold)
    stride = 1 << 24
    say(f"[gpu] tiered 64-bit addressing: slots={slots} int4 slot stride={stride} B")
    big = []
    for name in ("cold_k", "cold_v"):
        buf = torch.empty(slots * stride, dtype=torch.uint8, device="cuda")
        view = buf.as_strided((slots, hkv, 128), (stride, 128, 1))
        view.copy_(dev[name])
        dev[name] = view
        big.append(buf)
    sel, cu = synth.tiered_lists(rng, [2055, 700, 1, 0, 1500], slots, np.arange(slots), 0.3,
                                 dup_prob=0.05)
    q = synth.normal_bf16(rng, (5, 24, 256))
    decode_and_compare(q, dev, ring, cold, sel, cu, "64-bit addressing")
    del big, dev
    torch.cuda.empty_cache()


def test_tiered_graph_replay_matches_eager():
    """A captured graph of one tiered write (new tokens into the pool) plus
    one tiered decode, replayed with new tokens, slot ids, index lists and
    lengths copied into its buffers between replays; every replay's output
    and pool state equal those of the same calls made eagerly on a twin
    pool.  The pages call the tiered read graph-safe (no compactor, no
    unmapping mid-request)."""
    rng = np.random.default_rng(570)
    slots, hkv, r, bs, n_new = 8192, 2, 512, 8, 64
    x = synth.normal_bf16(rng, (slots, hkv, 256))
    y = synth.normal_bf16(rng, (slots, hkv, 256))
    order = rng.permutation(slots)
    ring, cold = write_history(x, y, synth.write_batches(rng, order[:4096], 4),
                               *layout.empty_tiered(r, slots, hkv))
    dev_g, dev_e = to_dev(ring, cold), to_dev(ring, cold)
    kbuf = torch.empty((n_new, hkv, 256), dtype=torch.bfloat16, device="cuda")
    vbuf = torch.empty_like(kbuf)
    locbuf = torch.empty(n_new, dtype=torch.int32, device="cuda")
    cap = bs * 2055
    selbuf = torch.zeros(cap, dtype=torch.int32, device="cuda")
    cubuf = torch.zeros(bs + 1, dtype=torch.int32, device="cuda")
    qbuf = synth.normal_bf16(rng, (bs, 24, 256)).cuda()
    out = torch.empty((bs, 24, 256), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((bs, 24), dtype=torch.float32, device="cuda")
    qsa.workspace_reserve(bs, 24, 2)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        qsa.kv_store_tiered(kbuf, vbuf, locbuf, dev_g)
        qsa.decode_tiered(qbuf, dev_g, selbuf, cubuf, out=out, lse=lse)

    written = 4096
    for rep in range(6):
        loc = order[written:written + n_new]
        written += n_new
        lens = rng.integers(0, 2056, size=bs)
        sel, cu = synth.tiered_lists(rng, lens, slots, order[written - r:written], 0.5)
        kbuf.copy_(x[loc])
        vbuf.copy_(y[loc])
        locbuf.copy_(torch.from_numpy(loc.astype(np.int32)))
        selbuf.zero_()
        selbuf[:sel.shape[0]].copy_(torch.from_numpy(sel))
        cubuf.copy_(torch.from_numpy(cu))
        g.replay()
        qsa.kv_store_tiered(kbuf, vbuf, locbuf, dev_e)
        oe, le = qsa.decode_tiered(qbuf, dev_e, selbuf, cubuf)
        torch.cuda.synchronize()
        say(f"  replay {rep}: n_sel={sel.shape[0]}")
        assert torch.equal(out.view(torch.int16), oe.view(torch.int16)), f"replay {rep}: out"
        assert torch.equal(lse.view(torch.int32), le.view(torch.int32)), f"replay {rep}: lse"
        for name in dev_g:
            assert torch.equal(dev_g[name].view(torch.uint8), dev_e[name].view(torch.uint8)), \
                f"replay {rep}: {name}"
        assert not dev_g["claim"].any().item()
    # the last replay against the oracle as well
    ring, cold = write_history(x, y, [order[4096:written]], ring, cold)
    o_ref, l_ref = oracle_tiered(qbuf.cpu(), ring, cold, sel, cu)
    compare(out, lse, o_ref, l_ref, np.diff(cu), label="graph replay")


def test_tiered_pool_descriptor_reused():
    """A TieredPool (the pool's descriptor built once) gives the dict form's
    results bit for bit: three rounds of a write then a decode, through each
    form on twin pools, and the twin pools end equal."""
    rng = np.random.default_rng(590)
    slots, hkv, r, bs, n_new = 4096, 2, 256, 6, 48
    x = synth.normal_bf16(rng, (slots, hkv, 256))
    y = synth.normal_bf16(rng, (slots, hkv, 256))
    order = rng.permutation(slots)
    ring, cold = write_history(x, y, synth.write_batches(rng, order[:2048], 3),
                               *layout.empty_tiered(r, slots, hkv))
    dev_a, dev_b = to_dev(ring, cold), to_dev(ring, cold)
    tp = qsa.TieredPool(dev_b)
    for step in range(3):
        loc = torch.from_numpy(rng.choice(slots, n_new, replace=False).astype(np.int32)).cuda()
        k_new = synth.normal_bf16(rng, (n_new, hkv, 256)).cuda()
        v_new = synth.normal_bf16(rng, (n_new, hkv, 256)).cuda()
        qsa.kv_store_tiered(k_new, v_new, loc, dev_a)
        qsa.kv_store_tiered(k_new, v_new, loc, tp)
        lens = [2055, 0, 700, 1, 2055, 64]
        sel, cu = synth.tiered_lists(rng, lens, slots, order[-r:], 0.3, dup_prob=0.05)
        q = synth.normal_bf16(rng, (bs, 12 * hkv, 256)).cuda()
        sel_d, cu_d = torch.from_numpy(sel).cuda(), torch.from_numpy(cu).cuda()
        oa, la = qsa.decode_tiered(q, dev_a, sel_d, cu_d)
        ob, lb = qsa.decode_tiered(q, tp, sel_d, cu_d)
        torch.cuda.synchronize()
        assert torch.equal(oa, ob) and torch.equal(la, lb), f"round {step}: outputs differ"
    for name in dev_a:
        assert torch.equal(dev_a[name], dev_b[name]), f"pool array {name} differs"
    assert all(v == 0 for v in qsa.debug_counters())
