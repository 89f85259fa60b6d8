"""Parity of the HIP indexer step (qsa_index) with the oracle, through the C ABI.

Pages: "[Kernel][WIP] Integrate native FlashInfer SM70 batch GDN and QSA
probes", follow-up "device-planned MQA and QSA quality attribution" (MQA
scoring + exact top-k + index expansion, 256K-token capacity, measured at
8K tokens for 4 / 8 / 16 concurrent rows), and "feat(qsa): quantized KV
pools with dequant-on-gather (fp8/int8/int4)", part 4 decode routing
paragraph (row width token_topk + compress_ratio - 1).  The lists are
integer results, so the GPU's sel and cu must equal the oracle's exactly:
both sides evaluate the block scores in the same fp32 order and take the
same top-k decisions.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from qsa_testlib import compare, oracle_threads, say

import sparse_index_paged_amd as qsa

pytestmark = pytest.mark.gpu


def to_dev(inp):
    d = dict(q=inp["q"].cuda(), k=inp["k_pool"].cuda(),
             bt=torch.from_numpy(inp["block_table"]).cuda(),
             r2t=torch.from_numpy(inp["req_to_token"]).cuda(),
             ctx=torch.from_numpy(inp["ctx_len"]).cuda())
    d["w"] = torch.from_numpy(inp["weights"]).cuda() if inp["weights"] is not None else None
    return d


def gpu_index(d, budget, c):
    sel, cu = qsa.index(d["q"], d["k"], d["bt"], d["r2t"], d["ctx"], budget=budget,
                        compress_ratio=c, head_weights=d["w"])
    torch.cuda.synchronize()
    return sel, cu


def check(inp, budget, c, label):
    ctx = inp["ctx_len"]
    say(f"[gpu] index {label}: bs={len(ctx)} hi={inp['q'].shape[1]} di={inp['q'].shape[2]} "
        f"c={c} budget={budget} ctx max {int(ctx.max())}")
    d = to_dev(inp)
    sel, cu = gpu_index(d, budget, c)
    ref_sel, ref_cu = oracle.index(inp["q"], inp["k_pool"], inp["block_table"],
                                   inp["req_to_token"], ctx, budget=budget, compress_ratio=c,
                                   weights=inp["weights"])
    got_cu = cu.cpu().numpy()
    np.testing.assert_array_equal(got_cu, ref_cu, err_msg=f"{label}: cu")
    np.testing.assert_array_equal(sel[: ref_cu[-1]].cpu().numpy(), ref_sel, err_msg=f"{label}: sel")
    return sel, cu


@pytest.mark.parametrize("bs", [4, 8, 16])
@pytest.mark.parametrize("c", [4, 8])
def test_eight_k_contexts(bs, c):
    """The pages' measured setting: 8K-token contexts at 4 / 8 / 16 rows,
    budget 2048 (rows of 2051 and 2055 entries)."""
    rng = np.random.default_rng(700 + bs + c)
    ctx = rng.integers(8192 - 64, 8192 + 64, size=bs)
    inp = synth.index_inputs(rng, ctx, hi=16, di=128, c=c)
    check(inp, 2048, c, f"8K ctx bs{bs} c{c}")


@pytest.mark.parametrize("hi,di,c,budget,weights", [(1, 64, 16, 512, True), (64, 128, 4, 2048, True),
                                                     (4, 64, 1, 1024, False), (7, 128, 2, 256, True)])
def test_shapes_and_mixed_lengths(hi, di, c, budget, weights):
    """Lengths 0, below c, exact block multiples, just past the budget and
    well past it, in one call."""
    rng = np.random.default_rng(710 + hi + c)
    ctx = [0, c - 1, c, budget, budget + c - 1, budget + c, 3 * budget + 1, 20000, 1, budget * 8]
    inp = synth.index_inputs(rng, ctx, hi=hi, di=di, c=c, weights=weights)
    check(inp, budget, c, f"mixed hi{hi} di{di} c{c} budget{budget}")


def test_ties_and_constant_scores():
    """Every key equal (all scores tie) in one row; keys drawn from 3 values
    in another (many ties at the threshold)."""
    rng = np.random.default_rng(720)
    inp = synth.index_inputs(rng, [9000, 9000, 9000], hi=4, di=64, c=4)
    k = inp["k_pool"]
    bt = inp["block_table"]
    k[bt[0]] = k[bt[0, 0]].clone()
    three = k[:3].clone()
    k[bt[1]] = three[torch.from_numpy(rng.integers(0, 3, bt.shape[1]))]
    inp["q"][2] = 0.0                                          # row 2: every score is 0
    check(inp, 2048, 4, "ties")


def test_full_capacity_rows():
    """Rows at the 256K-token capacity (65,536 blocks at c = 4)."""
    rng = np.random.default_rng(730)
    ctx = [262144, 262143, 100000]
    inp = synth.index_inputs(rng, ctx, hi=4, di=64, c=4, slots=1 << 24)
    check(inp, 2048, 4, "256K capacity")


def test_index_feeds_the_decode():
    """The indexer's lists decode on the device to the oracle's result for
    the oracle's lists (the two steps chained, bs=16 TP1)."""
    rng = np.random.default_rng(740)
    ctx = rng.integers(3000, 9000, size=16)
    slots = 65536
    inp = synth.index_inputs(rng, ctx, hi=8, di=128, c=4, slots=slots)
    d = to_dev(inp)
    sel, cu = check(inp, 2048, 4, "index -> decode")
    kv = synth.normal_bf16(rng, (slots, 2, 256))
    vv = synth.normal_bf16(rng, (slots, 2, 256))
    q = synth.normal_bf16(rng, (16, 24, 256))
    out, lse = qsa.decode(q.cuda(), kv.cuda(), vv.cuda(), sel, cu)
    torch.cuda.synchronize()
    ref_sel, ref_cu = oracle.index(inp["q"], inp["k_pool"], inp["block_table"], inp["req_to_token"],
                                   inp["ctx_len"], budget=2048, compress_ratio=4,
                                   weights=inp["weights"])
    o_ref, l_ref = oracle.decode(q, kv, vv, ref_sel, ref_cu, nthreads=oracle_threads())
    compare(out, lse, o_ref, l_ref, np.diff(ref_cu), label="index -> decode")


def test_bad_rows_list_nothing_and_are_reported():
    rng = np.random.default_rng(750)
    inp = synth.index_inputs(rng, [5000, 5000, 5000, 5000], hi=4, di=64, c=4, max_tokens=6000)
    d = to_dev(inp)
    d["ctx"] = torch.tensor([5000, -1, 7000, 4000], dtype=torch.int32, device="cuda")
    qsa.workspace_reset()
    sel, cu = gpu_index(d, 1024, 4)
    assert qsa.debug_device_error() == 8
    cu_h = cu.cpu().numpy()
    assert cu_h[2] - cu_h[1] == 0 and cu_h[3] - cu_h[2] == 0
    ok = [0, 3]
    ref_sel, ref_cu = oracle.index(inp["q"][ok], inp["k_pool"], inp["block_table"][ok],
                                   inp["req_to_token"][ok], np.array([5000, 4000], np.int32),
                                   budget=1024, compress_ratio=4, weights=inp["weights"][ok])
    got = sel.cpu().numpy()
    np.testing.assert_array_equal(got[cu_h[0]:cu_h[1]], ref_sel[ref_cu[0]:ref_cu[1]])
    np.testing.assert_array_equal(got[cu_h[3]:cu_h[4]], ref_sel[ref_cu[1]:ref_cu[2]])
    qsa.workspace_reset()
    assert qsa.debug_device_error() == 0


def test_graph_replay_with_changing_lengths():
    """Indexer + decode captured in one graph; context lengths, queries and
    keys change on the device between replays; every replay's lists equal
    the oracle's and the decode output equals an eager call's bitwise."""
    rng = np.random.default_rng(760)
    bs, slots = 8, 32768
    max_tokens = 12000
    inp = synth.index_inputs(rng, [max_tokens] * bs, hi=8, di=128, c=4, slots=slots)
    d = to_dev(inp)
    kv = synth.normal_bf16(rng, (slots, 2, 256)).cuda()
    vv = synth.normal_bf16(rng, (slots, 2, 256)).cuda()
    qd = synth.normal_bf16(rng, (bs, 24, 256)).cuda()
    sel = torch.empty(bs * 2051, dtype=torch.int32, device="cuda")
    cu = torch.empty(bs + 1, dtype=torch.int32, device="cuda")
    out = torch.empty(bs, 24, 256, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(bs, 24, dtype=torch.float32, device="cuda")
    qsa.index_reserve(bs, d["bt"].shape[1])
    qsa.workspace_reserve(bs, 24, 2)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        qsa.index(d["q"], d["k"], d["bt"], d["r2t"], d["ctx"], budget=2048, compress_ratio=4,
                  head_weights=d["w"], sel_out=sel, cu_out=cu)
        qsa.decode(qd, kv, vv, sel, cu, out=out, lse=lse)
    for rep in range(5):
        ctx = rng.integers(0, max_tokens + 1, size=bs).astype(np.int32)
        newq = synth.normal_bf16(rng, tuple(d["q"].shape))
        d["ctx"].copy_(torch.from_numpy(ctx))
        d["q"].copy_(newq)
        g.replay()
        torch.cuda.synchronize()
        ref_sel, ref_cu = oracle.index(newq, inp["k_pool"], inp["block_table"], inp["req_to_token"],
                                       ctx, budget=2048, compress_ratio=4, weights=inp["weights"])
        np.testing.assert_array_equal(cu.cpu().numpy(), ref_cu, err_msg=f"replay {rep}: cu")
        np.testing.assert_array_equal(sel[: ref_cu[-1]].cpu().numpy(), ref_sel, err_msg=f"replay {rep}: sel")
        oe, le = qsa.decode(qd, kv, vv, sel, cu)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), oe.view(torch.int16)), f"replay {rep}"
        assert torch.equal(lse.view(torch.int32), le.view(torch.int32)), f"replay {rep}"
        say(f"  replay {rep}: lists {int(ref_cu[-1])} entries")


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_outputs_are_bitwise_invariant_under_kv_relocation(fmt):
    """Moving every token's K/V to other physical slots (a relocation, with
    req_to_token rewritten to match) leaves indexer + decode outputs bitwise
    unchanged: the lists come out in logical order and the decode's
    arithmetic depends only on list order and the K/V values -- the
    property the pages' canonical-order planner restores for their path
    (page "[Kernel][WIP] Integrate native FlashInfer SM70 batch GDN and QSA
    probes", follow-up "stable planning": twelve physical relocations
    bitwise identical)."""
    rng = np.random.default_rng(770)
    bs, slots = 16, 65536
    ctx = rng.integers(2000, 12000, size=bs)
    inp = synth.index_inputs(rng, ctx, hi=8, di=128, c=4, slots=slots)
    k_log = synth.normal_bf16(rng, (slots, 2, 256))       # K/V by the slot ids of req_to_token
    v_log = synth.normal_bf16(rng, (slots, 2, 256))
    q = synth.normal_bf16(rng, (bs, 24, 256)).cuda()
    outs = []
    for reloc in range(3):
        perm = np.arange(slots) if reloc == 0 else rng.permutation(slots)   # old slot -> new slot
        kp = torch.empty_like(k_log)
        vp = torch.empty_like(v_log)
        kp[torch.from_numpy(perm)] = k_log
        vp[torch.from_numpy(perm)] = v_log
        d = to_dev(dict(inp, req_to_token=perm[inp["req_to_token"]].astype(np.int32)))
        sel, cu = gpu_index(d, 2048, 4)
        kw = {}
        kd, vd = kp.cuda(), vp.cuda()
        if fmt == "fp8":
            kc = torch.empty((slots, 2, 256), dtype=torch.uint8, device="cuda")
            vc = torch.empty_like(kc)
            ks = torch.empty((slots, 2, 1), dtype=torch.float32, device="cuda")
            vs = torch.empty_like(ks)
            qsa.kv_store(kd, vd, torch.arange(slots, dtype=torch.int32, device="cuda"), kc, vc,
                         kv_format="fp8", k_scale=ks, v_scale=vs)
            kd, vd = kc, vc
            kw = dict(kv_format="fp8", k_scale=ks, v_scale=vs)
        out, lse = qsa.decode(q, kd, vd, sel, cu, **kw)
        torch.cuda.synchronize()
        say(f"  {fmt} relocation {reloc}: {int(cu[-1])} entries")
        outs.append((out.clone(), lse.clone()))
    for o, l in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0][0].view(torch.int16))
        assert torch.equal(l.view(torch.int32), outs[0][1].view(torch.int32))
