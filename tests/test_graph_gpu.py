"""hipGraph capture / replay with cu_seqlens and indices rewritten on the
device between replays, and the split counters audited after every replay.

Page "fix(qsa): restore SM121 correctness with Humanize and Kernel Design
Agent": lengths are read live on the device so a captured graph replays
with changed cu_seqlens without host readback (section "Changes"), a
zero-length row included (kernel-in-isolation comment); counters return to
zero after every launch (section "Optimized kernel").  Sweep: every bs
1..16 plus 17/24/32/48/64/96/128, short / medium / saturated lists with
duplicate runs, two of the eight banks with zero-length rows (one of them
an all-empty call at bs = 1), 24Q/2KV and 12Q/1KV.
"""
import numpy as np
import pytest
import torch

import synth
from qsa_testlib import compare, oracle_rows, say

import sparse_index_paged_amd as qsa

pytestmark = pytest.mark.gpu

REPLAYS = 1000
SLOTS = 32768
BANKS = 8


@pytest.fixture(scope="module")
def pools():
    rng = np.random.default_rng(1049)
    out = {}
    for hkv in (2, 1):
        k = synth.normal_bf16(rng, (SLOTS, hkv, 256))
        v = synth.normal_bf16(rng, (SLOTS, hkv, 256))
        out[hkv] = (k, v, k.cuda(), v.cuda())
    qsa.workspace_reserve(128, 24, 2)
    return out


def _sweep_point(pools, hkv, kind, bs, replays, oracle_banks, oracle_rows_per_bank):
    k, v, kd, vd = pools[hkv]
    hq = 12 * hkv
    banks = synth.sweep_bank(1050 + bs, bs, kind, SLOTS, banks=BANKS)
    cap = banks[0][0].shape[0]
    sel_banks = torch.stack([torch.from_numpy(s) for s, _ in banks]).cuda()
    cu_banks = torch.stack([torch.from_numpy(c) for _, c in banks]).cuda()
    rng = np.random.default_rng(bs * 7 + hkv)
    q_host = synth.normal_bf16(rng, (bs, hq, 256))
    q = q_host.cuda()
    sel_buf = sel_banks[0].clone()
    cu_buf = cu_banks[0].clone()
    out = torch.empty(bs, hq, 256, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(bs, hq, dtype=torch.float32, device="cuda")

    # eager reference of every bank (separate output buffers)
    ref_o, ref_l = [], []
    for b in range(BANKS):
        o, l = qsa.decode(q, kd, vd, sel_banks[b], cu_banks[b])
        ref_o.append(o)
        ref_l.append(l)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        qsa.decode(q, kd, vd, sel_buf, cu_buf, out=out, lse=lse)

    audit = torch.zeros(1, dtype=torch.int32, device="cuda")
    mism = torch.zeros(1, dtype=torch.int64, device="cuda")
    for r in range(replays):
        b = r % BANKS
        sel_buf.copy_(sel_banks[b])
        cu_buf.copy_(cu_banks[b])
        g.replay()
        qsa.debug_audit_counters(audit)
        mism += (out != ref_o[b]).sum() + (lse != ref_l[b]).sum()
        if r % 250 == 249:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    assert audit.item() == 0, f"split counters not at rest: {audit.item()}"
    assert mism.item() == 0, f"replays differ from eager results in {mism.item()} values"

    # eager results against the oracle (sampled rows for large batches):
    # bank 0 and bank 3, which holds zero-length rows; those rows are
    # always among the checked ones
    for b in oracle_banks:
        sel_np, cu_np = banks[b]
        rows = list(range(bs)) if bs <= oracle_rows_per_bank else sorted(set(
            np.random.default_rng(b).choice(bs, oracle_rows_per_bank, replace=False).tolist())
            | set(synth.sweep_empty_rows(b, bs)))
        assert all(np.diff(cu_np)[j] == 0 for j in synth.sweep_empty_rows(b, bs))
        o_ref, l_ref = oracle_rows(q_host, k, v, sel_np, cu_np, rows)
        lens = np.diff(cu_np)[rows]
        compare(ref_o[b][rows], ref_l[b][rows], o_ref, l_ref, lens,
                label=f"hkv{hkv} {kind} bs{bs} bank{b}")
    del g


@pytest.mark.parametrize("hkv", [2, 1])
@pytest.mark.parametrize("kind", ["short", "medium", "saturated"])
def test_graph_replay_sweep(pools, hkv, kind):
    for bs in synth.SWEEP_BS:
        say(f"[gpu] graph sweep hkv={hkv} kind={kind} bs={bs} replays={REPLAYS}")
        _sweep_point(pools, hkv, kind, bs, REPLAYS, oracle_banks=(0, 3), oracle_rows_per_bank=4)


def test_capture_without_reserved_workspace_is_rejected(pools):
    """Under capture the library never allocates: too small a workspace is
    a QSA_ERR_WORKSPACE error, detected on the host before any launch."""
    k, v, kd, vd = pools[2]
    qsa.set_option("split_target", 1 << 20)
    qsa.set_option("max_splits", 64)
    try:
        q = torch.zeros(128, 24, 256, dtype=torch.bfloat16, device="cuda")
        sel = torch.zeros(128, dtype=torch.int32, device="cuda")
        cu = torch.arange(129, dtype=torch.int32, device="cuda")
        g = torch.cuda.CUDAGraph()
        with pytest.raises(qsa.QsaError, match="capturing"):
            with torch.cuda.graph(g):
                qsa.decode(q, kd, vd, sel, cu)
    finally:
        qsa.set_option("split_target", 0)
        qsa.set_option("max_splits", 16)
    torch.cuda.synchronize()


def test_replay_after_workspace_growth(pools):
    """Growing the shared workspace after a capture keeps the buffers the
    captured call uses: the counters (and error word) never move, the old
    partials stay allocated, so the graph still replays equal to eager calls
    and the sticky error bit set before the growth survives it."""
    k, v, kd, vd = pools[2]
    qsa.workspace_release()
    try:
        qsa.workspace_reserve(4, 24, 2)
        splits = qsa.plan(4, 2)[0]
        assert splits > 1, "bs=4 must split for the test to use partials"
        ptr0, n0 = qsa.debug_counter_ptr()
        bytes0 = qsa.workspace_bytes()
        # set the sticky row-range bit with a row longer than 2055
        bad_q = torch.zeros(1, 24, 256, dtype=torch.bfloat16, device="cuda")
        bad_sel = torch.zeros(3000, dtype=torch.int32, device="cuda")
        bad_cu = torch.tensor([0, 3000], dtype=torch.int32, device="cuda")
        qsa.decode(bad_q, kd, vd, bad_sel, bad_cu)
        torch.cuda.synchronize()
        assert qsa.debug_device_error() & 1

        banks = synth.sweep_bank(4242, 4, "saturated", SLOTS, banks=BANKS)
        sel_banks = [torch.from_numpy(s_).cuda() for s_, _ in banks]
        cu_banks = [torch.from_numpy(c_).cuda() for _, c_ in banks]
        q = synth.normal_bf16(np.random.default_rng(77), (4, 24, 256)).cuda()
        sel_buf, cu_buf = sel_banks[0].clone(), cu_banks[0].clone()
        out = torch.empty(4, 24, 256, dtype=torch.bfloat16, device="cuda")
        lse = torch.empty(4, 24, dtype=torch.float32, device="cuda")
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            qsa.decode(q, kd, vd, sel_buf, cu_buf, out=out, lse=lse)

        # grow: an eager bs=128 call and a larger reservation
        big = synth.sweep_bank(4243, 128, "saturated", SLOTS, banks=1)[0]
        qbig = torch.zeros(128, 24, 256, dtype=torch.bfloat16, device="cuda")
        qsa.decode(qbig, kd, vd, torch.from_numpy(big[0]).cuda(), torch.from_numpy(big[1]).cuda())
        qsa.set_option("splits", 9)
        try:
            qsa.decode(qbig, kd, vd, torch.from_numpy(big[0]).cuda(), torch.from_numpy(big[1]).cuda())
        finally:
            qsa.set_option("splits", 0)
        torch.cuda.synchronize()
        assert qsa.workspace_bytes() > bytes0, "the workspace did not grow"
        assert qsa.debug_counter_ptr() == (ptr0, n0), "the counters moved when the workspace grew"
        assert qsa.debug_device_error() & 1, "the sticky error bit was lost when the workspace grew"

        audit = torch.zeros(1, dtype=torch.int32, device="cuda")
        for r in range(40):
            b = r % BANKS
            sel_buf.copy_(sel_banks[b])
            cu_buf.copy_(cu_banks[b])
            g.replay()
            qsa.debug_audit_counters(audit)
            ref_o, ref_l = qsa.decode(q, kd, vd, sel_banks[b], cu_banks[b])
            assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"replay {r} differs"
        torch.cuda.synchronize()
        assert audit.item() == 0
        o_ref, l_ref = oracle_rows(q.cpu(), k, v, banks[0][0], banks[0][1])
        sel_buf.copy_(sel_banks[0])
        cu_buf.copy_(cu_banks[0])
        g.replay()
        torch.cuda.synchronize()
        compare(out, lse, o_ref, l_ref, np.diff(banks[0][1]), label="replay after growth")
        del g
    finally:
        qsa.workspace_reset()
        torch.cuda.synchronize()
        qsa.workspace_release()
        qsa.workspace_reserve(128, 24, 2)
