"""Concurrent streams with private workspaces, through the C ABI.

The pages keep scratch local to the call instead of sharing it between
callers (page "[Kernel][WIP] Integrate native FlashInfer SM70 batch GDN and
QSA probes", change summary).  Here a stream given its own workspace
(qsa_workspace_attach) holds its own split partials, split counters, error
word and indexer scores, so indexer + decode pipelines on two streams can run
at the same time.  Each stream's results must equal, bit for bit, what the
same calls give when run alone (the decode and the indexer are
deterministic), and every workspace's counters must be at rest after each of
its calls even while the other stream's kernels are in flight.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from qsa_testlib import compare, oracle_rows, say, to_device

import sparse_index_paged_amd as qsa

pytestmark = pytest.mark.gpu

BUDGET, C = 2048, 4


@pytest.fixture
def streams():
    s = [torch.cuda.Stream(), torch.cuda.Stream()]
    yield s
    torch.cuda.synchronize()
    for st in s:
        qsa.workspace_detach(st)


class Lane:
    """One indexer + decode pipeline with its own inputs and outputs."""

    def __init__(self, seed, bs, ctx_max, hkv):
        rng = np.random.default_rng(seed)
        slots = 32768
        self.bs, self.hkv, self.hq = bs, hkv, 12 * hkv
        ctx = rng.integers(ctx_max // 2, ctx_max + 1, size=bs)
        self.inp = synth.index_inputs(rng, ctx, hi=8, di=128, c=C, slots=slots)
        i = self.inp
        self.q_i = i["q"].cuda()
        self.k_i = i["k_pool"].cuda()
        self.bt = torch.from_numpy(i["block_table"]).cuda()
        self.r2t = torch.from_numpy(i["req_to_token"]).cuda()
        self.ctx = torch.from_numpy(i["ctx_len"]).cuda()
        self.w = torch.from_numpy(i["weights"]).cuda()
        self.k_host = synth.normal_bf16(rng, (slots, hkv, 256))
        self.v_host = synth.normal_bf16(rng, (slots, hkv, 256))
        self.q_host = synth.normal_bf16(rng, (bs, self.hq, 256))
        self.k, self.v, self.q = self.k_host.cuda(), self.v_host.cuda(), self.q_host.cuda()
        self.sel = torch.empty(bs * (BUDGET + C - 1), dtype=torch.int32, device="cuda")
        self.cu = torch.empty(bs + 1, dtype=torch.int32, device="cuda")
        self.out = torch.empty(bs, self.hq, 256, dtype=torch.bfloat16, device="cuda")
        self.lse = torch.empty(bs, self.hq, dtype=torch.float32, device="cuda")
        self.audit = torch.zeros(1, dtype=torch.int32, device="cuda")

    def reserve(self, stream):
        qsa.workspace_reserve(self.bs, self.hq, self.hkv, stream=stream)
        qsa.index_reserve(self.bs, self.bt.shape[1], stream=stream)

    def enqueue(self, stream, audit=True):
        qsa.index(self.q_i, self.k_i, self.bt, self.r2t, self.ctx, budget=BUDGET, compress_ratio=C,
                  head_weights=self.w, sel_out=self.sel, cu_out=self.cu, stream=stream)
        qsa.decode(self.q, self.k, self.v, self.sel, self.cu, out=self.out, lse=self.lse,
                   stream=stream)
        if audit:
            qsa.debug_audit_counters(self.audit, stream=stream)

    def snapshot(self):
        return [t.clone() for t in (self.sel, self.cu, self.out, self.lse)]

    def check_oracle(self, label):
        ref_sel, ref_cu = oracle.index(self.inp["q"], self.inp["k_pool"], self.inp["block_table"],
                                       self.inp["req_to_token"], self.inp["ctx_len"], budget=BUDGET,
                                       compress_ratio=C, weights=self.inp["weights"])
        np.testing.assert_array_equal(self.cu.cpu().numpy(), ref_cu, err_msg=f"{label}: cu")
        np.testing.assert_array_equal(self.sel[: ref_cu[-1]].cpu().numpy(), ref_sel,
                                      err_msg=f"{label}: sel")
        o_ref, l_ref = oracle_rows(self.q_host, self.k_host, self.v_host, ref_sel, ref_cu)
        compare(self.out, self.lse, o_ref, l_ref, np.diff(ref_cu), label=label)

    def same_as(self, snap, label):
        sel, cu, out, lse = snap
        assert torch.equal(self.cu, cu), f"{label}: cu"
        n = int(cu[-1])
        assert torch.equal(self.sel[:n], sel[:n]), f"{label}: sel"
        assert torch.equal(self.out.view(torch.int16), out.view(torch.int16)), f"{label}: out"
        assert torch.equal(self.lse.view(torch.int32), lse.view(torch.int32)), f"{label}: lse"


def gate(streams, cycles=20_000_000):
    """Hold every stream until a spin kernel on a third stream ends, so that
    the work enqueued next on each stream is queued together and overlaps."""
    g = torch.cuda.Stream()
    with torch.cuda.stream(g):
        torch.cuda._sleep(cycles)
        ev = torch.cuda.Event()
        ev.record(g)
    for s in streams:
        s.wait_event(ev)


def test_two_streams_run_concurrently_with_private_workspaces(streams):
    sa, sb = streams
    for s in streams:
        qsa.workspace_attach(s)
    qsa.workspace_attach(sa)                      # attaching twice does nothing
    lanes = [Lane(901, 8, 12000, 2), Lane(902, 6, 9000, 1)]
    for lane, s in zip(lanes, streams):
        lane.reserve(s)
    torch.cuda.synchronize()
    assert qsa.workspace_bytes() > 0

    refs = []
    for k, (lane, s) in enumerate(zip(lanes, streams)):  # each lane alone
        lane.enqueue(s)
        s.synchronize()
        lane.check_oracle(f"lane {k} alone")
        refs.append(lane.snapshot())
        say(f"  lane {k}: bs={lane.bs} hkv={lane.hkv} plan={qsa.plan(lane.bs, lane.hkv)}")

    iters = 40
    gate(streams)
    for _ in range(iters):
        for lane, s in zip(lanes, streams):
            lane.enqueue(s)
    torch.cuda.synchronize()
    for k, (lane, s) in enumerate(zip(lanes, streams)):
        assert lane.audit.item() == 0, f"lane {k}: counters seen away from rest"
        assert all(v == 0 for v in qsa.debug_counters(stream=s))
        assert qsa.debug_device_error(stream=s) == 0
        lane.same_as(refs[k], f"lane {k} after {iters} concurrent pipelines")
    say(f"  {iters} x 2 concurrent pipelines bitwise equal to the lone runs")


def test_graphs_captured_on_attached_streams_replay_concurrently(streams):
    """Each pipeline captured once on its own attached, reserved stream; the
    two graphs are replayed at the same time, again and again."""
    lanes = [Lane(911, 8, 12000, 2), Lane(912, 4, 12000, 2)]
    for lane, s in zip(lanes, streams):
        qsa.workspace_attach(s)
        lane.reserve(s)
    torch.cuda.synchronize()
    refs = []
    for lane, s in zip(lanes, streams):
        lane.enqueue(s)
        s.synchronize()
        refs.append(lane.snapshot())
    graphs = []
    for lane, s in zip(lanes, streams):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            lane.enqueue(s)
        graphs.append(g)
    torch.cuda.synchronize()
    for rep in range(3):
        gate(streams)
        for _ in range(10):
            for g, s in zip(graphs, streams):
                with torch.cuda.stream(s):
                    g.replay()
        torch.cuda.synchronize()
        for k, lane in enumerate(lanes):
            assert lane.audit.item() == 0, f"lane {k}: counters seen away from rest"
            lane.same_as(refs[k], f"lane {k} replay round {rep}")
    lanes[0].check_oracle("lane 0 after replays")
    say("  30 concurrent replays of each graph bitwise equal to eager runs")


def test_error_words_are_per_workspace(streams):
    sa, sb = streams
    qsa.workspace_attach(sa)
    case = synth.make_case(lengths=[30, 2056, 30], slots=1000, hkv=1, seed=931)
    d = to_device(case)
    qsa.workspace_reset(stream=sa)
    qsa.workspace_reset()                          # the shared workspace (current stream)
    out, lse = qsa.decode(d["q"], d["k"], d["v"], d["sel"], d["cu"], stream=sa)
    assert qsa.debug_device_error(stream=sa) == 1
    assert qsa.debug_device_error() == 0          # sb and the current stream use the shared one
    assert qsa.debug_device_error(stream=sb) == 0
    assert torch.isnan(out[1].float()).all()
    good = [0, 2]
    o_ref, l_ref = oracle_rows(case.q, case.k_pool, case.v_pool, case.sel, case.cu, good)
    compare(out[good], lse[good], o_ref, l_ref, case.lengths[good], label="good rows on sa")
    qsa.workspace_reset(stream=sa)
    assert qsa.debug_device_error(stream=sa) == 0


def test_detach_returns_a_stream_to_the_shared_workspace(streams):
    sa, _ = streams
    case = synth.make_case(lengths=[2055] * 6, slots=4096, hkv=2, seed=941, dup_prob=0.05)
    d = to_device(case)
    qsa.decode(d["q"], d["k"], d["v"], d["sel"], d["cu"])   # shared workspace exists
    torch.cuda.synchronize()
    shared = qsa.workspace_bytes()
    qsa.workspace_attach(sa)
    assert qsa.workspace_bytes() == shared        # a private workspace starts empty
    out, lse = qsa.decode(d["q"], d["k"], d["v"], d["sel"], d["cu"], stream=sa)
    sa.synchronize()
    private = qsa.workspace_bytes() - shared
    assert private > 0
    o_ref, l_ref = oracle_rows(case.q, case.k_pool, case.v_pool, case.sel, case.cu)
    compare(out, lse, o_ref, l_ref, case.lengths, label="private workspace")
    first = (out.clone(), lse.clone())
    qsa.workspace_detach(sa)
    assert qsa.workspace_bytes() == shared
    qsa.workspace_detach(sa)                      # detaching a detached stream does nothing
    out2, lse2 = qsa.decode(d["q"], d["k"], d["v"], d["sel"], d["cu"], stream=sa)
    sa.synchronize()
    assert torch.equal(out2.view(torch.int16), first[0].view(torch.int16))
    assert torch.equal(lse2.view(torch.int32), first[1].view(torch.int32))
    assert all(v == 0 for v in qsa.debug_counters(stream=sa))
    assert qsa.workspace_bytes() == shared
