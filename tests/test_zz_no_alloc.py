"""qsa_decode_noalloc, the entry point for callers that cannot allocate:
its outputs equal qsa_decode's, call after call, with the split scratch in
the library's fixed per-device array.

Checked through the C ABI (ctypes binding) on two calls in a row, the
second with a smaller input; against the oracle at the decode's parity bar
(rel-L2 <= 2e-3, |dlse| <= 1e-3, per-head floors) and bitwise against
qsa_decode on the same inputs; with no library workspace created; under
graph capture with changed device-side lengths; and a plan larger than the
scratch refused on the host.
"""
import numpy as np
import pytest
import torch

import synth
from qsa_testlib import compare, oracle_rows, say, to_device

import sparse_index_paged_amd as qsa

pytestmark = pytest.mark.gpu


def _run_both(case, label):
    d = to_device(case)
    out_n = torch.full((case.bs, case.hq, 256), 7.0, dtype=torch.bfloat16, device="cuda")
    lse_n = torch.full((case.bs, case.hq), 7.0, dtype=torch.float32, device="cuda")
    qsa.decode_noalloc(d["q"], d["k"], d["v"], d["sel"], d["cu"], out=out_n, lse=lse_n)
    out_w, lse_w = qsa.decode(d["q"], d["k"], d["v"], d["sel"], d["cu"])
    torch.cuda.synchronize()
    say(f"[gpu] no-alloc {label}: bs={case.bs} hkv={case.hkv} plan={qsa.plan(case.bs, case.hkv)}")
    assert torch.equal(out_n, out_w), f"{label}: out differs from qsa_decode"
    assert torch.equal(lse_n, lse_w), f"{label}: lse differs from qsa_decode"
    o_ref, l_ref = oracle_rows(case.q, case.k_pool, case.v_pool, case.sel, case.cu)
    compare(out_n, lse_n, o_ref, l_ref, case.lengths, label=f"no-alloc {label}")


def test_two_calls_match_decode_and_oracle():
    """Two calls in a row, the second smaller; both split (so the scratch's
    partials and counters are used), then the first size again."""
    qsa.workspace_release()
    a = synth.make_case(lengths=[2055, 1500, 0, 700, 2055, 64, 2055, 1999, 300, 2055, 17, 2055, 900,
                                 2055, 1, 2048], slots=8192, hkv=2, seed=71, dup_prob=0.1)
    b = synth.make_case(lengths=[2055, 0, 333, 1024], slots=8192, hkv=1, seed=72, dup_prob=0.1)
    assert qsa.plan(a.bs, a.hkv)[0] > 1 and qsa.plan(b.bs, b.hkv)[0] > 1
    d = to_device(a)
    out = torch.empty(a.bs, a.hq, 256, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(a.bs, a.hq, dtype=torch.float32, device="cuda")
    qsa.decode_noalloc(d["q"], d["k"], d["v"], d["sel"], d["cu"], out=out, lse=lse)
    torch.cuda.synchronize()
    assert qsa.workspace_bytes() == 0, "the no-alloc call created a library workspace"
    _run_both(a, "first call (bs 16, TP1)")
    _run_both(b, "second call (bs 4, TP2, smaller)")
    _run_both(a, "first size again")


def test_many_calls_and_quantized_pools():
    """Alternating sizes over many calls keep matching qsa_decode bitwise
    (a counter left non-zero would break the last-split detection), also
    for an int4 pool."""
    cases = [synth.make_case(lengths=[2055] * n, slots=4096, hkv=h, seed=80 + n, dup_prob=0.05)
             for n, h in ((8, 2), (3, 1), (32, 2), (1, 2))]
    devs = [to_device(c) for c in cases]
    refs = [qsa.decode(d["q"], d["k"], d["v"], d["sel"], d["cu"]) for d in devs]
    outs = [(torch.empty_like(o), torch.empty_like(l)) for o, l in refs]
    for r in range(200):
        i = r % len(cases)
        d = devs[i]
        qsa.decode_noalloc(d["q"], d["k"], d["v"], d["sel"], d["cu"], out=outs[i][0], lse=outs[i][1])
        if i == len(cases) - 1:
            torch.cuda.synchronize()
            for (o, l), (ro, rl) in zip(outs, refs):
                assert torch.equal(o, ro) and torch.equal(l, rl), f"call {r}: differs from qsa_decode"
    # int4 pool, 32-channel f32 scales
    import oracle
    c = cases[0]
    kc, ks = oracle.quant.quantize_int4(c.k_pool, 32)
    vc, vs = oracle.quant.quantize_int4(c.v_pool, 32)
    d = devs[0]
    kw = dict(kv_format="int4", k_scale=torch.from_numpy(ks).cuda(), v_scale=torch.from_numpy(vs).cuda(),
              group_size=32)
    kcd, vcd = torch.from_numpy(kc).cuda(), torch.from_numpy(vc).cuda()
    ro, rl = qsa.decode(d["q"], kcd, vcd, d["sel"], d["cu"], **kw)
    o, l = torch.empty_like(ro), torch.empty_like(rl)
    qsa.decode_noalloc(d["q"], kcd, vcd, d["sel"], d["cu"], out=o, lse=l, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o, ro) and torch.equal(l, rl), "int4: differs from qsa_decode"
    o_ref, l_ref = oracle_rows(c.q, kc, vc, c.sel, c.cu, fmt="int4", group=32, k_scale=ks, v_scale=vs)
    compare(o, l, o_ref, l_ref, c.lengths, label="no-alloc int4 g32")


def test_captured_call_replays_with_new_lengths():
    """Captured after a first eager call, the no-alloc decode replays with
    cu_seqlens and indices rewritten on the device, equal to eager calls."""
    banks = synth.sweep_bank(5151, 12, "saturated", 8192, banks=8)
    rng = np.random.default_rng(5)
    k = synth.normal_bf16(rng, (8192, 2, 256)).cuda()
    v = synth.normal_bf16(rng, (8192, 2, 256)).cuda()
    q = synth.normal_bf16(rng, (12, 24, 256)).cuda()
    sels = [torch.from_numpy(s_).cuda() for s_, _ in banks]
    cus = [torch.from_numpy(c_).cuda() for _, c_ in banks]
    sel_buf, cu_buf = sels[0].clone(), cus[0].clone()
    out = torch.empty(12, 24, 256, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(12, 24, dtype=torch.float32, device="cuda")
    qsa.decode_noalloc(q, k, v, sel_buf, cu_buf, out=out, lse=lse)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        qsa.decode_noalloc(q, k, v, sel_buf, cu_buf, out=out, lse=lse)
    for r in range(64):
        b = r % 8
        sel_buf.copy_(sels[b])
        cu_buf.copy_(cus[b])
        g.replay()
        ro, rl = qsa.decode(q, k, v, sels[b], cus[b])
        torch.cuda.synchronize()
        assert torch.equal(out, ro) and torch.equal(lse, rl), f"replay {r} (bank {b}) differs"
    del g


def test_plan_beyond_scratch_is_refused():
    qsa.set_option("max_splits", 64)
    qsa.set_option("splits", 64)
    try:
        q = torch.zeros(128, 24, 256, dtype=torch.bfloat16, device="cuda")
        k = torch.zeros(16, 2, 256, dtype=torch.bfloat16, device="cuda")
        sel = torch.zeros(1, dtype=torch.int32, device="cuda")
        cu = torch.zeros(129, dtype=torch.int32, device="cuda")
        out = torch.empty(128, 24, 256, dtype=torch.bfloat16, device="cuda")
        lse = torch.empty(128, 24, dtype=torch.float32, device="cuda")
        with pytest.raises(qsa.QsaError, match="scratch"):
            qsa.decode_noalloc(q, k, k, sel, cu, out=out, lse=lse)
    finally:
        qsa.set_option("splits", 0)
        qsa.set_option("max_splits", 16)
