"""Repeated launches leave every split counter at rest.

Page "fix(qsa): restore SM121 correctness with Humanize and Kernel Design
Agent": 150,000 consecutive launches with every cached atomic counter back
to zero, and a bs=17, 24Q/2KV long-list case that crosses the old scratch
boundary (sections "Optimized kernel" and the integration update).
"""
import numpy as np
import pytest
import torch

import synth
from qsa_testlib import compare, oracle_rows, say, to_device

import sparse_index_paged_amd as qsa

pytestmark = pytest.mark.gpu


def test_150k_launches_counters_at_rest():
    case = synth.make_case(lengths=[2055] * 15 + [2055, 1], slots=16384, hkv=2, seed=17,
                           dup_prob=0.1)
    d = to_device(case)
    out, lse = qsa.decode(d["q"], d["k"], d["v"], d["sel"], d["cu"])
    torch.cuda.synchronize()
    o_ref, l_ref = oracle_rows(case.q, case.k_pool, case.v_pool, case.sel, case.cu)
    compare(out, lse, o_ref, l_ref, case.lengths, label="bs17 tp1 first launch")
    first_o, first_l = out.clone(), lse.clone()

    audit = torch.zeros(1, dtype=torch.int32, device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(100):
            qsa.decode(d["q"], d["k"], d["v"], d["sel"], d["cu"], out=out, lse=lse)
            qsa.debug_audit_counters(audit)
    n = 0
    for rep in range(1500):
        g.replay()
        n += 100
        if rep % 300 == 299:
            torch.cuda.synchronize()
            say(f"  {n} launches, audit={audit.item()}")
    torch.cuda.synchronize()
    assert n == 150_000
    assert audit.item() == 0
    assert all(v == 0 for v in qsa.debug_counters())
    assert torch.equal(out, first_o) and torch.equal(lse, first_l)
