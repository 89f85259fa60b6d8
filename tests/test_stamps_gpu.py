"""The measurement build libqsa_stamps.so (include/qsa_stamps.h): its decode
gives libqsa.so's outputs bit for bit, and every workgroup's phase stamps
come in the order of the kernel's phases."""
import ctypes

import numpy as np
import pytest
import torch

import synth
from qsa_testlib import say

import sparse_index_paged_amd as qsa
from sparse_index_paged_amd import _binding as B

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("hkv", [2, 1])
def test_stamped_decode_matches_and_stamps_are_ordered(hkv):
    lib = B.load_stamps_library()
    case = synth.make_case(lengths=[2055, 300, 0, 1, 2055, 64, 1500, 17], slots=8192, hkv=hkv,
                           seed=640 + hkv, dup_prob=0.1)
    say(f"[gpu] stamped decode hkv={hkv}")
    q, k, v = case.q.cuda(), case.k_pool.cuda(), case.v_pool.cuda()
    sel, cu = torch.from_numpy(case.sel).cuda(), torch.from_numpy(case.cu).cuda()
    o_ref, l_ref = qsa.decode(q, k, v, sel, cu)
    ns, nw = ctypes.c_int(), ctypes.c_int()
    assert lib.qsa_plan(case.bs, hkv, ctypes.byref(ns), ctypes.byref(nw)) == 0
    stamps = torch.zeros(nw.value * 8, dtype=torch.int64, device="cuda")
    out = torch.empty_like(o_ref)
    lse = torch.empty_like(l_ref)
    assert lib.qsa_debug_set_phase_stamps(stamps.data_ptr(), stamps.numel()) == 0
    try:
        d = [B.describe(x) for x in (q, k, v, sel, cu, out, lse)]
        st = lib.qsa_decode(ctypes.byref(d[0]), ctypes.byref(d[1]), ctypes.byref(d[2]), None,
                            ctypes.byref(d[3]), ctypes.byref(d[4]), ctypes.byref(d[5]),
                            ctypes.byref(d[6]), B._stream_handle(None))
        assert st == 0, lib.qsa_last_error().decode()
        torch.cuda.synchronize()
    finally:
        lib.qsa_debug_set_phase_stamps(None, 0)
    assert torch.equal(out, o_ref) and torch.equal(lse, l_ref)
    s = stamps.view(nw.value, 8).cpu().numpy()
    active = s[:, 1] > 0
    assert active.sum() >= case.bs * hkv, "every (row, KV head) pair has at least one active workgroup"
    a = s[active]
    assert np.all(a[:, 0] <= a[:, 1]) and np.all(a[:, 1] <= a[:, 3]) and np.all(a[:, 3] <= a[:, 4])
    # slot 2 only where the workgroup's first wave has a tile (short rows leave it none)
    tiled = a[:, 2] > 0
    assert tiled.any()
    assert np.all(a[tiled, 1] <= a[tiled, 2]) and np.all(a[tiled, 2] <= a[tiled, 3])
    split = a[:, 5] > 0
    assert np.all(a[split, 4] <= a[split, 5])
    done = a[:, 6] > 0
    assert np.all(a[done, 6] >= a[done, 4]) and np.all(a[done & split, 6] >= a[done & split, 5])
    # every workgroup ends: unsplit ones write the output, split ones count their arrival
    assert np.all(done | split)
