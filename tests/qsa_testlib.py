"""Helpers shared by the GPU tests: move synthetic cases to the device,
run the HIP path through the C ABI binding, and compare with the oracle.

Acceptance (page "fix(qsa): restore SM121 correctness with Humanize and
Kernel Design Agent", section "Optimized kernel": relative L2 <= 2e-3
against an independent FP32 reference): whole-tensor relative L2 of the
bf16 output <= 2e-3 against the float64 oracle, |lse - lse_ref| <= 1e-3,
empty rows exactly o = 0, lse = -inf.
"""
from __future__ import annotations

import os
import sys

import numpy as np

REL_L2_TOL = 2e-3
LSE_TOL = 1e-3


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def oracle_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def to_device(case, device="cuda"):
    import torch
    return dict(
        q=case.q.to(device),
        k=case.k_pool.to(device),
        v=case.v_pool.to(device),
        sel=torch.from_numpy(case.sel).to(device),
        cu=torch.from_numpy(case.cu).to(device),
    )


def sub_case(q, sel, cu, rows):
    """Rows ``rows`` of a packed call as their own packed call (host data)."""
    rows = list(rows)
    lists = [sel[cu[b]:cu[b + 1]] for b in rows]
    lens = np.array([len(x) for x in lists])
    cu2 = np.zeros(len(rows) + 1, np.int32)
    cu2[1:] = np.cumsum(lens)
    sel2 = np.concatenate(lists).astype(np.int32) if lens.sum() else np.zeros(0, np.int32)
    return q[rows].contiguous(), sel2, cu2


def oracle_rows(q, k, v, sel, cu, rows=None, **kw):
    """Oracle output for all rows (rows=None) or a subset, in the subset's order."""
    import oracle
    if rows is None:
        return oracle.decode(q, k, v, sel, cu, nthreads=oracle_threads(), **kw)
    q2, sel2, cu2 = sub_case(q, sel, cu, rows)
    return oracle.decode(q2, k, v, sel2, cu2, nthreads=oracle_threads(), **kw)


def compare(out, lse, o_ref, l_ref, lengths, *, tol=REL_L2_TOL, lse_tol=LSE_TOL, label=""):
    """out/lse: GPU tensors or arrays for the same rows as o_ref/l_ref."""
    o = out.float().cpu().double().numpy() if hasattr(out, "cpu") else np.asarray(out, np.float64)
    lg = lse.cpu().double().numpy() if hasattr(lse, "cpu") else np.asarray(lse, np.float64)
    lengths = np.asarray(lengths)
    empty = lengths == 0
    if empty.any():
        assert not o[empty].any(), f"{label}: empty rows must be exactly 0"
        assert np.all(np.isneginf(lg[empty])), f"{label}: empty rows must have lse = -inf"
    full = ~empty
    if not full.any():
        return 0.0
    assert np.all(np.isfinite(o[full])), f"{label}: non-finite output"
    diff = o[full] - o_ref[full]
    rel = float(np.sqrt(np.sum(diff * diff) / np.sum(o_ref[full] * o_ref[full])))
    lse_err = float(np.max(np.abs(lg[full] - l_ref[full])))
    say(f"  {label}: rel-L2 {rel:.3e}  max|dlse| {lse_err:.2e}")
    assert rel <= tol, f"{label}: rel-L2 {rel:.3e} > {tol}"
    assert lse_err <= lse_tol, f"{label}: lse error {lse_err:.3e} > {lse_tol}"
    return rel


def run_and_compare(case, label, rows=None, quant=None, scale_dtype=None, **decode_kw):
    """Decode a synth.QsaCase on the GPU and compare with the oracle.
    quant = (fmt, group, kc, ks, vc, vs) for quantized pools (host arrays);
    scale_dtype = torch dtype the scales are handed to the GPU in (default
    float32; the oracle always gets their float32 values)."""
    import torch
    import sparse_index_paged_amd as qsa
    d = to_device(case)
    kw = {}
    okw = {}
    if quant is not None:
        fmt, group, kc, ks, vc, vs = quant
        d["k"] = torch.from_numpy(kc).cuda()
        d["v"] = torch.from_numpy(vc).cuda()
        sdt = scale_dtype or torch.float32
        kw = dict(kv_format=fmt, k_scale=torch.from_numpy(ks).to(sdt).cuda(),
                  v_scale=torch.from_numpy(vs).to(sdt).cuda(), group_size=group)
        okw = dict(fmt=fmt, group=group, k_scale=ks, v_scale=vs)
        kpool, vpool = kc, vc
    else:
        kpool, vpool = case.k_pool, case.v_pool
    kw.update(decode_kw)
    say(f"[gpu] {label}: bs={case.bs} hq={case.hq} hkv={case.hkv} "
        f"slots={case.k_pool.shape[0]} n_sel={case.sel.shape[0]}")
    out, lse = qsa.decode(d["q"], d["k"], d["v"], d["sel"], d["cu"], **kw)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle_rows(case.q, kpool, vpool, case.sel, case.cu, rows, **okw)
    lengths = case.lengths if rows is None else case.lengths[list(rows)]
    o_g = out if rows is None else out[list(rows)]
    l_g = lse if rows is None else lse[list(rows)]
    rel = compare(o_g, l_g, o_ref, l_ref, lengths, label=label)
    return out, lse, rel
