"""Helpers shared by the GPU tests: move synthetic cases to the device,
run the HIP path through the C ABI binding, and compare with the oracle.

Acceptance (page "fix(qsa): restore SM121 correctness with Humanize and
Kernel Design Agent", section "Optimized kernel": relative L2 <= 2e-3
against an independent FP32 reference): whole-tensor relative L2 of the
bf16 output <= 2e-3 against the float64 oracle, |lse - lse_ref| <= 1e-3,
empty rows exactly o = 0, lse = -inf.

Per (row, head) the output is also held to its own rounding floor.  Let
y = o_ref[b, h, :] (float64), x the kernel's fp32 result before its final
rounding and r = bf16(x) the stored output.  Where bf16(x) and bf16(y)
differ, y lies within |x_i - y_i| of a rounding midpoint, so for every
element |r_i - y_i| <= |bf16(y)_i - y_i| + 2 |x_i - y_i|, and by the
triangle inequality

    ||r - y|| / ||y||  <=  floor(y) + 2 ||x - y|| / ||y||,
    floor(y) = ||bf16(y) - y|| / ||y||   (at most 2^-8 for any y).

The fp32 arithmetic of the kernel (exact bf16 products, fp32 sums, P as a
hi + lo bf16 pair, fp32 scales and merges) is budgeted at
||x - y|| / ||y|| <= 1e-4 per head, so each head must satisfy
rel_h <= floor_h + 2e-4.  A head whose reference is exactly zero must be
exactly zero.
"""
from __future__ import annotations

import os
import sys

import numpy as np

REL_L2_TOL = 2e-3
LSE_TOL = 1e-3
HEAD_FP32_BUDGET = 1e-4        # ||x - y|| / ||y|| per (row, head), see above
HEAD_MARGIN = 2 * HEAD_FP32_BUDGET


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float64 -> nearest bf16 value (ties to even), via float32.  The double
    rounding can differ from a direct rounding only on exact float32 ties
    of the first step, which moves the floor below by at most one element's
    half ulp."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def head_report(o: np.ndarray, o_ref: np.ndarray):
    """Per (row, head) relative L2 of o against o_ref and the bf16 floor of
    o_ref, for arrays [rows, heads, 256]; heads with a zero reference get
    rel = 0 if o is zero there too, else inf."""
    ref_n = np.sqrt(np.sum(o_ref * o_ref, axis=-1))
    err_n = np.sqrt(np.sum((o - o_ref) ** 2, axis=-1))
    fl_n = np.sqrt(np.sum((bf16_round(o_ref) - o_ref) ** 2, axis=-1))
    zero = ref_n == 0
    safe = np.where(zero, 1.0, ref_n)
    rel = np.where(zero, np.where(err_n == 0, 0.0, np.inf), err_n / safe)
    floor = np.where(zero, 0.0, fl_n / safe)
    return rel, floor


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
    of, rf = o[full], o_ref[full]
    diff = of - rf
    ref2 = np.sum(rf * rf)
    rel = float(np.sqrt(np.sum(diff * diff) / ref2)) if ref2 > 0 else (0.0 if not diff.any() else np.inf)
    rb = bf16_round(rf)
    rel_vs_bf16 = float(np.sqrt(np.sum((of - rb) ** 2) / ref2)) if ref2 > 0 else 0.0
    mism = float(np.mean(of != rb))
    lse_err = float(np.max(np.abs(lg[full] - l_ref[full])))
    rel_h, floor_h = head_report(of, rf)
    excess = rel_h - floor_h
    worst = np.unravel_index(int(np.argmax(excess)), excess.shape)
    say(f"  {label}: rel-L2 {rel:.3e} (vs bf16(ref) {rel_vs_bf16:.2e}, {mism:.2%} elements "
        f"!= bf16(ref))  max|dlse| {lse_err:.2e}  worst head row{worst[0]}/h{worst[1]}: "
        f"rel {rel_h[worst]:.3e} floor {floor_h[worst]:.3e} (+{excess[worst]:.1e})")
    assert rel <= tol, f"{label}: rel-L2 {rel:.3e} > {tol}"
    assert lse_err <= lse_tol, f"{label}: lse error {lse_err:.3e} > {lse_tol}"
    assert excess[worst] <= HEAD_MARGIN, (
        f"{label}: head (row {worst[0]}, h {worst[1]}) rel-L2 {rel_h[worst]:.3e} exceeds its "
        f"bf16 floor {floor_h[worst]:.3e} by more than {HEAD_MARGIN:.0e}")
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
