"""Parity of the HIP decode path with the oracle, through the C ABI.

Workloads follow the packed decode contract of the page "fix(qsa): restore
SM121 correctness with Humanize and Kernel Design Agent" (section
"Changes"); quantized pools follow the page "feat(qsa): quantized KV pools
with dequant-on-gather (fp8/int8/int4)" (part 4 "Modifications").
"""
import numpy as np
import pytest
import torch

import synth
from oracle import quant
from qsa_testlib import compare, oracle_rows, run_and_compare, say, to_device

import sparse_index_paged_amd as qsa

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _default_options():
    yield
    qsa.set_option("split_target", 0)
    qsa.set_option("max_splits", 16)
    qsa.set_option("min_split_keys", 256)
    qsa.set_option("waves_per_workgroup", 0)
    qsa.set_option("splits", 0)
    qsa.set_option("xcc_lanes", 1)


def test_bs1_tp1_l128():
    run_and_compare(synth.case_bs1_tp1(), "bs1 tp1 L128")


def test_bs16_tp2_mixed_lengths():
    run_and_compare(synth.case_bs16_tp2_mixed(), "bs16 tp2 mixed")


def test_bs128_tp1_saturated_all_rows_small_pool():
    case = synth.case_bs128_tp1_saturated(seed=1031, slots=16384)
    run_and_compare(case, "bs128 tp1 sat2055 (16k-slot pool, all rows)")


def test_bs128_tp1_saturated_full_size_sampled_rows():
    """Full-size pools [262144, 2, 256] with 5% peaked keys, in the launch
    configuration the benchmark times; the oracle checks 16 sampled rows."""
    case = synth.case_bs128_tp1_saturated()
    rows = sorted(np.random.default_rng(7).choice(128, size=16, replace=False).tolist())
    out, lse, _ = run_and_compare(case, "bs128 tp1 sat2055 full size", rows=rows)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    assert all(v == 0 for v in qsa.debug_counters())


@pytest.mark.parametrize("fmt,group,seed", [("fp8", 256, 1041), ("int8", 256, 1042),
                                            ("int4", 32, 1043)])
def test_bs64_tp1_quantized_full_size(fmt, group, seed):
    case = synth.case_bs64_tp1_quantsrc(seed)
    kc, ks = quant.quantize(case.k_pool, fmt, group)
    vc, vs = quant.quantize(case.v_pool, fmt, group)
    run_and_compare(case, f"bs64 tp1 {fmt} g{group}", quant=(fmt, group, kc, ks, vc, vs))


@pytest.mark.parametrize("scale_dtype", [torch.float32, torch.float16])
def test_bs128_tp1_int4_unsplit_eight_waves(scale_dtype):
    """bs=128 TP1 runs unsplit, where int4 pools take 8-wave workgroups by
    default; 12 sampled rows against the oracle."""
    case = synth.case_bs64_tp1_quantsrc(1044, bs=128)
    assert qsa.plan(128, 2)[0] == 1
    sd = "f16" if scale_dtype == torch.float16 else "f32"
    kc, ks = quant.quantize(case.k_pool, "int4", 32, sd)
    vc, vs = quant.quantize(case.v_pool, "int4", 32, sd)
    rows = sorted(np.random.default_rng(9).choice(128, size=12, replace=False).tolist())
    run_and_compare(case, f"bs128 tp1 int4 {sd}", rows=rows, quant=("int4", 32, kc, ks, vc, vs),
                    scale_dtype=scale_dtype)


@pytest.mark.parametrize("fmt,group", [("fp8", 64), ("fp8", 32), ("int8", 64), ("int8", 32),
                                       ("int4", 64)])
@pytest.mark.parametrize("hkv", [1, 2])
@pytest.mark.parametrize("waves", [0, 4])   # 0: the default, 8 waves for quantized pools
def test_quantized_group_sizes(fmt, group, hkv, waves):
    qsa.set_option("waves_per_workgroup", waves)
    lens = [1, 17, 300, 2055, 64, 0, 1000]
    case = synth.make_case(lengths=lens, slots=4096, hkv=hkv, seed=2000 + group + hkv,
                           dup_prob=0.05)
    kc, ks = quant.quantize(case.k_pool, fmt, group)
    vc, vs = quant.quantize(case.v_pool, fmt, group)
    run_and_compare(case, f"{fmt} g{group} hkv{hkv}", quant=(fmt, group, kc, ks, vc, vs))


@pytest.mark.parametrize("fmt,group", [("fp8", 256), ("int4", 32)])
@pytest.mark.parametrize("splits", [0, 3])   # 0: the plan's split count
def test_quantized_rows_not_filling_the_xcds(fmt, group, splits):
    """Quantized pools put every KV head of row b on XCD b % 8 and round the
    rows up to a multiple of 8, so batch sizes that leave part of the last
    group of 8 rows empty launch idle workgroups past the last row.  Every
    row of each batch size below, in both layouts, is compared with the
    oracle; out and lse start as NaN, so a row no workgroup writes fails."""
    qsa.set_option("splits", splits)
    for bs in (1, 3, 4, 9, 12, 17, 33, 125):
        for hkv in (1, 2):
            rng = np.random.default_rng(9000 + 10 * bs + hkv)
            lens = rng.integers(0, 2056, size=bs).tolist()
            lens[0] = 2055
            case = synth.make_case(lengths=lens, slots=4096, hkv=hkv, seed=9100 + bs + hkv,
                                   dup_prob=0.05)
            kc, ks = quant.quantize(case.k_pool, fmt, group)
            vc, vs = quant.quantize(case.v_pool, fmt, group)
            out = torch.full((bs, case.hq, 256), float("nan"), dtype=torch.bfloat16, device="cuda")
            lse = torch.full((bs, case.hq), float("nan"), dtype=torch.float32, device="cuda")
            run_and_compare(case, f"{fmt} g{group} bs{bs} hkv{hkv} splits={splits}",
                            quant=(fmt, group, kc, ks, vc, vs), out=out, lse=lse)
    assert all(v == 0 for v in qsa.debug_counters())


@pytest.mark.parametrize("splits", [1, 2, 3, 4, 5, 6, 7, 8, 9])
@pytest.mark.parametrize("fmt", ["bf16", "int4"])
def test_every_split_count(splits, fmt):
    """Any partition of a list into contiguous splits merges to the same
    attention (page "fix(qsa): restore SM121 correctness with Humanize and
    Kernel Design Agent", section "Optimized kernel": splits combined by a
    stable fp32 log-sum-exp merge in the final split): each forced split
    count against the oracle, rows of every length class, counters at rest."""
    qsa.set_option("splits", splits)
    lens = [2055, 1, 257, 0, 1500, 2055, 768, 31]
    case = synth.make_case(lengths=lens, slots=8192, hkv=2, seed=300 + splits, dup_prob=0.1)
    assert qsa.plan(case.bs, 2)[0] == splits
    if fmt == "bf16":
        run_and_compare(case, f"splits={splits} bf16")
    else:
        kc, ks = quant.quantize(case.k_pool, "int4", 32, "f16")
        vc, vs = quant.quantize(case.v_pool, "int4", 32, "f16")
        run_and_compare(case, f"splits={splits} int4", quant=("int4", 32, kc, ks, vc, vs),
                        scale_dtype=torch.float16)
    assert all(v == 0 for v in qsa.debug_counters())


def designed_logit_case(seed: int) -> synth.QsaCase:
    """Rows whose logits follow set sequences.  Row r lists slots r*2055 ..
    r*2055 + 2054 in order; slot j's K row holds a_r[j] in channel 0 and
    zeros elsewhere, and head h's query holds 1 + h/24 in channel 0, so the
    logit of entry j for head h is a_r[j] (1 + h/24) / 16.  In log2 units:
    row 0 rises by 0.05-0.09 per entry (about 100-185 in all), row 1 is flat
    and then jumps by 27-54 at entry 1000, row 2 falls from its first entry,
    row 3 is noise with a spike of 6-11 every 97 entries.  V ~ N(0, 1)."""
    import torch
    rng = np.random.default_rng(seed)
    n = synth.CAPACITY
    j = np.arange(n, dtype=np.float64)
    seqs = [0.5 * j,
            np.where(j < 1000, 0.0, 300.0 + (j % 7)),
            500.0 - 0.25 * j,
            rng.normal(0.0, 8.0, n) + np.where(j % 97 == 0, 60.0, 0.0)]
    bs, hkv = len(seqs), 2
    k = torch.zeros(bs * n, hkv, 256, dtype=torch.bfloat16)
    for r, a in enumerate(seqs):
        k[r * n:(r + 1) * n, :, 0] = torch.from_numpy(a).to(torch.bfloat16)[:, None]
    v = synth.normal_bf16(rng, (bs * n, hkv, 256))
    q = torch.zeros(bs, 12 * hkv, 256, dtype=torch.bfloat16)
    q[:, :, 0] = torch.tensor([1.0 + h / 24 for h in range(12 * hkv)], dtype=torch.bfloat16)
    sel, cu = synth.pack([np.arange(r * n, (r + 1) * n, dtype=np.int32) for r in range(bs)])
    return synth.QsaCase(q=q, k_pool=k, v_pool=v, sel=sel, cu=cu, name="designed logits")


@pytest.mark.parametrize("fmt", ["bf16", "int4"])
@pytest.mark.parametrize("waves,splits", [(4, 1), (8, 1), (0, 0)])
def test_running_max_sequences(waves, splits, fmt):
    """The running max of the online softmax moves only once a tile's max
    exceeds it by more than 2^8; logits that rise slowly through that margin,
    jump far past it, fall from the start or spike (designed_logit_case),
    with one wave slice of 514 or 257 entries per wave or the default plan,
    all match the oracle."""
    qsa.set_option("waves_per_workgroup", waves)
    qsa.set_option("splits", splits)
    case = designed_logit_case(901)
    label = f"designed logits {fmt} waves={waves} splits={splits}"
    if fmt == "bf16":
        run_and_compare(case, label)
    else:
        # channel 0 is the only non-zero one of every K row: its group's
        # code is +-7 and the fp16 scale |a| / 7 carries the logit
        kc, ks = quant.quantize(case.k_pool, "int4", 32, "f16")
        vc, vs = quant.quantize(case.v_pool, "int4", 32, "f16")
        run_and_compare(case, label, quant=("int4", 32, kc, ks, vc, vs), scale_dtype=torch.float16)
    assert all(c == 0 for c in qsa.debug_counters())


EDGE_LENGTHS = [0, 1, 2, 15, 16, 17, 63, 64, 65, 255, 256, 257, 1023, 2054, 2055, 0, 3, 511]


@pytest.mark.parametrize("hkv", [1, 2])
@pytest.mark.parametrize("opts", [dict(), dict(split_target=1), dict(split_target=100000),
                                  dict(split_target=100000, min_split_keys=1),
                                  dict(split_target=100000, max_splits=64, min_split_keys=1),
                                  dict(waves_per_workgroup=8),
                                  dict(waves_per_workgroup=8, split_target=1),
                                  dict(waves_per_workgroup=8, split_target=100000,
                                       min_split_keys=1)])
def test_edge_lengths_and_split_plans(hkv, opts):
    for k, v in opts.items():
        qsa.set_option(k, v)
    case = synth.make_case(lengths=EDGE_LENGTHS, slots=8192, hkv=hkv, seed=77 + hkv,
                           dup_prob=0.1)
    run_and_compare(case, f"edge lengths hkv{hkv} {opts} plan={qsa.plan(case.bs, hkv)}")
    assert all(v == 0 for v in qsa.debug_counters())


@pytest.mark.parametrize("bs", [1, 2, 7, 17, 33, 64, 127, 128])
def test_batch_sizes_tp2_tp1(bs):
    rng = np.random.default_rng(bs)
    for hkv in (1, 2):
        lens = rng.integers(0, 2056, size=bs).tolist()
        case = synth.make_case(lengths=lens, slots=8192, hkv=hkv, seed=500 + bs, dup_prob=0.1)
        run_and_compare(case, f"bs{bs} hkv{hkv}")


def test_repeated_single_slot_is_exact():
    """A list of one slot repeated 2055 times: every weight is 1/2055 exactly
    and the output is that V row bit for bit; lse = s + ln 2055."""
    case = synth.make_case(lengths=[5], slots=64, hkv=2, seed=9)
    sel = np.full(2055, 11, np.int32)
    cu = np.array([0, 2055], np.int32)
    d = to_device(case)
    out, lse = qsa.decode(d["q"], d["k"], d["v"], torch.from_numpy(sel).cuda(),
                          torch.from_numpy(cu).cuda())
    torch.cuda.synchronize()
    for h in range(24):
        assert torch.equal(out[0, h].cpu(), case.v_pool[11, h // 12])
    s = (case.q[0].double() @ case.k_pool[11].double().repeat_interleave(12, 0).T).diagonal() / 16
    assert torch.allclose(lse[0].cpu().double(), s + np.log(2055), atol=1e-4)


def test_strided_views():
    """q / pools / out / lse as strided views of larger buffers."""
    case = synth.make_case(lengths=[40, 2055, 7], slots=3000, hkv=2, seed=31)
    big_q = torch.zeros(3, 40, 256, dtype=torch.bfloat16)
    big_q[:, 8:32] = case.q
    big_k = torch.zeros(3000, 4, 256, dtype=torch.bfloat16)
    big_v = torch.zeros(3000, 3, 256, dtype=torch.bfloat16)
    big_k[:, 1:3] = case.k_pool
    big_v[:, 0:2] = case.v_pool
    q = big_q.cuda()[:, 8:32]
    k = big_k.cuda()[:, 1:3]
    v = big_v.cuda()[:, 0:2]
    out_big = torch.full((3, 30, 256), 7.0, dtype=torch.bfloat16, device="cuda")
    lse_big = torch.full((3, 48), 7.0, dtype=torch.float32, device="cuda")
    out = out_big[:, 3:27]
    lse = lse_big[:, ::2]
    sel = torch.from_numpy(case.sel).cuda()
    cu = torch.from_numpy(case.cu).cuda()
    qsa.decode(q, k, v, sel, cu, out=out, lse=lse)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle_rows(case.q, case.k_pool, case.v_pool, case.sel, case.cu)
    compare(out, lse, o_ref, l_ref, case.lengths, label="strided views")
    assert torch.all(out_big[:, :3] == 7.0) and torch.all(out_big[:, 27:] == 7.0)
    assert torch.all(lse_big[:, 1::2] == 7.0)


def test_bitwise_deterministic_and_plan_independent():
    case = synth.make_case(lengths=[2055] * 8 + [700] * 8, slots=20000, hkv=2, seed=41,
                           dup_prob=0.1)
    d = to_device(case)
    o1, l1 = qsa.decode(d["q"], d["k"], d["v"], d["sel"], d["cu"])
    o2, l2 = qsa.decode(d["q"], d["k"], d["v"], d["sel"], d["cu"])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    qsa.set_option("split_target", 1)
    o3, l3 = qsa.decode(d["q"], d["k"], d["v"], d["sel"], d["cu"])
    torch.cuda.synchronize()
    diff = (o3.float() - o1.float()).norm() / o1.float().norm()
    assert diff < 2e-3 and (l3 - l1).abs().max() < 1e-4


def test_xcd_placement_is_checked_and_changes_no_output():
    """bf16 workgroups take their pair slot from the XCD they run on (XCC_ID)
    once the device has passed the dispatch check: 8 XCDs, workgroup i on
    XCD (i + r) % 8.  Which workgroup computes a (row, KV head, split) does
    not enter its arithmetic, so the outputs with that placement, with the
    blockIdx placement, and replayed from a captured graph are bitwise equal;
    the oracle checks the rows once."""
    qsa.set_option("xcc_lanes", 1)
    case = synth.make_case(lengths=[2055] * 20 + [900] * 12 + [5] * 4, slots=20000, hkv=2, seed=43,
                           dup_prob=0.05)
    d = to_device(case)
    o1, l1 = qsa.decode(d["q"], d["k"], d["v"], d["sel"], d["cu"])
    torch.cuda.synchronize()
    if qsa.get_option("xcc_lanes_active") != 1:
        pytest.skip("this device did not pass the dispatch check (fewer than 8 XCDs or no "
                    "round-robin dispatch); placement by blockIdx is used")
    o_ref, l_ref = oracle_rows(case.q, case.k_pool, case.v_pool, case.sel, case.cu, None)
    compare(o1, l1, o_ref, l_ref, case.lengths, label="XCD-read placement")
    for splits in (0, 3):
        qsa.set_option("splits", splits)
        try:
            qsa.set_option("xcc_lanes", 1)
            oa, la = qsa.decode(d["q"], d["k"], d["v"], d["sel"], d["cu"])
            qsa.set_option("xcc_lanes", 0)
            ob, lb = qsa.decode(d["q"], d["k"], d["v"], d["sel"], d["cu"])
            torch.cuda.synchronize()
            assert torch.equal(oa, ob) and torch.equal(la, lb), f"splits={splits}"
            qsa.set_option("xcc_lanes", 1)
            out = torch.empty_like(oa)
            lse = torch.empty_like(la)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                qsa.decode(d["q"], d["k"], d["v"], d["sel"], d["cu"], out=out, lse=lse)
            for _ in range(3):
                out.zero_()
                g.replay()
                torch.cuda.synchronize()
                assert torch.equal(out, oa) and torch.equal(lse, la), f"graph, splits={splits}"
            del g
        finally:
            qsa.set_option("xcc_lanes", 1)
            qsa.set_option("splits", 0)
    assert all(v == 0 for v in qsa.debug_counters())


@pytest.mark.parametrize("fmt,group,sdt", [("fp8", 256, torch.float32), ("int8", 64, torch.float16),
                                          ("int4", 32, torch.float16)])
def test_interleaved_scale_views_give_the_same_outputs(fmt, group, sdt):
    """K and V scales written and read as views of one [slots, 2, Hkv, groups]
    array (k_scale = [:, 0], v_scale = [:, 1]) instead of two arrays: the
    store writes the same codes and scales, the decode gives bitwise the same
    out and lse, and both match the oracle."""
    lens = [2055, 1, 700, 0, 1500, 2055, 33]
    case = synth.make_case(lengths=lens, slots=4096, hkv=2, seed=7000 + group, dup_prob=0.05)
    d = to_device(case)
    slots, width, ng = 4096, (128 if fmt == "int4" else 256), 256 // group
    cdt = torch.int8 if fmt == "int8" else torch.uint8
    loc = torch.arange(slots, dtype=torch.int32, device="cuda")
    buf = torch.empty(slots, 2, 2, ng, dtype=sdt, device="cuda")
    res = []
    for ks, vs in ((torch.empty(slots, 2, ng, dtype=sdt, device="cuda"),
                    torch.empty(slots, 2, ng, dtype=sdt, device="cuda")), (buf[:, 0], buf[:, 1])):
        kc = torch.empty(slots, 2, width, dtype=cdt, device="cuda")
        vc = torch.empty_like(kc)
        qsa.kv_store(d["k"], d["v"], loc, kc, vc, kv_format=fmt, k_scale=ks, v_scale=vs, group_size=group)
        o, l = qsa.decode(d["q"], kc, vc, d["sel"], d["cu"], kv_format=fmt, k_scale=ks, v_scale=vs,
                          group_size=group)
        torch.cuda.synchronize()
        res.append((kc, vc, ks, vs, o, l))
    (k1, v1, ks1, vs1, o1, l1), (k2, v2, ks2, vs2, o2, l2) = res
    assert torch.equal(k1, k2) and torch.equal(v1, v2)
    assert torch.equal(ks1, ks2) and torch.equal(vs1, vs2)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    kq, kss = quant.quantize(case.k_pool, fmt, group, "f16" if sdt == torch.float16 else "f32")
    vq, vss = quant.quantize(case.v_pool, fmt, group, "f16" if sdt == torch.float16 else "f32")
    o_ref, l_ref = oracle_rows(case.q, kq, vq, case.sel, case.cu, None, fmt=fmt, group=group,
                               k_scale=kss, v_scale=vss)
    compare(o2, l2, o_ref, l_ref, case.lengths, label=f"interleaved scales {fmt} g{group}")


def test_controls_k_zero_v_zero():
    """K := 0 gives uniform weights (mean of the listed V rows, lse = ln L);
    V := 0 gives exactly zero."""
    case = synth.make_case(lengths=[2055, 100, 1], slots=5000, hkv=2, seed=51)
    d = to_device(case)
    zk = torch.zeros_like(d["k"])
    out, lse = qsa.decode(d["q"], zk, d["v"], d["sel"], d["cu"])
    torch.cuda.synchronize()
    for b in range(case.bs):
        idx = torch.from_numpy(case.sel[case.cu[b]:case.cu[b + 1]].astype(np.int64))
        for g in range(2):
            mean = case.v_pool[idx, g].double().mean(0)
            got = out[b, 12 * g:12 * g + 12].cpu().double()
            rel = (got - mean).norm() / (mean.norm() * np.sqrt(12))
            assert rel < 2e-3
        assert torch.allclose(lse[b].cpu().double(),
                              torch.full((24,), float(np.log(case.lengths[b])), dtype=torch.float64),
                              atol=1e-5)
    out, _ = qsa.decode(d["q"], d["k"], torch.zeros_like(d["v"]), d["sel"], d["cu"])
    torch.cuda.synchronize()
    assert not out.float().any()


def test_device_errors_are_reported_and_isolated():
    """Rows whose lengths or slot ids are outside the contract come back as
    NaN with a device error bit; the other rows are unaffected."""
    case = synth.make_case(lengths=[30, 2056, 30, 30], slots=1000, hkv=1, seed=61)
    sel = case.sel.copy()
    sel[case.cu[2] + 5] = 1000          # slot id == slots: out of range
    qsa.workspace_reset()
    d = to_device(case)
    out, lse = qsa.decode(d["q"], d["k"], d["v"], torch.from_numpy(sel).cuda(), d["cu"])
    word = qsa.debug_device_error()
    assert word == 3, word
    assert torch.isnan(out[1].float()).all() and torch.isnan(lse[1]).all()
    assert torch.isnan(out[2].float()).all() and torch.isnan(lse[2]).all()
    good = [0, 3]
    o_ref, l_ref = oracle_rows(case.q, case.k_pool, case.v_pool, case.sel, case.cu, good)
    compare(out[good], lse[good], o_ref, l_ref, case.lengths[good], label="good rows")
    # cu beyond the end of sel
    cu_bad = torch.tensor([0, 30, 70000], dtype=torch.int32, device="cuda")
    q2 = d["q"][:2].contiguous()
    out2, lse2 = qsa.decode(q2, d["k"], d["v"], d["sel"], cu_bad)
    torch.cuda.synchronize()
    assert torch.isnan(out2[1].float()).all() and not torch.isnan(out2[0].float()).any()
    assert all(v == 0 for v in qsa.debug_counters())
    qsa.workspace_reset()
    assert qsa.debug_device_error() == 0


def test_one_launch_per_call_and_counters_at_rest():
    """torch's profiler sees exactly one kernel per qsa_decode call."""
    case = synth.make_case(lengths=[2055] * 4, slots=4096, hkv=2, seed=71)
    d = to_device(case)
    qsa.decode(d["q"], d["k"], d["v"], d["sel"], d["cu"])
    torch.cuda.synchronize()
    from torch.profiler import ProfilerActivity, profile
    with profile(activities=[ProfilerActivity.CUDA]) as prof:
        for _ in range(3):
            qsa.decode(d["q"], d["k"], d["v"], d["sel"], d["cu"])
        torch.cuda.synchronize()
    kernels = [e for e in prof.events() if e.device_type == torch.autograd.DeviceType.CUDA
               and "qsa_decode_kernel" in e.name]
    say(f"  decode kernels seen: {len(kernels)}")
    assert len(kernels) == 3
    assert all(v == 0 for v in qsa.debug_counters())


def test_pools_beyond_32bit_offsets():
    """Pools whose slot stride is 2^24 bytes (a strided view into a 4.4 GB
    buffer per pool), so row offsets do not fit the 32-bit address form and
    the 64-bit path is used; compared with the oracle on a compact copy."""
    slots, hkv = 260, 2
    case = synth.make_case(lengths=[2055, 700, 1, 0, 1500], slots=slots, hkv=hkv, seed=88,
                           dup_prob=0.05)
    stride = 1 << 23  # bf16 elements = 2^24 bytes per slot
    say(f"[gpu] 64-bit addressing: slots={slots} slot stride={2 * stride} B")
    kb = torch.empty(slots * stride, dtype=torch.bfloat16, device="cuda")
    vb = torch.empty(slots * stride, dtype=torch.bfloat16, device="cuda")
    k = kb.as_strided((slots, hkv, 256), (stride, 256, 1))
    v = vb.as_strided((slots, hkv, 256), (stride, 256, 1))
    k.copy_(case.k_pool.cuda())
    v.copy_(case.v_pool.cuda())
    out, lse = qsa.decode(case.q.cuda(), k, v, torch.from_numpy(case.sel).cuda(),
                          torch.from_numpy(case.cu).cuda())
    torch.cuda.synchronize()
    o_ref, l_ref = oracle_rows(case.q, case.k_pool, case.v_pool, case.sel, case.cu)
    compare(out, lse, o_ref, l_ref, case.lengths, label="64-bit addressing")
    del kb, vb
    torch.cuda.empty_cache()


@pytest.mark.parametrize("fmt,group", [("bf16", 256), ("fp8", 256), ("int4", 32)])
def test_kv_pool_descriptor_reused(fmt, group):
    """A KvPool (descriptors of the pools and scales built once) gives the
    plain calls' results bit for bit: a store of new tokens into twin pools,
    then qsa_decode and qsa_decode_noalloc through both forms."""
    rng = np.random.default_rng(611)
    case = synth.make_case(lengths=[2055, 0, 300, 1, 1500], slots=4096, hkv=2, seed=612, dup_prob=0.1)
    new_k = synth.normal_bf16(rng, (64, 2, 256)).cuda()
    new_v = synth.normal_bf16(rng, (64, 2, 256)).cuda()
    loc = torch.from_numpy(rng.choice(4096, 64, replace=False).astype(np.int32)).cuda()
    kw = {}
    if fmt == "bf16":
        pools = [(case.k_pool.cuda(), case.v_pool.cuda(), None, None) for _ in range(2)]
    else:
        kc, ks = quant.quantize(case.k_pool, fmt, group, "f16")
        vc, vs = quant.quantize(case.v_pool, fmt, group, "f16")
        mk = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
        f16 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.float16).cuda()
        pools = [(mk(kc), mk(vc), f16(ks), f16(vs)) for _ in range(2)]
        kw = dict(kv_format=fmt, group_size=group)
    ka, va, ksa, vsa = pools[0]
    kb, vb, ksb, vsb = pools[1]
    sc_a = dict(k_scale=ksa, v_scale=vsa) if fmt != "bf16" else {}
    pool = qsa.KvPool(kb, vb, k_scale=ksb, v_scale=vsb, **kw)
    qsa.kv_store(new_k, new_v, loc, ka, va, **kw, **sc_a)
    pool.store(new_k, new_v, loc)
    q = case.q.cuda()
    sel, cu = torch.from_numpy(case.sel).cuda(), torch.from_numpy(case.cu).cuda()
    oa, la = qsa.decode(q, ka, va, sel, cu, **kw, **sc_a)
    ob, lb = pool.decode(q, sel, cu)
    out = torch.empty_like(ob)
    lse = torch.empty_like(lb)
    oc, lc = pool.decode(q, sel, cu, out=out, lse=lse, noalloc=True)
    torch.cuda.synchronize()
    assert torch.equal(oa, ob) and torch.equal(la, lb)
    assert torch.equal(oa, oc) and torch.equal(la, lc)
    for a, b in zip(pools[0], pools[1]):
        if a is not None:
            assert torch.equal(a, b)
    assert all(v == 0 for v in qsa.debug_counters())
