"""Seeded random configurations of the single-tier decode against the
oracle: pool format, scale group and dtype, layout, batch size, list
lengths (0, 1 and 2055 among them), duplicate runs, forced split counts and
waves per workgroup drawn together, so combinations that no hand-written
test names are covered too (the same acceptance as every parity test: the
page "fix(qsa): restore SM121 correctness with Humanize and Kernel Design
Agent", section "Optimized kernel")."""
import numpy as np
import pytest
import torch

import synth
from oracle import quant
from qsa_testlib import run_and_compare

import sparse_index_paged_amd as qsa

pytestmark = pytest.mark.gpu

GROUPS = {"bf16": [256], "fp8": [256, 64, 32], "int8": [256, 64, 32], "int4": [64, 32]}
N_CASES = 40


def draw_case(i: int):
    rng = np.random.default_rng(7000 + i)
    fmt = ["bf16", "fp8", "int8", "int4"][int(rng.integers(4))]
    group = int(rng.choice(GROUPS[fmt]))
    sdt = "f16" if rng.random() < 0.5 else "f32"
    hkv = int(rng.integers(1, 3))
    bs = int(rng.integers(1, 13))
    lens = [int(x) for x in rng.choice([0, 1, 2, 15, 16, 17, 100, 777, 2054, 2055], size=bs)]
    if rng.random() < 0.5:
        lens[int(rng.integers(bs))] = 2055
    opts = dict(waves_per_workgroup=int(rng.choice([0, 4, 8])),
                splits=int(rng.choice([0, 0, 1, 2, 3, 5, 9, 12])))
    return dict(fmt=fmt, group=group, sdt=sdt, hkv=hkv, lens=lens, opts=opts,
                dup=float(rng.choice([0.0, 0.1])), seed=7100 + i)


@pytest.fixture(autouse=True)
def _reset_options():
    yield
    qsa.set_option("waves_per_workgroup", 0)
    qsa.set_option("splits", 0)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_configuration(i):
    c = draw_case(i)
    for name, value in c["opts"].items():
        qsa.set_option(name, value)
    case = synth.make_case(lengths=c["lens"], slots=4096, hkv=c["hkv"], seed=c["seed"],
                           dup_prob=c["dup"], peaked_frac=0.05)
    label = (f"case {i}: {c['fmt']} g{c['group']} {c['sdt']} hkv{c['hkv']} bs{len(c['lens'])} "
             f"{c['opts']} lens={c['lens']}")
    if c["fmt"] == "bf16":
        run_and_compare(case, label)
    else:
        kc, ks = quant.quantize(case.k_pool, c["fmt"], c["group"], c["sdt"])
        vc, vs = quant.quantize(case.v_pool, c["fmt"], c["group"], c["sdt"])
        run_and_compare(case, label, quant=(c["fmt"], c["group"], kc, ks, vc, vs),
                        scale_dtype=torch.float16 if c["sdt"] == "f16" else torch.float32)
    assert all(v == 0 for v in qsa.debug_counters()), f"{label}: counters not at rest"
