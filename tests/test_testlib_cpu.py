"""The GPU tests' comparison, checked on the CPU with planted mistakes.

The per-(row, head) bound of qsa_testlib.compare must pass a correctly
rounded output, and fail an output whose error is confined to one head
even when the whole-tensor relative L2 stays under 2e-3 (page "fix(qsa):
restore SM121 correctness with Humanize and Kernel Design Agent", section
"Optimized kernel", gives the whole-tensor threshold only).
"""
import numpy as np
import pytest
import torch

from qsa_testlib import bf16_round, compare, head_report


def _ref(seed=5, rows=8, heads=24):
    rng = np.random.default_rng(seed)
    o = rng.standard_normal((rows, heads, 256)) * rng.uniform(0.1, 3.0, (rows, heads, 1))
    lse = rng.standard_normal((rows, heads))
    return o, lse


def test_bf16_round_matches_torch_on_float32_values():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(200_000).astype(np.float32),
                        (rng.standard_normal(1000) * 1e-30).astype(np.float32),
                        np.float32([0.0, -0.0, 1.0, 65504.0, 3.0e38])])
    # exact ties: the low 16 bits of the float32 pattern are 0x8000
    ties = (rng.integers(0, 1 << 15, 5000).astype(np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties[np.isfinite(ties)]])
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(bf16_round(x.astype(np.float64)), want)


def test_correctly_rounded_output_passes():
    o_ref, l_ref = _ref()
    out = bf16_round(o_ref)
    compare(out, l_ref, o_ref, l_ref, np.full(o_ref.shape[0], 7), label="rounded")
    rel, floor = head_report(out, o_ref)
    np.testing.assert_allclose(rel, floor, rtol=0, atol=1e-15)
    assert floor.max() <= 2.0 ** -8


def test_error_confined_to_one_head_fails():
    o_ref, l_ref = _ref(rows=128)  # bs=128 TP1: 3072 heads
    o_ref /= np.linalg.norm(o_ref, axis=-1, keepdims=True)
    out = bf16_round(o_ref)
    out[3, 17] = bf16_round(o_ref[3, 17] * 1.06)   # a 6% error in one head's output
    diff = out - o_ref
    whole = np.sqrt(np.sum(diff ** 2) / np.sum(o_ref ** 2))
    assert whole <= 2e-3  # the whole-tensor threshold alone lets it through
    with pytest.raises(AssertionError, match="head \\(row 3, h 17\\)"):
        compare(out, l_ref, o_ref, l_ref, np.full(o_ref.shape[0], 7), label="planted")


def test_head_error_of_half_the_budget_fails_and_a_tenth_passes():
    """A random-direction error adds to the rounding error in quadrature:
    an error e (relative to the head's norm) raises rel_h to about
    sqrt(floor^2 + e^2), so 1e-3 (half the whole-tensor budget) in one head
    exceeds floor + 2e-4 and fails, while 1e-4 passes."""
    o_ref, l_ref = _ref(seed=9)
    n = np.linalg.norm(o_ref[5, 2])
    direction = np.random.default_rng(3).standard_normal(256)
    direction /= np.linalg.norm(direction)
    for e, ok in ((1e-3, False), (1e-4, True)):
        out = bf16_round(o_ref + 0.0)
        out[5, 2] = bf16_round(o_ref[5, 2] + e * n * direction)  # error before the rounding
        if ok:
            compare(out, l_ref, o_ref, l_ref, np.full(o_ref.shape[0], 3), label="small")
        else:
            with pytest.raises(AssertionError, match="exceeds its bf16 floor"):
                compare(out, l_ref, o_ref, l_ref, np.full(o_ref.shape[0], 3), label="large")


def test_zero_reference_head_must_be_zero():
    o_ref, l_ref = _ref()
    o_ref[1, 4] = 0.0
    out = bf16_round(o_ref)
    compare(out, l_ref, o_ref, l_ref, np.full(o_ref.shape[0], 2), label="zero head")
    out[1, 4, 7] = 1e-6
    with pytest.raises(AssertionError):
        compare(out, l_ref, o_ref, l_ref, np.full(o_ref.shape[0], 2), label="zero head nonzero")
