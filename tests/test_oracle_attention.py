"""Pins for the oracle's attention: library routines, closed forms and
invariants that hold independently of how the oracle is written.

The operation is the packed one-query decode of the page "fix(qsa): restore
SM121 correctness with Humanize and Kernel Design Agent" (section
"Changes"), with order and duplicates of the index list kept as on the page
"[Kernel][WIP] Integrate native FlashInfer SM70 batch GDN and QSA probes".
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth

SM = 1.0 / 16.0


def _bf16(x):
    return torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)


def _pools(slots, hkv, rng):
    k = synth.normal_bf16(rng, (slots, hkv, 256))
    v = synth.normal_bf16(rng, (slots, hkv, 256))
    return k, v


def _sdpa_reference(q, k, v, sel, cu):
    """float64 attention through torch's own routines: index_select gathers
    the rows, scaled_dot_product_attention does softmax(q k^T * scale) v,
    logsumexp gives the log-normaliser."""
    bs, hq, _ = q.shape
    hkv = k.shape[1]
    out = torch.zeros(bs, hq, 256, dtype=torch.float64)
    lse = torch.full((bs, hq), -math.inf, dtype=torch.float64)
    for b in range(bs):
        idx = torch.from_numpy(sel[cu[b]:cu[b + 1]].astype(np.int64))
        if idx.numel() == 0:
            continue
        kb = k.double().index_select(0, idx)          # [L, hkv, 256]
        vb = v.double().index_select(0, idx)
        for g in range(hkv):
            qg = q[b, 12 * g:12 * (g + 1)].double()[None]          # [1, 12, 256]
            kg = kb[:, g][None, None].expand(1, 12, -1, -1)         # [1, 12, L, 256]
            vg = vb[:, g][None, None].expand(1, 12, -1, -1)
            o = torch.nn.functional.scaled_dot_product_attention(
                qg[:, :, None, :], kg, vg, scale=SM)[0, :, 0]
            out[b, 12 * g:12 * (g + 1)] = o
            logits = torch.matmul(kb[:, g], q[b, 12 * g:12 * (g + 1)].double().T) * SM
            lse[b, 12 * g:12 * (g + 1)] = torch.logsumexp(logits, dim=0)
    return out.numpy(), lse.numpy()


@pytest.mark.parametrize("hkv", [1, 2])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_matches_torch_sdpa_float64(hkv, seed):
    rng = np.random.default_rng(seed)
    slots = 40
    k, v = _pools(slots, hkv, rng)
    bs = 4
    q = synth.normal_bf16(rng, (bs, 12 * hkv, 256))
    lists = [synth.draw_indices(rng, n, slots, dup_prob=0.3) for n in (1, 5, 16, 11)]
    sel, cu = synth.pack(lists)
    o, l = oracle.decode(q, k, v, sel, cu)
    o_ref, l_ref = _sdpa_reference(q, k, v, sel, cu)
    np.testing.assert_allclose(o, o_ref, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(l, l_ref, rtol=1e-12, atol=1e-12)


def test_single_index_returns_that_row():
    rng = np.random.default_rng(5)
    k, v = _pools(16, 2, rng)
    q = synth.normal_bf16(rng, (1, 24, 256))
    sel, cu = synth.pack([[7]])
    o, l = oracle.decode(q, k, v, sel, cu)
    for h in range(24):
        g = h // 12
        np.testing.assert_array_equal(o[0, h], v[7, g].double().numpy())
        # lse of a single logit is that logit: s = q.k / 16
        s = float(np.dot(q[0, h].double().numpy(), k[7, g].double().numpy())) / 16
        assert abs(l[0, h] - s) <= 1e-12 * max(1.0, abs(s))


def test_identical_keys_give_mean_of_values():
    rng = np.random.default_rng(6)
    k, v = _pools(32, 1, rng)
    # distinct slots whose K rows are copies of one row
    k[3:9] = k[3]
    q = synth.normal_bf16(rng, (1, 12, 256))
    sel, cu = synth.pack([[3, 4, 5, 6, 7, 8]])
    o, l = oracle.decode(q, k, v, sel, cu)
    mean_v = v[3:9, 0].double().mean(dim=0).numpy()
    s = (q[0].double() @ k[3, 0].double()).numpy() / 16
    for h in range(12):
        np.testing.assert_allclose(o[0, h], mean_v, rtol=1e-12, atol=1e-14)
        assert abs(l[0, h] - (s[h] + math.log(6))) < 1e-12


def test_zero_query_gives_mean_and_log_length():
    rng = np.random.default_rng(7)
    k, v = _pools(64, 2, rng)
    q = torch.zeros(1, 24, 256, dtype=torch.bfloat16)
    idx = synth.draw_indices(rng, 37, 64)
    sel, cu = synth.pack([idx])
    o, l = oracle.decode(q, k, v, sel, cu)
    for g in range(2):
        mean_v = v[torch.from_numpy(idx.astype(np.int64)), g].double().mean(0).numpy()
        for h in range(12 * g, 12 * g + 12):
            np.testing.assert_allclose(o[0, h], mean_v, rtol=1e-12, atol=1e-14)
            assert abs(l[0, h] - math.log(37)) < 1e-13


def _one_hot_setup(a, b0, b1, v0, v1):
    """q = a e_0 and k_i = b_i e_0, so the logits are s_i = a b_i / 16
    exactly; values v_i are constant vectors."""
    q = torch.zeros(1, 12, 256, dtype=torch.bfloat16)
    q[0, :, 0] = a
    k = torch.zeros(3, 1, 256, dtype=torch.bfloat16)
    k[0, 0, 0] = b0
    k[1, 0, 0] = b1
    v = torch.zeros(3, 1, 256, dtype=torch.bfloat16)
    v[0, 0, :] = v0
    v[1, 0, :] = v1
    return q, k, v


def test_two_rows_closed_form():
    a, b0, b1, v0, v1 = 3.0, 2.5, -1.25, 0.75, -2.0
    q, k, v = _one_hot_setup(a, b0, b1, v0, v1)
    sel, cu = synth.pack([[0, 1]])
    o, l = oracle.decode(q, k, v, sel, cu)
    s0, s1 = a * b0 / 16, a * b1 / 16
    sig = 1.0 / (1.0 + math.exp(-(s0 - s1)))
    expect = sig * v0 + (1 - sig) * v1
    np.testing.assert_allclose(o[0], np.full((12, 256), expect), rtol=1e-13)
    np.testing.assert_allclose(l[0], np.full(12, max(s0, s1) + math.log1p(math.exp(-abs(s0 - s1)))),
                               rtol=1e-13)


def test_duplicate_equals_log2_logit_shift():
    a, b0, b1, v0, v1 = -2.0, 1.5, 4.0, 1.25, 0.5
    q, k, v = _one_hot_setup(a, b0, b1, v0, v1)
    sel, cu = synth.pack([[0, 0, 1]])
    o, l = oracle.decode(q, k, v, sel, cu)
    s0, s1 = a * b0 / 16 + math.log(2), a * b1 / 16
    sig = 1.0 / (1.0 + math.exp(-(s0 - s1)))
    np.testing.assert_allclose(o[0], np.full((12, 256), sig * v0 + (1 - sig) * v1), rtol=1e-13)
    np.testing.assert_allclose(l[0], np.full(12, math.log(math.exp(s0) + math.exp(s1))), rtol=1e-13)


def _merge(parts):
    """Combine per-chunk (o_i, lse_i): lse = logsumexp_i lse_i,
    o = sum_i exp(lse_i - lse) o_i.  Empty chunks carry lse = -inf."""
    lses = np.stack([p[1] for p in parts])
    m = np.max(lses, axis=0)
    w = np.exp(lses - m)
    lse = m + np.log(w.sum(axis=0))
    o = sum(np.exp(p[1] - lse)[..., None] * p[0] for p in parts)
    return o, lse


@pytest.mark.parametrize("cuts", [[0, 100, 300], [0, 0, 50, 50, 300], [0, 1, 2, 299, 300],
                                  [0, 150, 150, 300]])
def test_split_invariance(cuts):
    rng = np.random.default_rng(11)
    k, v = _pools(500, 2, rng)
    q = synth.normal_bf16(rng, (1, 24, 256))
    idx = synth.draw_indices(rng, 300, 500, dup_prob=0.1)
    whole = oracle.decode(q, k, v, *synth.pack([idx]))
    parts = []
    for a, b in zip(cuts[:-1], cuts[1:]):
        parts.append(oracle.decode(q, k, v, *synth.pack([idx[a:b]])))
    o, lse = _merge(parts)
    np.testing.assert_allclose(o, whole[0], rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(lse, whole[1], rtol=1e-12)


def test_permutation_invariance():
    rng = np.random.default_rng(12)
    k, v = _pools(200, 1, rng)
    q = synth.normal_bf16(rng, (1, 12, 256))
    idx = synth.draw_indices(rng, 150, 200, dup_prob=0.2)
    a = oracle.decode(q, k, v, *synth.pack([idx]))
    b = oracle.decode(q, k, v, *synth.pack([rng.permutation(idx)]))
    np.testing.assert_allclose(a[0], b[0], rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(a[1], b[1], rtol=1e-12)


def test_tp1_equals_two_tp2_calls():
    """Q heads 0-11 read KV head 0 and heads 12-23 read KV head 1."""
    rng = np.random.default_rng(13)
    k, v = _pools(100, 2, rng)
    q = synth.normal_bf16(rng, (3, 24, 256))
    sel, cu = synth.pack([synth.draw_indices(rng, n, 100) for n in (9, 40, 2)])
    o, l = oracle.decode(q, k, v, sel, cu)
    for g in range(2):
        og, lg = oracle.decode(q[:, 12 * g:12 * g + 12].contiguous(), k[:, g:g + 1].contiguous(),
                               v[:, g:g + 1].contiguous(), sel, cu)
        np.testing.assert_array_equal(o[:, 12 * g:12 * g + 12], og)
        np.testing.assert_array_equal(l[:, 12 * g:12 * g + 12], lg)


def test_controls_k_zero_v_zero_v_doubled():
    rng = np.random.default_rng(14)
    k, v = _pools(64, 2, rng)
    q = synth.normal_bf16(rng, (2, 24, 256))
    sel, cu = synth.pack([synth.draw_indices(rng, n, 64) for n in (20, 33)])
    base_o, base_l = oracle.decode(q, k, v, sel, cu)
    # K := 0 -> uniform weights: mean of the listed V rows, lse = ln L
    o, l = oracle.decode(q, torch.zeros_like(k), v, sel, cu)
    for b, n in enumerate((20, 33)):
        idx = torch.from_numpy(sel[cu[b]:cu[b + 1]].astype(np.int64))
        for h in range(24):
            np.testing.assert_allclose(o[b, h], v[idx, h // 12].double().mean(0).numpy(), rtol=1e-12,
                                       atol=1e-14)
            assert abs(l[b, h] - math.log(n)) < 1e-13
    # V := 0 -> o = 0
    o, _ = oracle.decode(q, k, torch.zeros_like(v), sel, cu)
    assert not o.any()
    # V -> 2V -> o -> 2o exactly (x2 is exact in bf16 and double)
    o, l = oracle.decode(q, k, v * 2, sel, cu)
    np.testing.assert_array_equal(o, 2 * base_o)
    np.testing.assert_array_equal(l, base_l)


def test_empty_row():
    rng = np.random.default_rng(15)
    k, v = _pools(10, 1, rng)
    q = synth.normal_bf16(rng, (3, 12, 256))
    sel, cu = synth.pack([[1, 2], [], [3]])
    o, l = oracle.decode(q, k, v, sel, cu)
    assert not o[1].any()
    assert np.all(np.isneginf(l[1]))
    assert np.all(np.isfinite(l[[0, 2]]))


def test_rejects_contract_violations():
    rng = np.random.default_rng(16)
    k, v = _pools(10, 1, rng)
    q = synth.normal_bf16(rng, (1, 12, 256))
    with pytest.raises(ValueError, match="2055"):
        oracle.decode(q, k, v, np.zeros(2056, np.int32), np.array([0, 2056], np.int32))
    with pytest.raises(ValueError, match="slot"):
        oracle.decode(q, k, v, np.array([10], np.int32), np.array([0, 1], np.int32))
    with pytest.raises(ValueError, match="cu_seqlens"):
        oracle.decode(q, k, v, np.array([1, 2], np.int32), np.array([2, 1], np.int32))
    assert oracle.decode(q, k, v, np.zeros(2055, np.int32), np.array([0, 2055], np.int32))


def test_bf16_exact_widening():
    """bf16 inputs are widened exactly: a row of chosen bf16 values comes
    back bit for bit through a single-index call."""
    vals = np.array([1.0, -2.0, 0.5, 3.140625, -1e-3, 65280.0, 1e-38, 0.0] * 32, np.float32)
    v = _bf16(vals).reshape(1, 1, 256)
    k = torch.zeros_like(v)
    q = torch.zeros(1, 12, 256, dtype=torch.bfloat16)
    o, _ = oracle.decode(q, k, v, np.array([0], np.int32), np.array([0, 1], np.int32))
    np.testing.assert_array_equal(o[0, 0], v[0, 0].double().numpy())
