"""Pins for the oracle's QSA indexer step (qsa_index_oracle.c).

Sources: page "[Kernel][WIP] Integrate native FlashInfer SM70 batch GDN and
QSA probes", follow-up "device-planned MQA and QSA quality attribution" (MQA
scoring + exact top-k + index expansion, 256K-token capacity), and page
"feat(qsa): quantized KV pools with dequant-on-gather (fp8/int8/int4)", part
4 decode routing paragraph (row width token_topk + compress_ratio - 1,
tests/golden/index_row_width.json).  The scoring formula, the tie rule and
the expansion order are this build's reading (stated in the oracle's
header); the pins check the oracle against float64 arithmetic, numpy's sort
and closed forms, never against its own code.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def make_inputs(rng, ctx, **kw):
    return synth.index_inputs(rng, ctx, **kw)


def run(inp, budget, c, **kw):
    return oracle.index(inp["q"], inp["k_pool"], inp["block_table"], inp["req_to_token"],
                        inp["ctx_len"], budget=budget, compress_ratio=c, weights=inp["weights"],
                        **kw)


def positions(sel_row, r2t_row):
    """Logical token positions of a row's slot ids (r2t rows are injective)."""
    inv = {int(s): p for p, s in enumerate(r2t_row)}
    return np.array([inv[int(s)] for s in sel_row])


def test_scores_within_fp32_bound_of_float64():
    rng = np.random.default_rng(61)
    inp = make_inputs(rng, [4000, 37, 513], hi=8, di=128)
    _, _, sc = run(inp, 256, 4, return_scores=True)
    q = inp["q"].double()
    k = inp["k_pool"].double()
    w = torch.from_numpy(inp["weights"]).double()
    for b, t in enumerate(inp["ctx_len"]):
        n = t // 4
        keys = k[torch.from_numpy(inp["block_table"][b, :n].astype(np.int64))]
        per_head = keys @ q[b].T                                  # [n, hi]
        exact = (per_head * w[b]).sum(-1).numpy()
        mag = ((keys.abs() @ q[b].abs().T) * w[b]).sum(-1).numpy()
        bound = (128 + 8 + 2) * 2.0 ** -24 * mag
        err = np.abs(sc[b, :n].astype(np.float64) - exact)
        assert np.all(err <= bound), float((err / np.maximum(bound, 1e-30)).max())
        assert np.all(np.isnan(sc[b, n:]))


def test_one_hot_scores_are_exact():
    """q_h = a_h e_0, k_j = b_j e_0: s_j = b_j * sum_h w_h a_h exactly."""
    bs, hi, di, c = 1, 3, 16, 2
    a = np.array([0.5, 2.0, -1.0], np.float32)
    bvals = np.array([1, -3, 5, 0.25, 7, -0.5, 2, 4], np.float32)
    q = np.zeros((bs, hi, di), np.float32)
    q[0, :, 0] = a
    kp = np.zeros((8, di), np.float32)
    kp[:, 0] = bvals
    w = np.array([[1.0, 0.25, 0.5]], np.float32)              # sum_h w_h a_h = 0.5
    inp = dict(q=synth.to_bf16(q), k_pool=synth.to_bf16(kp),
               block_table=np.arange(8, dtype=np.int32)[None], req_to_token=np.arange(16, dtype=np.int32)[None],
               ctx_len=np.array([16], np.int32), weights=w)
    sel, cu, sc = run(inp, 6, c, return_scores=True)
    expect = bvals * np.float32((w[0] * a).sum())
    np.testing.assert_array_equal(sc[0], expect)
    top3 = np.sort(np.argsort(-expect, kind="stable")[:3])           # blocks 4, 2, 7
    assert list(top3) == [2, 4, 7]
    assert list(sel) == [4, 5, 8, 9, 14, 15]


@pytest.mark.parametrize("c,budget", [(4, 2048), (8, 2048), (16, 512), (4, 64)])
def test_topk_is_numpy_top_k_and_expansion_is_ordered(c, budget):
    rng = np.random.default_rng(62 + c)
    ctx = [20000, budget * 3 + c - 1, budget + 1, 7, 0, budget * 2]
    inp = make_inputs(rng, ctx, c=c)
    sel, cu, sc = run(inp, budget, c, return_scores=True)
    k_blocks = budget // c
    for b, t in enumerate(ctx):
        n = t // c
        row = sel[cu[b]:cu[b + 1]]
        assert len(row) == min(n, k_blocks) * c + t % c <= budget + c - 1
        pos = positions(row, inp["req_to_token"][b])
        assert np.all(np.diff(pos) > 0)                      # ascending logical order
        blocks = pos[: min(n, k_blocks) * c].reshape(-1, c)
        assert np.all(blocks == blocks[:, :1] + np.arange(c))  # whole blocks
        assert np.all(blocks[:, 0] % c == 0)
        assert list(pos[min(n, k_blocks) * c:]) == list(range(n * c, t))   # the tail
        chosen = blocks[:, 0] // c
        if n > k_blocks:
            ref = np.sort(np.argsort(-sc[b, :n], kind="stable")[:k_blocks])
            np.testing.assert_array_equal(chosen, ref)
        else:
            np.testing.assert_array_equal(chosen, np.arange(n))


def test_kept_blocks_are_a_top_k_under_float64_scores():
    """Whatever fp32 order the scores are evaluated in, the kept set must be
    a top-k of the exact (float64) scores up to the fp32 error bound
    (hi + di + 2) 2^-24 sum_h |w_h| |q_h| . |k_j| of each block: no dropped
    block may beat a kept one by more than their two bounds."""
    rng = np.random.default_rng(68)
    for hi, di in ((8, 128), (64, 64), (1, 128)):
        ctx = [8192, 3001, 2048 * 4 + 3]
        inp = make_inputs(rng, ctx, hi=hi, di=di, c=4)
        sel, cu = run(inp, 2048, 4)
        q = inp["q"].double()
        k = inp["k_pool"].double()
        w = torch.from_numpy(inp["weights"]).double()
        for b, t in enumerate(ctx):
            n, kb = t // 4, 512
            if n <= kb:
                continue
            keys = k[torch.from_numpy(inp["block_table"][b, :n].astype(np.int64))]
            exact = ((keys @ q[b].T) * w[b]).sum(-1).numpy()
            bound = (hi + di + 2) * 2.0 ** -24 * ((keys.abs() @ q[b].abs().T) * w[b].abs()).sum(-1).numpy()
            pos = positions(sel[cu[b]:cu[b + 1]], inp["req_to_token"][b])
            kept = np.zeros(n, bool)
            kept[pos[: kb * 4: 4] // 4] = True
            assert kept.sum() == kb
            assert (exact[kept] + bound[kept]).min() >= (exact[~kept] - bound[~kept]).max()


def test_ties_go_to_the_lower_block_index():
    rng = np.random.default_rng(63)
    inp = make_inputs(rng, [4096, 4096], c=4, hi=2, di=32)
    same = inp["k_pool"][0].clone()
    inp["k_pool"][:] = same                      # every block scores the same
    sel, cu = run(inp, 128, 4)
    for b in range(2):
        pos = positions(sel[cu[b]:cu[b + 1]], inp["req_to_token"][b])
        assert list(pos) == list(range(128))


def test_short_contexts_list_every_token_in_order():
    rng = np.random.default_rng(64)
    ctx = [1, 3, 4, 5, 100, 2051]
    inp = make_inputs(rng, ctx, c=4, max_tokens=2051)
    sel, cu = run(inp, 2048, 4)
    for b, t in enumerate(ctx):
        np.testing.assert_array_equal(sel[cu[b]:cu[b + 1]], inp["req_to_token"][b, :t])


def test_row_width_printed_on_the_pages():
    g = json.load(open(os.path.join(GOLDEN, "index_row_width.json")))
    rng = np.random.default_rng(65)
    c, budget = g["compress_ratio"], g["budget"]
    inp = make_inputs(rng, [budget * 5 + c - 1, 262144], c=c, hi=2, di=32)
    sel, cu = run(inp, budget, c)
    assert cu[1] - cu[0] == g["row_width"] == budget + c - 1
    assert cu[2] - cu[1] == budget                  # 262144 is a multiple of 4: no tail
    inp8 = make_inputs(rng, [budget * 3 + 7], c=8, hi=2, di=32)
    assert run(inp8, budget, 8)[1][1] == 2055


def test_indexer_output_feeds_the_decode():
    """The selected slots decode to softmax attention over exactly those
    tokens' K/V rows (composition with the decode oracle)."""
    rng = np.random.default_rng(66)
    ctx = [3000, 900]
    inp = make_inputs(rng, ctx, c=4, hi=2, di=32, max_tokens=3000)
    inp["req_to_token"] = np.stack([rng.permutation(8192)[:3000] for _ in ctx]).astype(np.int32)
    sel, cu = run(inp, 512, 4)
    kv = synth.normal_bf16(rng, (8192, 2, 256))
    vv = synth.normal_bf16(rng, (8192, 2, 256))
    qd = synth.normal_bf16(rng, (2, 24, 256))
    o, l = oracle.decode(qd, kv, vv, sel, cu)
    for b in range(2):
        idx = torch.from_numpy(sel[cu[b]:cu[b + 1]].astype(np.int64))
        for g in range(2):
            lg = qd[b, 12 * g:12 * g + 12].double() @ kv[idx, g].double().T / 16
            ref = torch.softmax(lg, -1) @ vv[idx, g].double()
            np.testing.assert_allclose(o[b, 12 * g:12 * g + 12], ref.numpy(), rtol=1e-10, atol=1e-12)


def test_rejections():
    rng = np.random.default_rng(67)
    inp = make_inputs(rng, [100], c=4)
    bad = dict(inp, ctx_len=np.array([101], np.int32))
    with pytest.raises(ValueError, match="context length"):
        run(bad, 64, 4)
    bt = inp["block_table"].copy()
    bt[0, 3] = 10 ** 6
    with pytest.raises(ValueError, match="block table"):
        run(dict(inp, block_table=bt), 64, 4)
