"""Pins for the oracle's dequantization and the write-side quantizers.

Sources: page "feat(qsa): quantized KV pools with dequant-on-gather
(fp8/int8/int4)", part 4 "Modifications" (pool layouts, int4 nibble order,
offset-binary codes, rint ties, fp16 scale clamp, registered unit tests and
their error bands) and "Motivation" (bytes per token).  The fp8 format is
OCP e4m3fn; torch's float8_e4m3fn is the library routine it is pinned to.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import layout, quant

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_fp8_e4m3fn_decode_exhaustive_vs_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).double().numpy()
    got = np.array([oracle.fp8_e4m3fn_to_double(c) for c in range(256)])
    nan = np.isnan(ref)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan], ref[~nan])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9


def _row_pool(codes_row: np.ndarray, scale_row: np.ndarray):
    return codes_row.reshape(1, 1, -1), scale_row.reshape(1, 1, -1).astype(np.float32)


def test_int4_nibble_order_and_offset_binary():
    # byte i holds channel 2i in its low nibble and channel 2i+1 in its high
    # nibble; a nibble n stands for the code n - 8
    packed = np.zeros(128, np.uint8)
    packed[0] = 0x9F          # ch0: 0xF -> +7, ch1: 0x9 -> +1
    packed[1] = 0x08          # ch2: 0x8 -> 0,  ch3: 0x0 -> -8
    packed[2] = 0x71          # ch4: 0x1 -> -7, ch5: 0x7 -> -1
    packed[3:] = 0x88
    scales = np.array([0.5] + [2.0] * 7, np.float32)   # group 0 = channels 0..31
    pool, sc = _row_pool(packed, scales)
    row = oracle.dequant_row(pool, sc, 0, 0, fmt="int4", group=32)
    np.testing.assert_array_equal(row[:6], [3.5, 0.5, 0.0, -4.0, -3.5, -0.5])
    assert not row[6:].any()


def test_int8_and_fp8_row_dequant():
    codes = np.arange(-128, 128, dtype=np.int8)
    scales = np.array([0.25, 1.0, 2.0, 0.125], np.float32)        # 64-channel groups
    pool, sc = _row_pool(codes.view(np.uint8), scales)
    row = oracle.dequant_row(pool, sc, 0, 0, fmt="int8", group=64)
    expect = codes.astype(np.float64) * np.repeat(scales.astype(np.float64), 64)
    np.testing.assert_array_equal(row, expect)

    fp8 = np.array([0x38, 0xB8, 0x7E, 0x01, 0x00, 0x80, 0x3C, 0x41] * 32, np.uint8)
    pool, sc = _row_pool(fp8, np.array([3.0], np.float32))
    row = oracle.dequant_row(pool, sc, 0, 0, fmt="fp8", group=256)
    ref = torch.from_numpy(fp8).view(torch.float8_e4m3fn).double().numpy() * 3.0
    np.testing.assert_array_equal(row, ref)


def test_quantized_pool_through_decode_equals_dequantized_bf16_free_path():
    """Decode over quantized pools equals plain softmax attention over the
    dequantized values (the decode path is unchanged by dequantization)."""
    rng = np.random.default_rng(21)
    x = synth.normal_bf16(rng, (50, 2, 256))
    y = synth.normal_bf16(rng, (50, 2, 256))
    q = synth.normal_bf16(rng, (2, 24, 256))
    sel, cu = synth.pack([synth.draw_indices(rng, n, 50, 0.2) for n in (17, 30)])
    for fmt, group in (("fp8", 256), ("int8", 256), ("int8", 64), ("int4", 32)):
        kc, ks = quant.quantize(x, fmt, group)
        vc, vs = quant.quantize(y, fmt, group)
        o, l = oracle.decode(q, kc, vc, sel, cu, fmt=fmt, group=group, k_scale=ks, v_scale=vs)
        kd = torch.from_numpy(quant.dequantize(kc, ks, fmt, group))
        vd = torch.from_numpy(quant.dequantize(vc, vs, fmt, group))
        for b in range(2):
            idx = torch.from_numpy(sel[cu[b]:cu[b + 1]].astype(np.int64))
            for g in range(2):
                qg = q[b, 12 * g:12 * g + 12].double()
                logits = qg @ kd[idx, g].T / 16
                p = torch.softmax(logits, dim=-1)
                np.testing.assert_allclose(o[b, 12 * g:12 * g + 12], (p @ vd[idx, g]).numpy(),
                                           rtol=1e-10, atol=1e-12)
                np.testing.assert_allclose(l[b, 12 * g:12 * g + 12],
                                           torch.logsumexp(logits, -1).numpy(), rtol=1e-12)


def test_rint_ties_to_even():
    # absmax 127 -> int8 scale exactly 1; absmax 7 -> int4 scale exactly 1
    x = np.zeros(256, np.float32)
    x[:7] = [127.0, 2.5, 3.5, -2.5, 0.5, 1.5, -126.5]
    codes, scale = quant.quantize_int8(x[None], 256)
    assert scale[0, 0] == 1.0
    np.testing.assert_array_equal(codes[0, :7], [127, 2, 4, -2, 0, 2, -126])
    x4 = np.zeros(256, np.float32)
    x4[:6] = [7.0, 2.5, 3.5, -0.5, 6.5, -5.5]
    packed, scale4 = quant.quantize_int4(x4[None], 32)
    assert scale4[0, 0] == 1.0
    np.testing.assert_array_equal(quant.unpack_int4(packed)[0, :6], [7, 2, 4, 0, 6, -6])


def test_int4_pack_layout():
    x = np.zeros(256, np.float32)
    x[0::2] = 7.0
    x[1::2] = -7.0
    packed, scale = quant.quantize_int4(x[None], 32)
    assert np.all(scale == 1.0)
    # even channel +7 -> nibble 15 (low), odd channel -7 -> nibble 1 (high)
    assert np.all(packed == 0x1F)


def test_fp16_scale_clamp_and_zero_groups():
    x = np.zeros((2, 256), np.float32)
    x[0, 0] = 1e7
    _, s8 = quant.quantize_int8(x, 64, "f16")
    _, s4 = quant.quantize_int4(x, 32, "f16")
    assert s8[0, 0] == 65504.0 and s4[0, 0] == 65504.0
    assert np.all(s8[1] == 0) and np.all(s4[1] == 0)
    c8, _ = quant.quantize_int8(x, 64, "f16")
    assert c8[0, 0] == 127 and not c8[1].any()
    c4, _ = quant.quantize_int4(x, 32, "f16")
    assert np.all(c4[1] == 0x88)


def test_fp8_saturates_never_nan():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((64, 256)).astype(np.float32) * 1e4
    x[0, :4] = [3e38, -3e38, 1e-45, 0.0]
    codes, scale = quant.quantize_fp8(x, 256)
    assert not np.isin(codes, [0x7F, 0xFF]).any()
    assert np.all(np.isfinite(scale))
    # the absmax element of each row lands on +-448
    top = np.abs(codes.view(np.uint8) & 0x7F).max(axis=1)
    assert np.all(top == 0x7E)


def test_error_bands_from_pages():
    bands = json.load(open(os.path.join(GOLDEN, "quant_error_bands.json")))["bands"]
    rng = np.random.default_rng(30)
    x3 = rng.standard_normal((4096, 256)).astype(np.float32) * 3
    c, s = quant.quantize_int8(x3, 64, "f16")
    r = quant.rel_rms(x3, quant.dequantize(c, s, "int8", 64))
    assert r < bands["int8_g64_fp16scale_N(0,3)"]["upper"]
    assert abs(r - 0.0062) < 0.1 * 0.0062           # printed: 0.62 %
    c, s = quant.quantize_int4(x3, 32, "f16")
    r = quant.rel_rms(x3, quant.dequantize(c, s, "int4", 32))
    b = bands["int4_g32_fp16scale"]
    assert b["lower"] < r < b["upper"]
    c, s = quant.quantize_fp8(x3, 256)
    r = quant.rel_rms(x3, quant.dequantize(c, s, "fp8", 256))
    b = bands["fp8_e4m3_N(0,3)"]
    assert b["lower"] < r < b["upper"]


def test_layout_bytes_per_token_match_pages():
    gold = json.load(open(os.path.join(GOLDEN, "pool_layout_bytes.json")))
    ex = gold["exact_bytes"]
    assert layout.bytes_per_token("bf16") == ex["bf16"]
    assert layout.bytes_per_token("int8", 64) == ex["int8_g64"]
    assert layout.bytes_per_token("int4", 32) == ex["int4_g32"]
    t = gold["tiered"]
    tiered = layout.tiered_bytes_per_token(t["ring_slots"], t["context"])
    assert round(tiered) == ex["tiered_int8ring8192_int4_at_256k"]
    # printed rounded figures
    assert math.isclose(ex["int8_g64"] / 1024, 12.4, abs_tol=0.05)
    assert ex["int4_g32"] / 1024 == 6.75
    assert ex["bf16"] / 1024 == 24


def test_quantizer_roundtrip_codes_are_reproduced():
    """Codes re-quantized from their own dequantized values come back
    unchanged (the scale is stored and the codes are its exact multiples)."""
    rng = np.random.default_rng(31)
    x = rng.standard_normal((256, 256)).astype(np.float32)
    for fmt, group in (("int8", 64), ("int8", 256), ("int4", 32)):
        c, s = quant.quantize(x, fmt, group)
        xr = quant.dequantize(c, s, fmt, group).astype(np.float32)
        c2, s2 = quant.quantize(xr, fmt, group)
        np.testing.assert_array_equal(s2, s)
        np.testing.assert_array_equal(c2, c)
