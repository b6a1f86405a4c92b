"""Pins of the oracle's MX (E8M0-scaled E4M3) codec, exhaustively (CPU only)."""
import json
import os

import numpy as np

import bruteforce as bfc
import workloads as wk

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_ocp_points.json")


def test_decode_table_from_format_definition(orc):
    ref = bfc.e4m3_values()
    for c in range(256):
        v = orc.e4m3_decode(c)
        assert (np.isnan(v) and np.isnan(ref[c])) or v == ref[c]


def test_decode_matches_spec_points(orc):
    # points stated by the OCP 8-bit floating point specification (OFP8) for E4M3
    pts = json.load(open(GOLDEN))["points"]
    for p in pts:
        v = orc.e4m3_decode(int(p["code"], 16))
        if p["value"] == "nan":
            assert np.isnan(v)
        else:
            assert v == float(p["value"]), p


def test_encode_exhaustive_bf16_against_nearest_search(orc):
    # every non-negative finite bf16 value, scaled by 2^-s for a spread of scales, encodes
    # to the nearest E4M3 code (ties to even, saturating)
    bits = np.arange(0, 0x7F80, dtype=np.uint16)
    vals = wk.bf16_bits_to_f32(bits).astype(np.float64)
    for s in range(-20, 21, 4):
        a = vals * 2.0 ** s
        a = a[a <= 1e6]
        ref = bfc.e4m3_nearest(a)
        got = np.array([orc.e4m3_encode(v) for v in a], np.uint8)
        assert np.array_equal(got, ref), s
        neg = np.array([orc.e4m3_encode(-v) for v in a[1:]], np.uint8)
        assert np.array_equal(neg, ref[1:] | 0x80)


def test_block_scale_rules(orc):
    rs = np.random.default_rng(9)
    a = rs.standard_normal((64, 128)) * np.exp2(rs.integers(-30, 30, size=(64, 1)))
    a[3] = 0.0
    codes, scales = orc.mx_quantize(a)
    assert scales[3].max() == 0 and codes[3].max() == 0
    deq = orc.mx_dequantize(codes, scales)
    blocks = a.reshape(64, 4, 32)
    for r in range(64):
        for b in range(4):
            amax = np.abs(blocks[r, b]).max()
            if amax == 0:
                continue
            X = 2.0 ** (int(scales[r, b]) - 127)
            # the block maximum lands in [256, 512) before saturation at 448
            assert 256 <= amax / X < 512
            q = codes[r].reshape(4, 32)[b]
            top = np.abs(np.array([orc.e4m3_decode(c) for c in q])).max()
            assert 256 <= top <= 448
            # every element is within half a step of E4M3 (relative 2^-4) or saturated
            d = deq[r].reshape(4, 32)[b]
            v = blocks[r, b]
            ok = (np.abs(d - v) <= np.abs(v) * 2.0 ** -4 + X * 2.0 ** -10) | (np.abs(v) / X > 448)
            assert ok.all()
    # powers of two within range round-trip exactly
    p2 = np.exp2(np.arange(-20, 20, dtype=np.float64))[None, :32].repeat(2, 0)
    c2, s2 = orc.mx_quantize(p2)
    back = orc.mx_dequantize(c2, s2)
    big = p2 / 2.0 ** (int(s2[0, 0]) - 127) >= 2.0 ** -9
    assert np.array_equal(back[big], p2[big])


def test_ceil_mode_never_saturates(orc):
    rs = np.random.default_rng(10)
    a = rs.standard_normal((16, 64))
    codes, scales = orc.mx_quantize(a, mode=1)
    X = np.exp2(scales.astype(np.int64) - 127)
    amax = np.abs(a).reshape(16, 2, 32).max(-1)
    # the smallest power of two that keeps the block maximum within 448
    assert np.all(amax / X <= 448) and np.all(amax / (X / 2) > 448)
