"""Pins of the oracle's 4-bit group encoding (the scheme is this project's
reading; the pages name 4-bit KV caches without a scheme: xllm-io review,
section 五 量化组合).

* a hand-built group whose scale and zero-point are exact in fp16 gives known
  codes (tests/golden/int4_quarter_steps.txt);
* codes lie in 0..15, the group minimum maps to 0 and the maximum to 15;
* the round trip error is within half a step plus the fp16 rounding of s and z;
* a constant group has s = 0 and all codes 0 and decodes exactly;
* packing round-trips and puts the even channel in the low nibble.
"""
import os

import numpy as np

import oracle
from duo_synth import rng, normal, round_fp16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load_golden():
    vals, codes, packed, s, z = [], [], None, None, None
    with open(os.path.join(GOLDEN, "int4_quarter_steps.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            parts = line.split()
            if parts[0] == "packed":
                packed = [int(x, 16) for x in parts[1:]]
            elif parts[0] == "s":
                s = int(parts[1], 16)
            elif parts[0] == "z":
                z = int(parts[1], 16)
            else:
                vals.append(float(parts[1]))
                codes.append(int(parts[2]))
    return np.array(vals, np.float32), np.array(codes), np.array(packed, np.uint8), s, z


def test_hand_built_group():
    vals, codes, packed, s_bits, z_bits = _load_golden()
    c, s, z = oracle.quantize_int4_g32(vals[None])
    np.testing.assert_array_equal(c[0], codes)
    assert s.view(np.uint16)[0, 0] == s_bits
    assert z.view(np.uint16)[0, 0] == z_bits
    np.testing.assert_array_equal(oracle.pack_nibbles(c[0]), packed)
    np.testing.assert_array_equal(oracle.dequantize_int4_g32(c, s, z)[0], vals)


def test_code_range_and_extremes():
    g = rng(31)
    x = round_fp16(normal(g, (2000, 128)))
    c, s, z = oracle.quantize_int4_g32(x)
    assert c.min() == 0 and c.max() == 15
    grp = x.reshape(2000, 4, 32)
    cg = c.reshape(2000, 4, 32)
    rows = np.arange(2000)[:, None]
    heads = np.arange(4)[None, :]
    assert (cg[rows, heads, grp.argmin(axis=-1)] == 0).all()
    assert (cg[rows, heads, grp.argmax(axis=-1)] == 15).all()


def test_round_trip_error_bound():
    g = rng(32)
    x = round_fp16(normal(g, (4000, 128)) * 3.0)
    c, s, z = oracle.quantize_int4_g32(x)
    xh = oracle.dequantize_int4_g32(c, s, z)
    s32 = s.astype(np.float32)
    z32 = z.astype(np.float32)
    ulp16 = lambda a: np.spacing(np.abs(a).astype(np.float16)).astype(np.float32)
    bound = s32 / 2 + ulp16(z32) + 7.5 * ulp16(s32) + np.spacing(np.float32(8.0))
    err = np.abs(x - xh).reshape(4000, 4, 32).max(axis=-1)
    assert (err <= bound).all()
    # and the encoding is not trivially lossless: the error is of order s/4
    assert err.mean() > 0.1 * s32.mean()


def test_constant_group():
    x = np.full((3, 32), 1.5, np.float32)
    c, s, z = oracle.quantize_int4_g32(x)
    assert (s == 0).all() and (c == 0).all()
    np.testing.assert_array_equal(oracle.dequantize_int4_g32(c, s, z), x)


def test_rint_ties_to_even():
    # group with min 0 and max 15*0.5: s = 0.5; values 0.25 and 0.75 sit on
    # half-steps (0.5 and 1.5 steps) and round to codes 0 and 2 (ties to even)
    x = np.zeros((1, 32), np.float32)
    x[0, 1] = 7.5
    x[0, 2] = 0.25
    x[0, 3] = 0.75
    c, s, z = oracle.quantize_int4_g32(x)
    assert float(s[0, 0]) == 0.5 and float(z[0, 0]) == 0.0
    assert list(c[0, :4]) == [0, 15, 0, 2]


def test_pack_roundtrip():
    g = rng(33)
    c = g.integers(0, 16, size=(10, 128)).astype(np.uint8)
    p = oracle.pack_nibbles(c)
    assert p.shape == (10, 64)
    np.testing.assert_array_equal(p & 0xF, c[:, 0::2])
    np.testing.assert_array_equal(oracle.unpack_nibbles(p), c)
