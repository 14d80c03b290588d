"""Pins of the oracle's number formats (E4M3, E2M1, E8M0, bf16, fp16) against
independent sources: torch's own casts, the OCP tables in tests/golden, and a
brute-force nearest-value search with exact rationals."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_e4m3_decode_matches_torch_all_codes(orc):
    codes = np.arange(256, dtype=np.uint8)
    ours = orc.e4m3_decode_array(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # signed zeros are distinct codes
    assert math.copysign(1.0, ours[0x80]) == -1.0


def test_e4m3_golden_points(orc):
    g = _gold("ocp_formats.json")["e4m3fn"]
    fp8max = _gold("fp8_max.json")["ocp_e4m3fn_max"]
    assert g["max"] == fp8max == 448.0
    assert orc.e4m3_decode(g["max_code"]) == 448.0
    for c in g["nan_codes"]:
        assert math.isnan(orc.e4m3_decode(c))
    assert orc.e4m3_decode(1) == g["min_subnormal"]
    assert orc.e4m3_decode(g["min_normal_code"]) == g["min_normal"]
    # largest finite magnitude of all non-NaN codes is FP8_MAX
    vals = [abs(orc.e4m3_decode(c)) for c in range(256) if c not in (127, 255)]
    assert max(vals) == fp8max


def test_e4m3_roundtrip_all_codes(orc):
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        assert orc.e4m3_encode(orc.e4m3_decode(c)) == c


def test_e4m3_midpoints_tie_to_even(orc):
    pos = sorted({orc.e4m3_decode(c) for c in range(0x7F)})
    for a, b in zip(pos[:-1], pos[1:]):
        mid = np.float32((a + b) / 2)
        assert float(mid) == (a + b) / 2        # midpoints are exact in fp32
        ca, cb = orc.e4m3_encode(a), orc.e4m3_encode(b)
        want = ca if ca % 2 == 0 else cb
        assert orc.e4m3_encode(float(mid)) == want, (a, b)
        assert orc.e4m3_encode(-float(mid)) == want | 0x80


def test_e4m3_encode_matches_torch_cast(orc):
    rng = np.random.default_rng(123)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * 50,
        rng.uniform(-464, 464, 20000).astype(np.float32),
        (rng.standard_normal(20000) * 2.0 ** -8).astype(np.float32),
        np.float32([464.0, -464.0, 463.99, 448.0, 1.0625, 1.1875, 3 * 2 ** -10, 2 ** -10]),
    ])
    ours = orc.e4m3_encode_array(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_saturates(orc):
    assert orc.e4m3_encode(465.0) == 0x7E
    assert orc.e4m3_encode(1e30) == 0x7E
    assert orc.e4m3_encode(-1e30) == 0xFE
    assert orc.e4m3_encode(float("inf")) == 0x7E


def _nearest_even(x: Fraction, table):
    """Brute force: nearest entry of a sorted table of (value, code), ties to
    the even code; saturates at the ends."""
    best = None
    for v, c in table:
        d = abs(Fraction(v) - x)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1]


def test_e2m1_table_matches_ocp(orc):
    g = _gold("ocp_formats.json")
    vals = g["e2m1_positive_values_by_code"]
    for c in range(8):
        assert orc.e2m1_decode(c) == vals[c]
        assert orc.e2m1_decode(c | 8) == -vals[c]
    assert max(vals) == 1.5 * 2 ** g["e2m1_emax"]


def test_e2m1_encode_brute_force(orc):
    vals = _gold("ocp_formats.json")["e2m1_positive_values_by_code"]
    table = [(v, c) for c, v in enumerate(vals)]
    pts = set()
    for a, b in zip(vals[:-1], vals[1:]):
        for t in np.linspace(a, b, 9):
            pts.add(float(t))
    pts.update([0.0, 6.5, 7.0, 100.0, 0.1, 5.999])
    for x in sorted(pts):
        want = _nearest_even(Fraction(x), table)
        assert orc.e2m1_encode(x) == want, x
        assert orc.e2m1_encode(-x) == (want | 8 if x != 0 else 8), x


def test_e8m0_decode_matches_torch(orc):
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e8m0fnu).float().numpy()
    for c in range(256):
        o = orc.e8m0_decode(c)
        if c == 255:
            assert math.isnan(o) and math.isnan(ref[c])
        else:
            assert o == 2.0 ** (c - 127)
            if ref[c] != 0:        # torch flushes 2^-127 to 0 in float32 view
                assert o == ref[c]


def test_mx_shared_exponent_brute_force(orc):
    rng = np.random.default_rng(7)
    xs = np.concatenate([np.abs(rng.standard_normal(3000)) * 10.0 ** rng.integers(-30, 30, 3000),
                         np.float32([1e-42, 1e-45, 6.0, 4.0, 8.0, 7.999, 3.4e38])]).astype(np.float32)
    for a in xs:
        a = float(a)
        if a == 0 or not math.isfinite(a):
            continue
        m, e = math.frexp(a)          # a = m 2^e, m in [0.5, 1)
        flog2 = e - 1
        want = max(-127, min(127, flog2 - 2))
        got = orc.mx_shared_exponent(a)
        assert got == want, a
        if -127 < want < 127:
            assert 4.0 <= a * 2.0 ** -got < 8.0
    assert orc.mx_shared_exponent(0.0) == -127


def test_bf16_fp16_rounding_matches_torch(orc):
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(5000) * 10.0 ** rng.integers(-6, 6, 5000),
                        [1 + 2 ** -8, 1 + 3 * 2 ** -8, 65504.0, 65520.0, 1e-6, 6e-8]]).astype(np.float32)
    ours_bf = orc.bf16_round_bits(x)
    ref_bf = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours_bf, ref_bf)
    ours_h = orc.fp16_round_bits(x)
    ref_h = torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours_h, ref_h)


def test_pack_fp4_low_nibble_is_even_element(orc):
    codes = np.arange(16, dtype=np.uint8)
    p = orc.pack_fp4(codes)
    assert p[0] == 0x10 and p[7] == 0xFE
    assert np.array_equal(orc.unpack_fp4(p), codes)


def test_e2m1_code_scaled_brute_force(orc):
    """An MX block element's code, E2M1(x 2^-e) [OCP MX v1.0], for every shared
    exponent e: the E2M1 values and the points between them, scaled by 2^e
    (each exactly representable in binary32, subnormals included), against a
    nearest-even search in exact rationals; the array form agrees."""
    vals = _gold("ocp_formats.json")["e2m1_positive_values_by_code"]
    table = [(v, c) for c, v in enumerate(vals)]
    pts = set()
    for a, b in zip(vals[:-1], vals[1:]):
        for t in np.linspace(a, b, 5):
            pts.add(float(t))
    pts.update([6.5, 7.0, 7.75])
    pts = sorted(pts)
    fmax = float(np.finfo(np.float32).max)
    for e in range(-127, 128):
        pe = [x for x in pts if math.ldexp(x, e) <= fmax]   # e = 126, 127: binary32's top binades
        xs = np.array([math.ldexp(x, e) for x in pe], dtype=np.float32)
        assert all(math.ldexp(float(v), -e) == x for v, x in zip(xs, pe)), e   # exact in binary32
        got = orc.e2m1_code_scaled_array(xs, e)
        neg = orc.e2m1_code_scaled_array(-xs, e)
        for x, g, gn, v in zip(pe, got, neg, xs):
            want = _nearest_even(Fraction(x), table)
            assert g == want, (e, x)
            assert gn == (want | 8 if x != 0 else 8), (e, x)
            assert orc.e2m1_code_scaled(float(v), e) == g


def test_mxfp4_quantizer_codes_are_scaled_element_codes(orc):
    """orc_quant_mxfp4's element codes are E2M1(x 2^-e) with e its own E8M0
    code - 127, for random blocks spanning many binades."""
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((3, 64)) * 2.0 ** rng.integers(-40, 40, (3, 64))).astype(np.float32)
    codes, e8 = orc.quant_mxfp4(x.reshape(1, 1, 3, 64))
    codes, e8 = codes.reshape(3, 64), e8.reshape(3, 2)
    for r in range(3):
        for b in range(2):
            blk = x[r, 32 * b:32 * b + 32]
            assert np.array_equal(codes[r, 32 * b:32 * b + 32],
                                  orc.e2m1_code_scaled_array(blk, int(e8[r, b]) - 127))
