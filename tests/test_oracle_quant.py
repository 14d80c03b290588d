"""Pins of the oracle's Hadamard matrix and quantizers: library routines
(scipy's Sylvester Hadamard, numpy's float64 mean), invariants that any correct
quantizer satisfies, and brute force on small blocks."""
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg


def test_hadamard_is_sylvester(orc):
    for R in (1, 2, 4, 32, 128):
        H = orc.hadamard(R)
        assert np.array_equal(H, scipy.linalg.hadamard(R).astype(np.float32))
        assert np.array_equal(H @ H.T, R * np.eye(R, dtype=np.float32))
        assert np.array_equal(H, H.T)


def _rand(shape, seed, scale=1.0):
    return (np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float32)


def test_rotation_matches_matrix_product_and_is_orthogonal(orc):
    x = _rand((1, 2, 37, 256), 1, 3.0)
    y = orc.rotate(x, 128)
    H = scipy.linalg.hadamard(128).astype(np.float64) / np.sqrt(128.0)
    want = np.concatenate([x[..., :128].astype(np.float64) @ H,
                           x[..., 128:].astype(np.float64) @ H], axis=-1)
    assert np.allclose(y, want, rtol=3e-7, atol=1e-6)
    # norms and dot products are preserved; rotating twice returns the input
    assert np.allclose((y.astype(np.float64) ** 2).sum(-1), (x.astype(np.float64) ** 2).sum(-1),
                       rtol=1e-6)
    z = orc.rotate(y, 128)
    assert np.allclose(z, x, rtol=1e-5, atol=1e-5)


def test_k_mean_and_smoothing(orc):
    k = _rand((2, 3, 77, 64), 2, 2.0) + 5.0
    mu = orc.k_mean(k)
    want = k.astype(np.float64).mean(axis=2).astype(np.float32)
    assert np.array_equal(mu, want)
    ks = orc.smooth_k(k, mu)
    assert np.array_equal(ks, (k - mu[:, :, None, :]).astype(np.float32))
    assert np.abs(ks.astype(np.float64).mean(axis=2)).max() < 1e-5


@pytest.mark.parametrize("L,block", [(256, 128), (130, 128), (100, 64), (1, 64)])
def test_int8_quant_invariants(orc, L, block):
    x = _rand((1, 2, L, 64), 3, 4.0)
    x[0, 1, :min(L, block)] = 0.0                  # an all-zero block
    codes, scales = orc.quant_int8(x, block)
    nb = (L + block - 1) // block
    assert scales.shape == (1, 2, nb)
    for h in range(2):
        for bi in range(nb):
            xb = x[0, h, bi * block:(bi + 1) * block]
            cb = codes[0, h, bi * block:(bi + 1) * block].astype(np.int64)
            s = scales[0, h, bi]
            amax = np.abs(xb).max()
            if amax == 0:
                assert s == 0 and not cb.any()
                continue
            # the scale comes from this block's own rows only (ragged tail too)
            assert s == np.float32(amax / np.float32(127))
            assert np.abs(cb).max() == 127
            assert np.abs(cb).max() <= 127
            err = np.abs(xb.astype(np.float64) - cb * np.float64(s))
            assert err.max() <= 0.5 * s * (1 + 2 ** -20) + 1e-12


def test_int8_quant_brute_force_small(orc):
    x = np.float32([[[[0.3, -1.7, 2.54, 0.0], [1.27, -2.54, 0.01, 0.635]]]])
    codes, scales = orc.quant_int8(x, 2)
    s = Fraction(float(scales[0, 0, 0]))
    inv = Fraction(float(np.float32(127) / np.float32(2.54)))
    for idx, v in np.ndenumerate(x[0, 0]):
        # nearest integer to fp32(x * inv), ties to even, within [-127, 127]
        prod = Fraction(float(np.float32(v) * np.float32(float(inv))))
        n = round(prod)              # Python round: ties to even
        assert codes[0, 0][idx] == max(-127, min(127, n))
    assert float(s) == float(np.float32(2.54) / np.float32(127))


def test_v_fp8_quant(orc):
    v = _rand((1, 2, 300, 64), 4)
    v[0, 1, :, 5] = 0.0
    codes, scales = orc.quant_v_fp8(v)
    dec = orc.e4m3_decode_array(codes)
    for h in range(2):
        for d in range(64):
            s = scales[0, h, d]
            col = v[0, h, :, d].astype(np.float64)
            if s == 0:
                assert not codes[0, h, :, d].any()
                continue
            assert np.abs(dec[0, h, :, d]).max() == 448.0
            y = col / s
            norm = np.abs(y) >= 2.0 ** -6
            rel = np.abs(dec[0, h, norm, d] - y[norm]) / np.abs(y[norm])
            assert rel.max() <= 2.0 ** -4 * (1 + 1e-6)
            sub = ~norm
            assert (np.abs(dec[0, h, sub, d] - y[sub]) <= 2.0 ** -10 * (1 + 1e-6)).all()


def test_mxfp4_quant_brute_force(orc):
    x = _rand((1, 1, 5, 64), 5, 3.0)
    x[0, 0, 0, :32] = 0.0
    x[0, 0, 1, 32:] *= 1e-38        # subnormal-range block
    codes, e8 = orc.quant_mxfp4(x)
    assert e8[0, 0, 0, 0] == 0 and not codes[0, 0, 0, :32].any()
    table = [(orc.e2m1_decode(c), c) for c in range(8)]
    for row in range(5):
        for bl in range(2):
            xb = x[0, 0, row, bl * 32:(bl + 1) * 32]
            e = int(e8[0, 0, row, bl]) - 127
            amax = float(np.abs(xb).max())
            if amax == 0:
                continue
            if -127 < e < 127:
                assert 4.0 <= amax * 2.0 ** -e < 8.0
            for d in range(32):
                y = Fraction(float(xb[d])) * Fraction(2) ** (-e)
                best = min(table, key=lambda vc: (abs(Fraction(vc[0]) - abs(y)), vc[1] % 2))
                want = best[1] | (8 if xb[d] < 0 or (xb[d] == 0 and np.signbit(xb[d])) else 0)
                assert codes[0, 0, row, bl * 32 + d] == want, (row, bl, d)
