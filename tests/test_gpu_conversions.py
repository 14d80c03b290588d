"""The two hardware conversions the kernels code with, held against the
oracle's encoders (OCP 8-bit floating point E4M3, OCP MX v1.0 E2M1), code for
code, through the library's test hooks (sage_debug_cvt_e4m3 /
sage_debug_cvt_e2m1, which call the kernels' own device functions):

* fp32 -> e4m3 (P8 = e4m3(448 p) in attention and decode, the V codes, the
  decode's query codes): every fp32 input of magnitude below 464 -- every
  value the kernels convert, and the rounding slack above 448 -- both signs.
* fp32 * 2^-e -> E2M1 (the MXFP4 quantizer's element codes, the fused-Q
  prologue's): every fp32 input of magnitude below 16 at e = 0 (block values
  lie below 8, the rest is saturation), and at every shared exponent e in
  [-127, 127] the E2M1 values, the points half-way between them and their
  binary32 neighbours, scaled by 2^e, plus seeded random inputs below 8 2^e.

The oracle side runs on the host's cores in threads (its ctypes calls release
the interpreter lock).
"""
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

from quantized_attention_block_amd import sage
from tests._util import require_gpu, say

pytestmark = pytest.mark.gpu

CHUNK = 1 << 27            # fp32 inputs per GPU call (512 MB)
THREADS = max(1, min(16, os.cpu_count() or 1))


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _oracle_codes(orc, fn, x, *args):
    """Codes of host fp32 array x by the oracle's array encoder fn(ptr, n, *args, out)."""
    out = np.empty(x.shape, dtype=np.uint8)
    bounds = np.linspace(0, x.size, THREADS + 1).astype(np.int64)

    def part(i):
        a, b = int(bounds[i]), int(bounds[i + 1])
        if b > a:
            fn(x[a:b].ctypes.data, b - a, *args, out[a:b].ctypes.data)

    with ThreadPoolExecutor(THREADS) as ex:
        list(ex.map(part, range(THREADS)))
    return out


def _sweep(dev, orc, hi_bits, gpu_fn, orc_fn, *args):
    """Every fp32 bit pattern in [0, hi_bits) and its negation, GPU against
    the oracle; returns the number of inputs compared."""
    total = 0
    for lo in range(0, hi_bits, CHUNK):
        n = min(CHUNK, hi_bits - lo)
        for sign_bit in (0, 0x80000000):
            host = (np.arange(lo, lo + n, dtype=np.uint32) | np.uint32(sign_bit)).view(np.float32)
            got = gpu_fn(torch.from_numpy(host).to(dev), *args).cpu().numpy()
            want = _oracle_codes(orc, orc_fn, host, *args)
            bad = np.flatnonzero(got != want)
            if bad.size:
                i = bad[:8]
                pytest.fail(f"{bad.size} codes differ, e.g. inputs "
                            f"{[hex(int(v)) for v in host.view(np.uint32)[i]]}: GPU "
                            f"{got[i].tolist()} oracle {want[i].tolist()}")
            total += n
    return total


def test_e4m3_conversion_every_fp32_below_464(dev, orc):
    hi = int(np.float32(464.0).view(np.uint32))
    say("e4m3 conversion: every fp32 with |x| < 464")
    n = _sweep(dev, orc, hi, sage.sage_debug_cvt_e4m3, orc.lib().orc_e4m3_encode_array)
    assert n == 2 * hi
    # NaN inputs give a NaN code (either sign)
    nan = np.array([0x7FC00000, 0x7F800001, 0xFFC00000], dtype=np.uint32).view(np.float32)
    got = sage.sage_debug_cvt_e4m3(torch.from_numpy(nan).to(dev)).cpu().numpy()
    assert all((int(c) & 0x7F) == 0x7F for c in got)


def test_e2m1_conversion_every_fp32_below_16_at_exponent_0(dev, orc):
    hi = int(np.float32(16.0).view(np.uint32))
    say("E2M1 conversion at exponent 0: every fp32 with |x| < 16")
    n = _sweep(dev, orc, hi, sage.sage_debug_cvt_e2m1, orc.lib().orc_e2m1_code_scaled_array, 0)
    assert n == 2 * hi


def test_e2m1_conversion_boundaries_at_every_exponent(dev, orc):
    vals = [orc.e2m1_decode(c) for c in range(8)]
    base = set(vals)
    for a, b in zip(vals[:-1], vals[1:]):
        base.add((a + b) / 2)
    base.update([6.5, 7.0, 7.75])
    rng = np.random.default_rng(20)
    fmax = float(np.finfo(np.float32).max)
    say("E2M1 conversion: boundaries at every exponent in [-127, 127]")
    for e in range(-127, 128):
        pts = []
        for x in sorted(base):
            v = math.ldexp(x, e)
            if v > fmax:
                continue
            f = np.float32(v)
            pts += [f, np.nextafter(f, np.float32(0)), np.nextafter(f, np.float32(np.inf))]
        top = min(8.0 * 2.0 ** e, fmax)
        rand = (rng.random(4096) * top).astype(np.float32)
        x = np.concatenate([np.array(pts, dtype=np.float32), rand])
        x = x[np.isfinite(x)]
        x = np.concatenate([x, -x])
        got = sage.sage_debug_cvt_e2m1(torch.from_numpy(x).to(dev), e).cpu().numpy()
        want = orc.e2m1_code_scaled_array(x, e)
        bad = np.flatnonzero(got != want)
        assert bad.size == 0, (e, x[bad[:8]].tolist(), got[bad[:8]].tolist(), want[bad[:8]].tolist())
