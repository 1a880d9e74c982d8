"""CPU check of the arithmetic identity the quantiser kernels use for x / s:
RN32(x * RN64(1/s)) equals the IEEE fp32 quotient RN32(x / s) for finite
fp32 x and positive normal fp32 s (a quotient of two fp32 values never lies
within 2^-49, relative, of an fp32 rounding midpoint, while the two fp64
roundings move it by less than 2^-51).  numpy's fp32 division is the IEEE
one and its fp64 -> fp32 cast rounds to nearest even, like the device's
conversion.  Cases: random significands over many binades, quotients
steered next to fp32 midpoints (x = RN32(s * m) for midpoints m), and the
quantiser's own scales and block values."""
import numpy as np

import oracle
from moe_grouped_gemm_scaled_amd import synth


def _via_reciprocal(x, s):
    y = 1.0 / s.astype(np.float64)
    return (x.astype(np.float64) * y).astype(np.float32)


def _check(x, s):
    want = (x / s).astype(np.float32)
    got = _via_reciprocal(x, s)
    bad = want.view(np.uint32) != got.view(np.uint32)
    assert not bad.any(), (x[bad][:4], s[bad][:4], want[bad][:4], got[bad][:4])


def test_random_significands_over_many_binades():
    n = 4_000_000
    bx = synth.randint(91, 0, n, 0, (1 << 23) - 1).astype(np.uint32)
    bs = synth.randint(91, 1, n, 0, (1 << 23) - 1).astype(np.uint32)
    ex = synth.randint(91, 2, n, 100, 154).astype(np.uint32)     # 2^-27 .. 2^27
    es = synth.randint(91, 3, n, 100, 140).astype(np.uint32)
    sign = (synth.randint(91, 4, n, 0, 1).astype(np.uint32) << 31)
    x = (sign | (ex << 23) | bx).view(np.float32)
    s = ((es << 23) | bs).view(np.float32)
    _check(x, s)


def test_quotients_next_to_midpoints():
    """x = RN32(s * m) for fp32 midpoints m (a 25-bit significand), so that
    x / s lands as close to a rounding boundary as fp32 operands allow."""
    n = 2_000_000
    bs = synth.randint(92, 0, n, 0, (1 << 23) - 1).astype(np.uint32)
    s = ((np.uint32(120) << 23) | bs).view(np.float32)
    mid = (synth.randint(92, 1, n, 1 << 23, (1 << 24) - 1).astype(np.float64) * 2 + 1) * 2.0 ** -24   # in [1, 2)
    x = (s.astype(np.float64) * mid).astype(np.float32)
    for dx in (-1, 0, 1):                                           # and its fp32 neighbours
        xx = (x.view(np.uint32).astype(np.int64) + dx).astype(np.uint32).view(np.float32)
        _check(xx, s)
    # tiny and subnormal fp32 numerators as well
    _check((x * np.float32(2.0 ** -130)).astype(np.float32), s)


def test_quantiser_scales_and_blocks():
    x = synth.normal_f32(93, 0, (512, 1024)) * np.ldexp(np.float32(1.0), synth.randint(93, 1, 512 * 1024, -30, 30).reshape(512, 1024)).astype(np.float32)
    _, sf = oracle.quantize_1x128(x)
    s = np.repeat(sf[:, :512].T, 128, axis=1)
    _check(x, s.astype(np.float32))
