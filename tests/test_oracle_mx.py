"""Pins for the oracle's MX variant (CPU only).

The MX setting of fp4_quantize's flags (32-element blocks, ue8m0 scales) is
read as the OCP Microscaling Formats v1.0 conversion for MXFP4: X =
2^(floor(log2 amax) - 2), elements e2m1(v / X) nearest-even saturating at 6.
The checks recompute that definition independently with exact rationals
(the exponent found by comparison with powers of two, the nearest e2m1
value by exhaustive search), and the GEMM with exact rational arithmetic.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
from test_oracle_gemm import e2m1_frac, swz

E2M1_POS = [e2m1_frac(c) for c in range(8)]          # 0, 1/2, 1, 3/2, 2, 3, 4, 6
FLT_MAX = Fraction(np.finfo(np.float32).max.item())


def floor_log2(a):
    """Largest e with 2^e <= a (a > 0 rational)."""
    e = 0
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def e2m1_nearest(v):
    """Code of the e2m1 value nearest to rational v (ties to the even index),
    saturating at 6, sign kept."""
    sign = 8 if v < 0 else 0
    a = abs(v)
    best = min(range(8), key=lambda i: (abs(a - E2M1_POS[i]), i & 1))
    return sign | best


def ref_block(vals):
    """(scale code, 32 codes) of one block by the definition."""
    vs = []
    for v in vals:
        v = float(v)
        if np.isnan(v):
            v = 0.0
        elif np.isinf(v):
            v = float(np.copysign(np.finfo(np.float32).max, v))
        vs.append(Fraction(v))
    amax = max(abs(v) for v in vs)
    if amax == 0:
        return 0, [0 | (8 if np.signbit(float(x)) and not np.isnan(float(x)) else 0) for x in vals]
    shared = max(-127, min(127, floor_log2(amax) - 2))
    X = Fraction(2) ** shared
    codes = []
    for v, raw in zip(vs, vals):
        c = e2m1_nearest(v / X)
        if v == 0 and np.signbit(float(raw)) and not np.isnan(float(raw)):
            c = 8            # -0 keeps its sign bit
        codes.append(c)
    return shared + 127, codes


def unpack(q, k):
    return np.stack([q & 15, q >> 4], axis=-1).reshape(q.shape[0], k)


def check_against_definition(x, k):
    q, sf = O.quantize_mx(x)
    codes = unpack(q, k)
    for r in range(x.shape[0]):
        for c in range(k // 32):
            sc, want = ref_block(x[r, c * 32:(c + 1) * 32])
            assert sf[swz(r, c, k // 2)] == sc, (r, c)       # k/32 scale columns
            assert codes[r, c * 32:(c + 1) * 32].tolist() == want, (r, c)
    return q, sf


def test_ue8m0_values_and_sizes():
    assert O.ue8m0_value(127) == 1.0
    assert O.ue8m0_value(0) == 2.0 ** -127
    assert O.ue8m0_value(254) == 2.0 ** 127
    assert np.isnan(O.ue8m0_value(255))
    assert O.sf_size_mx(1, 32) == 128 * 4
    assert O.sf_size_mx(129, 160) == 256 * 8        # pad_up(129,128) x pad_up(5,4)


def test_random_blocks_fp32():
    rng = np.random.default_rng(41)
    x = (rng.standard_normal((6, 96)) * np.exp(rng.normal(0, 3, size=(6, 1)))).astype(np.float32)
    x[1, 5] = 40.0            # an outlier in one block
    check_against_definition(x, 96)


def test_special_values_and_ranges():
    x = np.zeros((5, 64), dtype=np.float32)
    x[0, :32] = 0.0                                   # all-zero block -> code 0
    x[0, 7] = -0.0
    x[0, 32:] = np.float32(2.0 ** -140)               # subnormal fp32 amax, shared exponent clamped
    x[0, 40] = np.float32(3 * 2.0 ** -141)
    x[1, :32] = np.linspace(-7.9, 7.9, 32, dtype=np.float32)   # amax in [4, 8): X = 1, saturation at 6
    x[1, 32:] = np.float32(1.0)                       # amax a power of two: max -> e2m1 4
    x[2, :] = np.float32(3.0e38)                      # near FLT_MAX
    x[2, 3] = np.inf
    x[2, 4] = -np.inf
    x[2, 5] = np.nan
    x[3, :32] = np.arange(32, dtype=np.float32) * np.float32(0.25)   # ties at e2m1 midpoints
    x[4, 32:] = -np.float32(2.0 ** 100) * np.arange(1, 33, dtype=np.float32)
    q, sf = check_against_definition(x, 64)
    assert sf[swz(0, 0, 32)] == 0
    assert sf[swz(1, 1, 32)] == 127 - 2               # amax 1 = 2^0 -> X = 2^-2
    assert unpack(q, 64)[1, 32] == 6                  # 1 / 2^-2 = 4 -> e2m1 code 6 (4.0)


def test_random_blocks_bf16_with_outlier_channels():
    rng = np.random.default_rng(42)
    x = rng.standard_normal((8, 128)).astype(np.float32)
    x[:, [3, 77]] *= 30.0
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)     # truncation: any bf16 values will do
    xf = (bits.astype(np.uint32) << 16).view(np.float32)
    q1, s1 = O.quantize_mx(bits)
    q2, s2 = check_against_definition(xf, 128)
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2)


def test_largest_element_decodes_to_4_or_6():
    """X = 2^(floor(log2 amax) - 2) puts amax / X in [4, 8): the largest
    magnitude of every nonzero block encodes as 4 or 6."""
    rng = np.random.default_rng(43)
    x = (rng.standard_normal((16, 256)) * 10.0 ** rng.uniform(-20, 20, size=(16, 1))).astype(np.float32)
    q, sf = O.quantize_mx(x)
    codes = unpack(q, 256)
    for r in range(16):
        for c in range(8):
            blk = np.abs(x[r, c * 32:(c + 1) * 32])
            j = int(np.argmax(blk))
            assert codes[r, c * 32 + j] & 7 in (6, 7)


def mx_frac(code):
    return Fraction(2) ** (int(code) - 127)


def test_tiny_gemm_exact_rational():
    rng = np.random.default_rng(44)
    m, n, k = 3, 5, 96
    a = (rng.standard_normal((m, k)) * 3).astype(np.float32)
    b = (rng.standard_normal((n, k)) * 0.05).astype(np.float32)
    qa, sa = O.quantize_mx(a)
    qb, sb = O.quantize_mx(b)
    alpha = np.float32(0.75)
    bias = np.array([0x3F80, 0xBF00, 0, 0x4000, 0x3E80], dtype=np.uint16)   # 1, -0.5, 0, 2, 0.25
    out = O.gemm_mx_rows(qa, qb, sa, sb, alpha, m, n, k, bias=bias)
    ca, cb = unpack(qa, k), unpack(qb, k)
    bias_v = [Fraction(1), Fraction(-1, 2), Fraction(0), Fraction(2), Fraction(1, 4)]
    for i in range(m):
        for j in range(n):
            acc = sum(e2m1_frac(ca[i, kk]) * mx_frac(sa[swz(i, kk // 32, k // 2)]) *
                      e2m1_frac(cb[j, kk]) * mx_frac(sb[swz(j, kk // 32, k // 2)]) for kk in range(k))
            ref = Fraction(float(alpha)) * acc + bias_v[j]
            assert abs(Fraction(out[i, j]) - ref) <= Fraction(k) * Fraction(2) ** -52 * (abs(ref) + 1)


def test_quantize_rejects_bad_width():
    with pytest.raises(ValueError):
        O.quantize_mx(np.zeros((2, 48), dtype=np.float32))
