"""Pins for the oracle's scalar codecs (CPU only).

Each codec is checked against something other than itself: the format's own
definition (exponent/mantissa arithmetic written out here), torch's float8 and
bfloat16 conversions, an independent threshold formulation, and a
high-precision decimal evaluation of silu.
"""
from decimal import Decimal, getcontext

import numpy as np
import pytest
import torch

import oracle as O


# ---- e2m1 -------------------------------------------------------------------

def e2m1_from_definition(code):
    """e2m1: 1 sign, 2 exponent bits (bias 1), 1 mantissa bit; exponent field
    0 is subnormal (0.m * 2^0)."""
    s = -1.0 if code & 8 else 1.0
    e = (code >> 1) & 3
    m = code & 1
    if e == 0:
        return s * (m * 0.5)
    return s * (1.0 + m * 0.5) * 2.0 ** (e - 1)


def test_e2m1_value_set():
    # the value set of the format: {0, 0.5, 1, 1.5, 2, 3, 4, 6} and negatives
    vals = sorted({abs(O.e2m1_value(c)) for c in range(16)})
    assert vals == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for c in range(16):
        assert O.e2m1_value(c) == e2m1_from_definition(c)


def test_e2m1_roundtrip():
    for c in range(16):
        v = O.e2m1_value(c)
        if c == 8:
            v = -0.0
        assert O.e2m1_encode(v) == c


@pytest.mark.parametrize(
    "v,code",
    [(0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6),
     (-0.25, 8), (-0.75, 10), (-5.0, 14), (6.0, 7), (6.5, 7), (1e30, 7), (float("inf"), 7),
     (-float("inf"), 15), (-0.0, 8), (0.0, 0), (-0.08, 8), (0.2499999, 0), (0.2500001, 1)],
)
def test_e2m1_ties_and_saturation(v, code):
    assert O.e2m1_encode(v) == code


def e2m1_threshold(v):
    """Independent formulation: count the decision thresholds passed; at a
    threshold that sits on a tie the comparison is strict when the lower code
    is the even one."""
    a = abs(v)
    # (threshold, lower index is even -> strict)
    th = [(0.25, True), (0.75, False), (1.25, True), (1.75, False), (2.5, True),
          (3.5, False), (5.0, True)]
    idx = 0
    for t, strict in th:
        if (a > t) if strict else (a >= t):
            idx += 1
    return idx | (8 if np.signbit(v) else 0)


def test_e2m1_matches_threshold_formulation():
    rng = np.random.default_rng(0)
    pts = list(rng.uniform(-8, 8, 20000).astype(np.float32))
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0]
    for mpt in mids:
        f = np.float32(mpt)
        for s in (1, -1):
            pts += [s * f, s * np.nextafter(f, np.float32(0)), s * np.nextafter(f, np.float32(9))]
    for v in pts:
        assert O.e2m1_encode(v) == e2m1_threshold(float(v)), v


# ---- ue4m3 ------------------------------------------------------------------

def test_ue4m3_decode_matches_torch_e4m3fn():
    lut = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64)
    for c in range(0x7F):
        assert O.ue4m3_value(c) == lut[c].item()
    assert O.ue4m3_value(0x7E) == 448.0          # largest ue4m3 value
    assert O.ue4m3_value(0x01) == 2.0 ** -9      # smallest subnormal
    assert np.isnan(O.ue4m3_value(0x7F))


def test_ue4m3_encode_roundtrip_and_saturation():
    for c in range(0x7F):
        assert O.ue4m3_encode(O.ue4m3_value(c)) == c
    for v in (448.0, 448.5, 463.9, 464.0, 480.0, 1e9, float("inf")):
        assert O.ue4m3_encode(v) == 0x7E       # saturating: never 0x7F
    for v in (0.0, -0.0, -1.0, -1e9, float("nan")):
        assert O.ue4m3_encode(v) == 0


def test_ue4m3_encode_matches_torch_rne():
    # torch's fp32 -> float8_e4m3fn is round-to-nearest-even and overflows to
    # NaN past 464; below that it is the reference rounding.
    rng = np.random.default_rng(1)
    v = np.concatenate([
        rng.uniform(0, 464, 20000),
        np.exp2(rng.uniform(-12, 8.85, 20000)),
    ]).astype(np.float32)
    # every exact value, every midpoint and their neighbours
    vals = np.array([O.ue4m3_value(c) for c in range(0x7F)])
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    extra = np.concatenate([mids, np.nextafter(mids, 0), np.nextafter(mids, 1000),
                            vals.astype(np.float32)])
    v = np.concatenate([v, extra])
    v = v[(v >= 0) & (v < 464)]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([O.ue4m3_encode(x) for x in v], dtype=np.uint8)
    bad = np.nonzero(ref != got)[0]
    assert len(bad) == 0, (v[bad[:5]], ref[bad[:5]], got[bad[:5]])


# ---- bf16 -------------------------------------------------------------------

def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(2)
    u = rng.integers(0, 2 ** 32, 50000, dtype=np.uint64).astype(np.uint32)
    f = u.view(np.float32)
    f = f[np.isfinite(f)]
    # ties: low half exactly 0x8000
    ties = ((rng.integers(0, 2 ** 16, 2000, dtype=np.uint32) << 16) | 0x8000).view(np.float32)
    edge = np.array([3.3895314e38, 3.3961775e38, 3.4e38, np.finfo(np.float32).max, 1e-40, -1e-45],
                    dtype=np.float32)
    f = np.concatenate([f, ties[np.isfinite(ties)], edge])
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = O.f32_to_bf16(f)
    bad = np.nonzero(ref != got)[0]
    assert len(bad) == 0, (f[bad[:5]], ref[bad[:5]], got[bad[:5]])


# ---- silu -------------------------------------------------------------------

def _round_to_f32(d: Decimal) -> np.float32:
    """Correctly rounded Decimal -> float32 (ties to even), by comparing with
    the exact midpoints to the neighbours of a first guess."""
    f = np.float32(float(d))
    best = f
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    bd = None
    for c in cands:
        if not np.isfinite(c):
            continue
        e = abs(Decimal(float(c)) - d)
        if bd is None or e < bd or (e == bd and (int(np.array(c).view(np.uint32)) & 1) == 0):
            bd, best = e, c
    return np.float32(best)


def test_silu_correctly_rounded_all_bf16():
    """S(g) for every finite bf16 g equals g/(1+e^-g) evaluated to 40 digits
    and rounded once to fp32."""
    getcontext().prec = 40
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    g = O.bf16_to_f32(codes)
    fin = np.isfinite(g)
    L = O.lib()
    bad = []
    for gi in g[fin]:
        got = np.float32(L.nvo_silu(float(gi)))
        dg = Decimal(float(gi))
        if dg == 0:
            ref = np.float32(gi)
        elif dg < -200:
            ref = np.float32(-0.0)   # |value| < 1e-80: rounds to -0
        else:
            ref = _round_to_f32(dg / (1 + (-dg).exp()))
        if got.view(np.uint32) != ref.view(np.uint32):
            bad.append((gi, got, ref))
    assert not bad, bad[:5]


def test_silu_special_values():
    assert O.silu(0.0) == 0.0
    assert O.silu(100.0) == np.float32(100.0)
    assert np.isinf(O.silu(float("inf")))
    assert np.isnan(O.silu(float("-inf")))
