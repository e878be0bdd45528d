"""Pins for the oracle's block-scaled GEMM (CPU only).

The eager meaning of an NVFP4 matmul on the nvFuser page is "dequantize, then
a plain linear".  The checks:
  * exact rational arithmetic on tiny shapes (Fractions, with the codes decoded
    from the format definitions written out here);
  * torch float64 matmul of matrices dequantized independently (torch's
    float8_e4m3fn decode for scales, format-definition decode for e2m1);
  * the SVDQuant special cases on the flashinfer mm_nvfp4_svdquant page:
    d = l1 = 0 gives the plain GEMM; an all-zero residual gives
    alpha*(d@l1^T) + bias.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
from nvfp4_block_scaled_04_amd import synth


def e2m1_frac(code):
    code = int(code)
    s = -1 if code & 8 else 1
    e = (code >> 1) & 3
    m = code & 1
    if e == 0:
        return s * Fraction(m, 2)
    return s * (1 + Fraction(m, 2)) * Fraction(2) ** (e - 1)


def e4m3_frac(code):
    code = int(code)
    e = (code >> 3) & 15
    m = code & 7
    if e == 0:
        return Fraction(m, 2 ** 9)
    return (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)


def swz(r, c, k):
    cp = -(-(k // 16) // 4) * 4
    return ((r // 128) * (cp // 4) + c // 4) * 512 + (r % 32) * 16 + ((r % 128) // 32) * 4 + c % 4


def dequant_torch(q, sf, rows, k):
    """Independent dequantization: nibble table from the e2m1 definition,
    scales through torch's float8_e4m3fn decode."""
    lut = torch.tensor([float(e2m1_frac(c)) for c in range(16)], dtype=torch.float64)
    qt = torch.from_numpy(q.astype(np.int64))
    codes = torch.stack([qt & 15, qt >> 4], dim=-1).reshape(rows, k)
    vals = lut[codes]
    sdec = torch.from_numpy(sf.copy()).view(torch.float8_e4m3fn).to(torch.float64)
    idx = torch.tensor([[swz(r, c, k) for c in range(k // 16)] for r in range(rows)])
    scales = sdec[idx].repeat_interleave(16, dim=1)
    return vals * scales


def rand_quant(rng, rows, k, scale=1.0):
    x = (rng.standard_normal((rows, k)) * scale).astype(np.float32)
    q, sf, gs = O.quantize(x)
    return q, sf, gs[0]


def test_tiny_gemm_exact_rational():
    rng = np.random.default_rng(11)
    m, n, k = 3, 4, 48
    a, asf, ga = rand_quant(rng, m, k, 3.0)
    b, bsf, gb = rand_quant(rng, n, k, 0.5)
    alpha = np.float32(1.0) / (ga * gb)
    out = O.gemm_rows(a, b, asf, bsf, alpha, m, n, k)
    for i in range(m):
        for j in range(n):
            acc = Fraction(0)
            for kk in range(k):
                ca = (a[i, kk // 2] >> (4 * (kk & 1))) & 15
                cb = (b[j, kk // 2] >> (4 * (kk & 1))) & 15
                acc += (e2m1_frac(ca) * e4m3_frac(asf[swz(i, kk // 16, k)])
                        * e2m1_frac(cb) * e4m3_frac(bsf[swz(j, kk // 16, k)]))
            ref = Fraction(float(alpha)) * acc
            # every product is exact in fp64; only the k-term summation rounds
            assert abs(Fraction(out[i, j]) - ref) <= Fraction(k) * Fraction(2) ** -52 * (abs(ref) + 1)


@pytest.mark.parametrize("m,n,k", [(128, 256, 256), (37, 19, 80), (1, 5, 16)])
def test_gemm_matches_torch_float64(m, n, k):
    rng = np.random.default_rng(m + n + k)
    a, asf, ga = rand_quant(rng, m, k, 2.0)
    b, bsf, gb = rand_quant(rng, n, k, 0.02)
    alpha = np.float32(1.0) / (ga * gb)
    out = O.gemm_rows(a, b, asf, bsf, alpha, m, n, k)
    ref = float(alpha) * (dequant_torch(a, asf, m, k) @ dequant_torch(b, bsf, n, k).T)
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-12 * float(np.abs(ref).max()))


def test_gemm_row_subset_and_bias():
    rng = np.random.default_rng(12)
    m, n, k = 20, 33, 64
    a, asf, ga = rand_quant(rng, m, k)
    b, bsf, gb = rand_quant(rng, n, k)
    bias = torch.randn(n).to(torch.bfloat16)
    bias_bits = synth.bits(bias)
    full = O.gemm_rows(a, b, asf, bsf, 0.5, m, n, k, bias=bias_bits)
    rows = np.array([19, 0, 7])
    sub = O.gemm_rows(a, b, asf, bsf, 0.5, m, n, k, rows=rows, bias=bias_bits)
    assert np.array_equal(sub, full[rows])
    nob = O.gemm_rows(a, b, asf, bsf, 0.5, m, n, k)
    np.testing.assert_allclose(full - nob, np.broadcast_to(bias.double().numpy(), (m, n)), rtol=0, atol=1e-12)


def test_svdquant_zero_lora_reduces_to_plain():
    rng = np.random.default_rng(13)
    m, n, k, r = 16, 24, 64, 32
    a, asf, ga = rand_quant(rng, m, k)
    b, bsf, gb = rand_quant(rng, n, k)
    d = np.zeros((m, r), dtype=np.uint16)
    l1 = np.zeros((n, r), dtype=np.uint16)
    x = O.gemm_rows(a, b, asf, bsf, 0.25, m, n, k, d=d, l1=l1)
    y = O.gemm_rows(a, b, asf, bsf, 0.25, m, n, k)
    assert np.array_equal(x, y)


def test_svdquant_zero_residual_is_lora_plus_bias():
    rng = np.random.default_rng(14)
    m, n, k, r = 16, 24, 64, 32
    a, asf, _ = rand_quant(rng, m, k)
    b = np.zeros((n, k // 2), dtype=np.uint8)
    bsf = np.zeros(O.sf_size(n, k), dtype=np.uint8)
    alpha = np.float32(0.125)
    d = torch.randn(m, r).to(torch.bfloat16)
    l1 = torch.randn(n, r).to(torch.bfloat16)
    bias = torch.randn(n).to(torch.bfloat16)
    out = O.gemm_rows(a, b, asf, bsf, alpha, m, n, k, bias=synth.bits(bias),
                      d=synth.bits(d), l1=synth.bits(l1))
    ref = float(alpha) * (d.double() @ l1.double().T) + bias.double()
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-13, atol=1e-13)


# ---- weight-only form (nvFuser page: f16a_nvfp4weight_scaled_mm) -------------------


def test_w4a16_reduces_to_nvfp4_gemm():
    """An activation whose bf16 values are exactly its own NVFP4 dequantization
    (e2m1 x block scale, at most 6 significant bits) gives the NVFP4 x NVFP4
    product bit for bit: the two oracle routines then sum identical fp64 terms."""
    rng = np.random.default_rng(31)
    m, n, k = 9, 21, 96
    a, asf, ga = rand_quant(rng, m, k, 2.0)
    b, bsf, gb = rand_quant(rng, n, k, 0.02)
    a_dq = dequant_torch(a, asf, m, k)
    a_bf16 = a_dq.to(torch.bfloat16)
    assert torch.equal(a_bf16.double(), a_dq), "dequantized NVFP4 values are exact in bf16"
    alpha = np.float32(1.0) / gb
    bias = torch.randn(n).to(torch.bfloat16)
    w = O.gemm_w4a16_rows(synth.bits(a_bf16), b, bsf, alpha, m, n, k, bias=synth.bits(bias))
    ref = O.gemm_rows(a, b, asf, bsf, alpha, m, n, k, bias=synth.bits(bias))
    assert np.array_equal(w, ref)


def test_w4a16_matches_exact_weight():
    """A weight built from e2m1 values times powers of two, every 16-block
    holding its own +-6 x 2^j, quantizes without loss (gs = 448 / 2^jmax and
    every block scale a power-of-two multiple of 448): the dequantized weight
    is exactly w * gs, so the weight-only product must equal the float64
    product a @ (w * gs)^T (exact: at most 14-bit products, 64 terms) times
    the fp32 alpha = 1/gs, bit for bit."""
    rng = np.random.default_rng(32)
    m, n, k = 7, 12, 64
    vals = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    w = rng.choice(vals, size=(n, k)) * rng.choice([-1.0, 1.0], size=(n, k))
    w[:, ::16] = 6.0 * rng.choice([-1.0, 1.0], size=(n, k // 16))  # each block's maximum
    pw = 2.0 ** rng.integers(-6, 3, size=(n, k // 16))
    w = w * np.repeat(pw, 16, axis=1)
    q, sf, gs = O.quantize(w.astype(np.float32))
    assert gs[0] == np.float32(448.0 / pw.max())
    a = torch.randn(m, k).to(torch.bfloat16)
    alpha = np.float32(1.0) / gs[0]
    out = O.gemm_w4a16_rows(synth.bits(a), q, sf, alpha, m, n, k)
    ref = float(alpha) * (a.double().numpy() @ (w * float(gs[0])).T)
    assert np.array_equal(out, ref), np.abs(out - ref).max()


def test_w4a16_row_subset():
    rng = np.random.default_rng(33)
    m, n, k = 11, 9, 48
    b, bsf, gb = rand_quant(rng, n, k)
    a = synth.bits(torch.randn(m, k).to(torch.bfloat16))
    full = O.gemm_w4a16_rows(a, b, bsf, 0.5, m, n, k)
    rows = np.array([10, 0, 4])
    assert np.array_equal(O.gemm_w4a16_rows(a, b, bsf, 0.5, m, n, k, rows=rows), full[rows])


# ---- SVDQuant LoRA-down (flashinfer mm_nvfp4_svdquant: d = x @ (pqs[:, None] * L2^T)) ----


def test_lora_down_exact_rational():
    """A tiny case against exact rational arithmetic on the bf16 inputs."""
    g = torch.Generator().manual_seed(41)
    m, k, r = 3, 32, 4
    x = torch.randn(m, k, generator=g).to(torch.bfloat16)
    p = torch.exp(0.5 * torch.randn(k, generator=g)).to(torch.bfloat16)
    l2 = (0.02 * torch.randn(r, k, generator=g)).to(torch.bfloat16)
    d = O.lora_down(synth.bits(x), synth.bits(p), synth.bits(l2))
    for i in range(m):
        for j in range(r):
            ref = sum(Fraction(float(x[i, kk])) * Fraction(float(p[kk])) * Fraction(float(l2[j, kk]))
                      for kk in range(k))
            assert abs(Fraction(d[i, j]) - ref) <= Fraction(k) * Fraction(2) ** -52 * (abs(ref) + 1)


def test_lora_down_unit_rows_select_smoothed_columns():
    """With L2's rows unit vectors e_c, d[:, j] is the smoothed column x * pqs
    (exact: a product of two bf16 values fits fp32 and fp64)."""
    g = torch.Generator().manual_seed(42)
    m, k = 5, 48
    x = torch.randn(m, k, generator=g).to(torch.bfloat16)
    p = torch.exp(0.5 * torch.randn(k, generator=g)).to(torch.bfloat16)
    cols = [3, 0, 47, 16]
    l2 = torch.zeros(len(cols), k)
    for j, c in enumerate(cols):
        l2[j, c] = 1.0
    d = O.lora_down(synth.bits(x), synth.bits(p), synth.bits(l2.to(torch.bfloat16)))
    ref = (x.double() * p.double())[:, cols]
    assert np.array_equal(d, ref.numpy())


def _split_inputs(seed, r, k, spread=0.5):
    g = torch.Generator().manual_seed(seed)
    p = torch.exp(spread * torch.randn(k, generator=g)).to(torch.bfloat16)
    l2 = (0.02 * torch.randn(r, k, generator=g)).to(torch.bfloat16)
    return p, l2


def test_lora_weight_split_sums_to_the_product_exactly():
    """hi + lo is pqs[k] * l2[j, k] exactly (fp64 holds the product of two
    bf16 values exactly), for every element; a dropped lo, a wrong sign or a
    transposed pqs index fails here."""
    p, l2 = _split_inputs(43, 6, 96, spread=3.0)
    w = O.lora_weight_split(synth.bits(p), synth.bits(l2))
    assert w.shape == (2, 6, 96) and w.dtype == np.uint16
    hi = O.bf16_to_f32(w[0]).astype(np.float64)
    lo = O.bf16_to_f32(w[1]).astype(np.float64)
    exact = l2.double().numpy() * p.double().numpy()[None, :]
    assert np.array_equal(hi + lo, exact)
    assert np.count_nonzero(lo) > 0.5 * lo.size   # the low halves are really used


def test_lora_weight_split_hi_is_the_nearest_bf16():
    """hi is the bf16 nearest the product (brute force over its two
    neighbours, ties to the even code), and torch's own fp32 -> bf16
    rounding of the product gives the same bits."""
    p, l2 = _split_inputs(44, 4, 64, spread=2.0)
    w = O.lora_weight_split(synth.bits(p), synth.bits(l2))
    exact = l2.double().numpy() * p.double().numpy()[None, :]
    hi = w[0].astype(np.int64)
    for delta in (-1, 1):
        nb = O.bf16_to_f32((hi + delta).astype(np.uint16)).astype(np.float64)
        d_hi = np.abs(exact - O.bf16_to_f32(w[0]).astype(np.float64))
        d_nb = np.abs(exact - nb)
        assert np.all((d_hi < d_nb) | ((d_hi == d_nb) & (hi % 2 == 0)))
    prod32 = (l2.float() * p.float()[None, :]).to(torch.bfloat16)
    assert np.array_equal(w[0], synth.bits(prod32))


def test_lora_weight_split_unit_scale_is_the_weight():
    """pqs = 1: hi is l2 itself and lo is +0."""
    _, l2 = _split_inputs(45, 3, 32)
    ones = torch.ones(32, dtype=torch.bfloat16)
    w = O.lora_weight_split(synth.bits(ones), synth.bits(l2))
    assert np.array_equal(w[0], synth.bits(l2))
    assert np.all(w[1] == 0)


def test_lora_weight_split_projection_equals_lora_down():
    """x @ (hi + lo)^T in fp64 equals the oracle's LoRA-down projection of
    the smoothed activation (the same exact products, summed in another
    order)."""
    g = torch.Generator().manual_seed(46)
    x = torch.randn(7, 80, generator=g).to(torch.bfloat16)
    p, l2 = _split_inputs(47, 5, 80)
    w = O.lora_weight_split(synth.bits(p), synth.bits(l2))
    wf = O.bf16_to_f32(w[0]).astype(np.float64) + O.bf16_to_f32(w[1]).astype(np.float64)
    d = O.lora_down(synth.bits(x), synth.bits(p), synth.bits(l2))
    assert np.allclose(x.double().numpy() @ wf.T, d, rtol=1e-13, atol=1e-15)


def unit_scale_operand(rng, E, rows, k, codes=None):
    """E matrices of random e2m1 codes (all 16) with every block scale 1.0
    (ue4m3 code 0x38), padding scale bytes 0."""
    if codes is None:
        codes = rng.integers(0, 16, size=(E, rows, k))
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    sf = np.zeros((E, O.sf_size(rows, k)), dtype=np.uint8)
    for r in range(rows):
        for c in range(k // 16):
            sf[:, swz(r, c, k)] = 0x38
    return codes, packed, sf


def int_products(ca, cb):
    """2*e2m1 values are the integers 0,1,2,3,4,6,8,12 (signed): exact
    integer matmul of [E, m, k] and [E, n, k] code arrays, in units of 1/4."""
    lut = np.array([int(2 * e2m1_frac(c)) for c in range(16)], dtype=np.int64)
    return np.einsum("emk,enk->emn", lut[ca], lut[cb])


def test_gemm_silu_quantize_exact_products():
    """With unit block scales and a power-of-two alpha every product and every
    partial sum is exact in fp32, so h is the integer matmul scaled, rounded
    once to bf16; the composition must equal the silu quantize of that h."""
    rng = np.random.default_rng(31)
    E, m, n2, k = 3, 40, 96, 64
    ca, a, asf = unit_scale_operand(rng, E, m, k)
    cb, b, bsf = unit_scale_operand(rng, E, n2, k)
    alpha = np.full(E, 2.0 ** -3, dtype=np.float32)
    gs = np.array([3.0, 100.0, 7.5], dtype=np.float32)
    mask = np.array([40, 17, 0], dtype=np.int32)
    acc = int_products(ca, cb)                       # units of 1/4, |acc| <= 64 * 144
    hv = (acc.astype(np.float64) / 4.0 * 2.0 ** -3).astype(np.float32)
    assert np.array_equal(hv.astype(np.float64), acc / 4.0 * 2.0 ** -3)   # exact in fp32
    h = O.f32_to_bf16(hv).reshape(E, m, n2)
    for e in range(E):
        h[e, mask[e]:] = 0
    want_q, want_sf, _ = O.quantize(h, prologue=O.PRO_SILU, mask=mask, gs=gs, gs_mode=O.STATIC)
    got_q, got_sf = O.gemm_silu_quantize(a, b, asf, bsf, alpha, gs, mask, m, n2, k)
    assert np.array_equal(got_q, want_q)
    assert np.array_equal(got_sf, want_sf)
    assert not got_q[1, 17:].any() and not got_q[2].any()


def test_gemm_silu_quantize_gate_is_first_half():
    """Up rows that select a column of ones make u = 1, so the result is the
    plain quantize of bf16(silu(g)); gate and up swapped would give
    silu(1) * g instead."""
    rng = np.random.default_rng(32)
    E, m, H, k = 1, 24, 32, 32
    ca = rng.integers(0, 16, size=(E, m, k))
    ca[..., 0] = 2                                   # e2m1 code 2 = 1.0
    ca, a, asf = unit_scale_operand(rng, E, m, k, ca)
    cb = rng.integers(0, 16, size=(E, 2 * H, k))
    cb[:, H:, :] = 0
    cb[:, H:, 0] = 2                                 # up row = e_0 -> u = 1
    cb, b, bsf = unit_scale_operand(rng, E, 2 * H, k, cb)
    alpha = np.ones(E, dtype=np.float32)
    gs = np.array([50.0], dtype=np.float32)
    mask = np.array([m], dtype=np.int32)
    g = (int_products(ca, cb)[0, :, :H] / 4.0).astype(np.float32)
    sg = np.array([O.silu(v) for v in g.ravel()], dtype=np.float32)
    hs = O.f32_to_bf16(sg).reshape(m, H)
    want_q, want_sf, _ = O.quantize(hs, gs=gs, gs_mode=O.STATIC)
    got_q, got_sf = O.gemm_silu_quantize(a, b, asf, bsf, alpha, gs, mask, m, 2 * H, k)
    assert np.array_equal(got_q[0], want_q)
    assert np.array_equal(got_sf[0], want_sf)


def test_f64_to_bf16_via_f32_double_rounding():
    """fp64 -> fp32 -> bf16: ties at each step go to even; a value just above
    a bf16 tie that fp32 rounds onto the tie then rounds to even."""
    v = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -40, 1.0 + 3 * 2.0 ** -8, -0.0, 2.0 ** 130])
    got = O.f64_to_bf16_via_f32(v)
    # 1+2^-8 is the bf16 tie between 1 and 1+2^-7 (even: 1); + 2^-40 is lost in
    # fp32 (1 + 2^-8 exactly), so the tie again goes to 1; 1+3*2^-8 ties to 1+2^-6
    assert got.tolist() == [0x3F80, 0x3F80, 0x3F80, 0x3F82, 0x8000, 0x7F80]
