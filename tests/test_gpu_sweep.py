"""Seeded sweeps of random odd shapes through every entry point, each case
against the oracle to the same bar as the targeted tests (bytes bit-exact,
GEMM rows within 1e-2 of the row maximum).  The shapes are drawn once from a
fixed seed, so a failure names a reproducible case; they land on both sides
of every kernel-selection threshold (M = 64 skinny / tiled, tile counts,
K % 128, one-launch / three-kernel dynamic quantize)."""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import np_bits, row_tolerance_check, say
from test_gpu_gemm import gemm_case, grouped_case, oq, t_u8
from test_gpu_quantize import run_batched, run_single
from test_gpu_swiglu import composed, fused, quantized_operands, assert_close_quantized, check_masked_rows

pytestmark = pytest.mark.gpu

RNG = np.random.default_rng(20261203)


def draw(n, fn):
    return [fn(RNG) for _ in range(n)]


QUANT = draw(60, lambda r: (int(r.integers(1, 400)), 16 * int(r.integers(1, 160)), bool(r.integers(0, 2)),
                            bool(r.integers(0, 2)), bool(r.integers(0, 2))))
BATCHED = draw(30, lambda r: (int(r.integers(1, 5)), int(r.integers(1, 260)), 16 * int(r.integers(1, 48)),
                             bool(r.integers(0, 2)), bool(r.integers(0, 2))))
GEMM = draw(60, lambda r: (int(r.integers(1, 520)), int(r.integers(1, 700)), 16 * int(r.integers(1, 80)),
                           bool(r.integers(0, 2))))
GROUPED = draw(20, lambda r: (int(r.integers(1, 5)), int(r.integers(1, 300)), int(r.integers(1, 300)),
                             16 * int(r.integers(1, 40))))
SVD = draw(20, lambda r: (int(r.integers(1, 300)), int(r.integers(1, 300)), 16 * int(r.integers(1, 40)),
                         32 * int(r.integers(1, 5))))
W4 = draw(30, lambda r: (int(r.integers(1, 100)), int(r.integers(1, 500)), 16 * int(r.integers(1, 100)),
                        bool(r.integers(0, 2))))
SWIGLU = draw(16, lambda r: (int(r.integers(1, 4)), int(r.integers(1, 300)), 16 * int(r.integers(1, 30)),
                            16 * int(r.integers(1, 40))))
MX = draw(40, lambda r: (int(r.integers(1, 400)), int(r.integers(1, 600)), 32 * int(r.integers(1, 60))))


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from nvfp4_block_scaled_04_amd import ops as _ops
    return _ops


@pytest.mark.parametrize("case", QUANT, ids=lambda c: "x".join(map(str, c)))
def test_quantize(ops, case):
    m, k, f32, dynamic, smooth = case
    g = torch.Generator().manual_seed(m * 7919 + k)
    x = torch.randn(m, k, generator=g) * torch.exp(torch.randn(m, 1, generator=g))
    x = x if f32 else x.to(torch.bfloat16)
    pqs = torch.exp(0.5 * torch.randn(k, generator=g)).to(torch.bfloat16) if smooth else None
    mode = ops.GS_DYNAMIC if dynamic else ops.GS_STATIC
    run_single(ops, x, mode, gs=None if dynamic else float(np.float32(2688.0 / 9.0)), pqs=pqs)


@pytest.mark.parametrize("case", BATCHED, ids=lambda c: "x".join(map(str, c)))
def test_batched_and_silu(ops, case):
    b, m, k, silu, dynamic = case
    g = torch.Generator().manual_seed(b * 31 + m * 7 + k)
    x = torch.randn(b, m, 2 * k if silu else k, generator=g).to(torch.bfloat16)
    mask = torch.randint(0, m + 1, (b,), generator=g, dtype=torch.int32)
    gs = None if dynamic else torch.full((b,), 2688.0 / 6.0, dtype=torch.float32)
    run_batched(ops, x, mask, ops.GS_DYNAMIC if dynamic else ops.GS_STATIC, silu=silu, gs=gs)


@pytest.mark.parametrize("case", GEMM, ids=lambda c: "x".join(map(str, c)))
def test_gemm(ops, case):
    m, n, k, bias = case
    g = torch.Generator().manual_seed(m * 131 + n * 7 + k)
    a = (torch.randn(m, k, generator=g) * 2).to(torch.bfloat16)
    w = (torch.randn(n, k, generator=g) * 0.02).to(torch.bfloat16)
    b = (torch.randn(n, generator=g) * 0.1).to(torch.bfloat16) if bias else None
    rows = np.unique(np.random.default_rng(m + n + k).integers(0, m, size=min(m, 24)))
    gemm_case(ops, a, w, bias=b, rows=rows, label="sweep")


@pytest.mark.parametrize("case", GROUPED, ids=lambda c: "x".join(map(str, c)))
def test_grouped(ops, case):
    E, m, n, k = case
    mask = np.random.default_rng(E + m + n + k).integers(0, m + 1, size=E).tolist()
    grouped_case(ops, E, m, n, k, mask, rows_per_expert=12, seed=E * 17 + m + n + k)


@pytest.mark.parametrize("case", SVD, ids=lambda c: "x".join(map(str, c)))
def test_svdquant(ops, case):
    m, n, k, r = case
    say("svdquant sweep", (m, n, k, r))
    g = torch.Generator().manual_seed(m + 3 * n + 7 * k + r)
    a = (torch.randn(m, k, generator=g) * 2).to(torch.bfloat16)
    w = (torch.randn(n, k, generator=g) * 0.02).to(torch.bfloat16)
    d = (torch.randn(m, r, generator=g) * 0.5).to(torch.bfloat16)
    l1 = (torch.randn(n, r, generator=g) * 0.05).to(torch.bfloat16)
    bias = (torch.randn(n, generator=g) * 0.1).to(torch.bfloat16)
    qa, sa, ga = oq(a)
    qb, sb, gb = oq(w)
    alpha = np.float32(1.0) / (ga[0] * gb[0])
    out = ops.nvfp4_gemm_svdquant(t_u8(qa), t_u8(qb), t_u8(sa), t_u8(sb),
                                  torch.tensor([alpha], dtype=torch.float32, device="cuda"),
                                  d.cuda(), l1.cuda(), bias=bias.cuda())
    torch.cuda.synchronize()
    ref = O.gemm_rows(qa, qb, sa, sb, alpha, m, n, k, bias=np_bits(bias), d=np_bits(d), l1=np_bits(l1))
    assert row_tolerance_check(out.float().cpu().numpy(), ref) <= 1e-2


@pytest.mark.parametrize("case", W4, ids=lambda c: "x".join(map(str, c)))
def test_w4a16(ops, case):
    m, n, k, bias = case
    say("w4a16 sweep", (m, n, k), bias)
    g = torch.Generator().manual_seed(m * 11 + n + k)
    a = (torch.randn(m, k, generator=g) * 2).to(torch.bfloat16)
    w = (torch.randn(n, k, generator=g) * 0.02).to(torch.bfloat16)
    b = (torch.randn(n, generator=g) * 0.1).to(torch.bfloat16) if bias else None
    qb, sb, gb = oq(w)
    alpha = np.float32(1.0) / gb[0]
    out = ops.nvfp4_gemm_w4a16(a.cuda(), t_u8(qb), t_u8(sb), torch.tensor([alpha], dtype=torch.float32, device="cuda"),
                               bias=None if b is None else b.cuda())
    torch.cuda.synchronize()
    ref = O.gemm_w4a16_rows(np_bits(a), qb, sb, alpha, m, n, k, bias=None if b is None else np_bits(b))
    assert row_tolerance_check(out.float().cpu().numpy(), ref) <= 1e-2


@pytest.mark.parametrize("case", SWIGLU, ids=lambda c: "x".join(map(str, c)))
def test_swiglu(ops, case):
    E, m, H, k = case
    say("swiglu sweep", (E, m, H, k))
    mk = np.random.default_rng(E + m + H + k).integers(0, m + 1, size=E).astype(np.int32)
    qa, sa, qb, sb, alpha = quantized_operands(E, m, 2 * H, k, mk, seed=E + m + H + k)
    gs = np.full(E, 2688.0 / 3.0, dtype=np.float32)
    args = (t_u8(qa), t_u8(qb), t_u8(sa), t_u8(sb), torch.from_numpy(alpha).cuda(),
            torch.from_numpy(mk).cuda(), torch.from_numpy(gs).cuda(), m, H)
    got_q, got_sf = fused(ops, *args)
    two_q, two_sf = composed(ops, *args)
    check_masked_rows(got_q, mk, m)
    assert np.array_equal(got_q, two_q) and np.array_equal(got_sf, two_sf)
    want_q, want_sf = O.gemm_silu_quantize(qa, qb, sa, sb, alpha, gs, mk, m, 2 * H, k)
    for e in range(E):
        if mk[e]:
            rows = np.arange(int(mk[e]))
            assert_close_quantized(got_q[e], got_sf[e], rows, want_q[e], want_sf[e], rows, H)


@pytest.mark.parametrize("case", MX, ids=lambda c: "x".join(map(str, c)))
def test_mx(ops, case):
    m, n, k = case
    say("mx sweep", (m, n, k))
    g = torch.Generator().manual_seed(m * 3 + n * 5 + k)
    a = (torch.randn(m, k, generator=g) * 2).to(torch.bfloat16)
    w = (torch.randn(n, k, generator=g) * 0.02).to(torch.bfloat16)
    fa, sfa = ops.mxfp4_quantize(a.cuda())
    fw, sfw = ops.mxfp4_quantize(w.cuda())
    out = ops.mxfp4_gemm(fa, fw, sfa, sfw)
    torch.cuda.synchronize()
    qa, sa = O.quantize_mx(np_bits(a))
    qb, sb = O.quantize_mx(np_bits(w))
    assert np.array_equal(fa.cpu().numpy(), qa) and np.array_equal(sfa.cpu().numpy(), sa)
    assert np.array_equal(fw.cpu().numpy(), qb) and np.array_equal(sfw.cpu().numpy(), sb)
    ref = O.gemm_mx_rows(qa, qb, sa, sb, 1.0, m, n, k)
    assert row_tolerance_check(out.float().cpu().numpy(), ref) <= 1e-2
