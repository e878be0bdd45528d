"""GPU parity of the MX setting (32-element blocks, ue8m0 scales): the
quantizer bit for bit against the oracle (FP4 and scale bytes), the GEMM on
gfx950's block-scaled MFMA within max|gpu - oracle| <= 1e-2 * max|oracle row|.
"""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import OUT_CANARY, assert_all_written, np_bits, row_tolerance_check, say, tile_rows

pytestmark = pytest.mark.gpu

CANARY = 0xA5
TOL = 1e-2


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from nvfp4_block_scaled_04_amd import ops as _ops
    return _ops


def t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def quantize_both(ops, x_cpu):
    m, k = x_cpu.shape
    q = torch.full((m, k // 2), CANARY, dtype=torch.uint8, device="cuda")
    sf = torch.full((O.sf_size_mx(m, k),), CANARY, dtype=torch.uint8, device="cuda")
    ops.mxfp4_quantize(x_cpu.to("cuda"), out_fp4=q, out_sf=sf)
    torch.cuda.synchronize()
    wq, wsf = O.quantize_mx(np_bits(x_cpu))
    return q.cpu().numpy(), sf.cpu().numpy(), wq, wsf


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("m,k", [(1, 32), (37, 96), (128, 256), (129, 160), (300, 992), (64, 4096)])
def test_quantize_bit_exact(ops, dtype, m, k):
    say("mx quantize", dtype, (m, k))
    g = torch.Generator().manual_seed(m * 7 + k)
    x = torch.randn(m, k, generator=g) * torch.exp(torch.randn(m, 1, generator=g) * 2)
    x[:, ::17] *= 25.0
    x = x.to(dtype)
    gq, gsf, wq, wsf = quantize_both(ops, x)
    assert np.array_equal(gq, wq)
    assert np.array_equal(gsf, wsf)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_quantize_special_values(ops, dtype):
    say("mx quantize special", dtype)
    x = torch.randn(4, 256, generator=torch.Generator().manual_seed(3))
    x[0, :32] = 0.0
    x[0, 7] = -0.0
    x[0, 32:64] = 2.0 ** -130 if dtype == torch.float32 else 2.0 ** -126
    x[1, :32] = torch.linspace(-7.9, 7.9, 32)
    x[1, 32:64] = 1.0
    x[2, :] = 3.0e38
    x[2, 3] = float("inf")
    x[2, 4] = float("-inf")
    x[2, 5] = float("nan")
    x[3, :32] = torch.arange(32) * 0.25
    x[3, 64:96] = -(2.0 ** 100)
    x = x.to(dtype)
    gq, gsf, wq, wsf = quantize_both(ops, x)
    assert np.array_equal(gq, wq)
    assert np.array_equal(gsf, wsf)


def test_quantize_prefill_activation(ops):
    """The prefill activation (8192 x 5120 bf16 with outlier channels), every byte."""
    from nvfp4_block_scaled_04_amd import synth
    d = synth.prefill()
    say("mx quantize prefill", tuple(d.a.shape))
    gq, gsf, wq, wsf = quantize_both(ops, d.a)
    assert np.array_equal(gq, wq)
    assert np.array_equal(gsf, wsf)


def gemm_case(ops, m, n, k, bias=False, rows=None, seed=0, alpha=0.5):
    say("mx gemm", (m, n, k), "bias", bias)
    g = torch.Generator().manual_seed(seed + m + n + k)
    a = (torch.randn(m, k, generator=g) * 2).to(torch.bfloat16)
    w = (torch.randn(n, k, generator=g) * 0.02).to(torch.bfloat16)
    b16 = (torch.randn(n, generator=g) * 0.1).to(torch.bfloat16) if bias else None
    qa, sa = O.quantize_mx(np_bits(a))
    qb, sb = O.quantize_mx(np_bits(w))
    out_bits = torch.full((m, n), OUT_CANARY, dtype=torch.int16, device="cuda")
    out = out_bits.view(torch.bfloat16)
    al = torch.tensor([alpha], dtype=torch.float32, device="cuda") if alpha is not None else None
    ops.mxfp4_gemm(t(qa), t(qb), t(sa), t(sb), alpha=al, bias=None if b16 is None else b16.to("cuda"), out=out)
    torch.cuda.synchronize()
    assert_all_written(out_bits)
    if rows is None:
        rows = np.arange(m)
    ref = O.gemm_mx_rows(qa, qb, sa, sb, 1.0 if alpha is None else alpha, m, n, k, rows=rows,
                         bias=None if b16 is None else np_bits(b16))
    got = out.float().cpu().numpy()[rows]
    ratio = row_tolerance_check(got, ref)
    print(f"  worst row error / row max = {ratio:.3e}")
    assert ratio <= TOL
    return ratio


@pytest.mark.parametrize("m,n,k", [(1, 1, 32), (16, 33, 96), (127, 64, 128), (129, 257, 416),
                                   (256, 512, 1024), (300, 200, 4064)])
def test_gemm_ragged(ops, m, n, k):
    gemm_case(ops, m, n, k, bias=(m % 2 == 1))


def test_gemm_no_alpha(ops):
    gemm_case(ops, 64, 128, 256, alpha=None)


def test_gemm_large_tile(ops):
    """4096 x 4096 (the 256 x 256 tile), K % 128 != 0, sampled rows."""
    rows = np.array([0, 1, 255, 256, 1000, 2047, 2048, 4095])
    gemm_case(ops, 4096, 4096, 544, bias=True, rows=rows)


def test_gemm_prefill_shape(ops):
    """The prefill linear 8192 x 16384 x 5120 (the bench's launch): every
    output written (canary), 512 rows stratified over the 32 M-tiles of 256
    against the oracle; operands quantized by the oracle."""
    from nvfp4_block_scaled_04_amd import synth
    d = synth.prefill()
    say("mx gemm prefill", (d.m, d.n, d.k))
    qa, sa = O.quantize_mx(np_bits(d.a))
    qb, sb = O.quantize_mx(np_bits(d.w))
    out_bits = torch.full((d.m, d.n), OUT_CANARY, dtype=torch.int16, device="cuda")
    out = ops.mxfp4_gemm(t(qa), t(qb), t(sa), t(sb), out=out_bits.view(torch.bfloat16))
    torch.cuda.synchronize()
    assert_all_written(out_bits)
    rows = tile_rows(d.m, 256, 16, 6)
    ref = O.gemm_mx_rows(qa, qb, sa, sb, 1.0, d.m, d.n, d.k, rows=rows)
    ratio = row_tolerance_check(out.float().cpu().numpy()[rows], ref)
    print(f"  worst row error / row max = {ratio:.3e}")
    assert ratio <= TOL
