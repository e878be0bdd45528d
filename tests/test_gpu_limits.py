"""GPU tests at the largest sizes the boundary accepts.

* GEMMs whose weight spans just under 2^32 bytes (32767 x 262144 FP4, the
  limit of the kernels' 32-bit staging offsets), NVFP4 and MX, in the
  skinny and the tiled kernels.  Every row of A and of B is constant (its own
  e2m1 code and power-of-two block scale), so out[i, j] = alpha * K *
  a_i * b_j in closed form; with power-of-two scales and alpha every partial
  sum is exact in fp32, so all m x n outputs must equal bf16 of the closed
  form bit for bit, and a row fetched from a wrapped offset would show.
* Quantization with 65535 row tiles (the largest grid), compared with the
  oracle over every byte.
"""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import np_bits, say
from test_oracle_gemm import e2m1_frac

pytestmark = pytest.mark.gpu

E2M1 = np.array([float(e2m1_frac(c)) for c in range(16)])


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from nvfp4_block_scaled_04_amd import ops as _ops
    return _ops


def row_constant_operand(rows, k, codes, scale_codes, block):
    """Device FP4 matrix [rows, k/2] whose row r holds e2m1 code codes[r]
    everywhere, and its swizzled scale buffer (pad_up(rows,128) x
    pad_up(k/block, 4) bytes) with scale_codes[r] in every block of row r."""
    q = torch.from_numpy((codes | (codes << 4)).astype(np.uint8)).cuda()
    q = q[:, None].expand(rows, k // 2).contiguous()
    rpad = (rows + 127) // 128 * 128
    cgroups = ((k // block + 3) // 4 * 4) // 4
    sc = np.zeros(rpad, dtype=np.uint8)
    sc[:rows] = scale_codes
    # one 512-byte tile per (128-row tile, 4-column group): row r's 4 bytes
    # sit at (r % 32) * 16 + ((r % 128) // 32) * 4
    tile = np.zeros((rpad // 128, 512), dtype=np.uint8)
    r = np.arange(rpad)
    for b in range(4):
        tile[r // 128, (r % 32) * 16 + ((r % 128) // 32) * 4 + b] = sc
    sf = torch.from_numpy(tile).cuda()[:, None, :].expand(rpad // 128, cgroups, 512).contiguous().view(-1)
    return q, sf


def closed_form_check(out, a_val, b_val, k, alpha):
    """Every output equals bf16 of the closed form; values compare as numbers
    (a zero dot product of signed-zero terms may come out as +0 or -0)."""
    ref = (alpha * k) * np.outer(a_val, b_val)
    want = torch.from_numpy(ref.astype(np.float32)).to(torch.bfloat16)   # exact fp32, then RNE
    got = out.cpu()
    bad = (got.float() != want.float()).nonzero()
    assert bad.numel() == 0, (f"{bad.shape[0]} mismatches, first at {bad[0].tolist()}: "
                              f"{got[tuple(bad[0])].item()} vs {want[tuple(bad[0])].item()}")


@pytest.mark.parametrize("m", [16, 256, 1024])   # skinny, 128x256 split over K, 256x256
def test_nvfp4_gemm_largest_weight(ops, m):
    n, k = 32767, 262144
    assert n * (k // 2) <= 2 ** 32 - 64
    say("nvfp4 gemm largest weight", (m, n, k))
    i, j = np.arange(m), np.arange(n)
    ca, cb = (i * 5) % 16, (j * 7 + 3) % 16
    sa = np.array([0x30, 0x38, 0x40])[i % 3]          # ue4m3 0.5, 1, 2
    sb = np.array([0x38, 0x40, 0x30, 0x48])[j % 4]    # 1, 2, 0.5, 4
    qa, sfa = row_constant_operand(m, k, ca, sa, 16)
    qb, sfb = row_constant_operand(n, k, cb, sb, 16)
    alpha = 2.0 ** -22
    out = ops.nvfp4_gemm(qa, qb, sfa, sfb, torch.tensor([alpha], dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    dec = {0x30: 0.5, 0x38: 1.0, 0x40: 2.0, 0x48: 4.0}
    a_val = E2M1[ca] * np.array([dec[c] for c in sa])
    b_val = E2M1[cb] * np.array([dec[c] for c in sb])
    closed_form_check(out, a_val, b_val, k, alpha)
    del qb, sfb, out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("m", [16, 512])         # 128x128, 256x256
def test_mx_gemm_largest_weight(ops, m):
    n, k = 32767, 262144
    say("mx gemm largest weight", (m, n, k))
    i, j = np.arange(m), np.arange(n)
    ca, cb = (i * 3 + 1) % 16, (j * 11) % 16
    sa = np.array([126, 127, 128])[i % 3]             # e8m0 0.5, 1, 2
    sb = np.array([127, 129, 125])[j % 3]             # 1, 4, 0.25
    qa, sfa = row_constant_operand(m, k, ca, sa, 32)
    qb, sfb = row_constant_operand(n, k, cb, sb, 32)
    alpha = 2.0 ** -22
    out = ops.mxfp4_gemm(qa, qb, sfa, sfb, alpha=torch.tensor([alpha], dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    a_val = E2M1[ca] * 2.0 ** (sa.astype(np.float64) - 127)
    b_val = E2M1[cb] * 2.0 ** (sb.astype(np.float64) - 127)
    closed_form_check(out, a_val, b_val, k, alpha)
    del qb, sfb, out
    torch.cuda.empty_cache()


def test_quantize_most_row_tiles(ops):
    """65535 row tiles (8388480 rows x 16): the dynamic path's amax partials,
    finish and pass over the largest grid, every byte against the oracle."""
    m, k = 65535 * 128, 16
    say("quantize most row tiles", (m, k))
    g = torch.Generator().manual_seed(77)
    x = (torch.randn(m, k, generator=g) * 3).to(torch.bfloat16)
    q, sf, gs = ops.nvfp4_quantize(x.cuda())
    torch.cuda.synchronize()
    wq, wsf, wgs = O.quantize(np_bits(x))
    assert np_bits(gs).view(np.uint32)[0] == wgs.view(np.uint32)[0]
    assert np.array_equal(q.cpu().numpy(), wq)
    assert np.array_equal(sf.cpu().numpy(), wsf)


def test_mx_quantize_most_row_tiles(ops):
    m, k = 65535 * 128, 32
    say("mx quantize most row tiles", (m, k))
    g = torch.Generator().manual_seed(78)
    x = (torch.randn(m, k, generator=g) * torch.exp(torch.randn(m, 1, generator=g) * 4)).to(torch.bfloat16)
    q, sf = ops.mxfp4_quantize(x.cuda())
    torch.cuda.synchronize()
    wq, wsf = O.quantize_mx(np_bits(x))
    assert np.array_equal(q.cpu().numpy(), wq)
    assert np.array_equal(sf.cpu().numpy(), wsf)
