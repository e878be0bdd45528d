"""Seeded large ragged shapes for the GEMM paths that only large problems
select: the 256 x 256 tile (at least 512 tiles), one round of 256 x 192
tiles, the K-split 128 x 256 tile (128-256 tiles, an even number of K steps,
scales staged per 128-row band) and the split-tail schedule of a single
problem (more 128 x 256 tiles than CUs, given the workspace).  Every output
starts as the NaN canary and must be written; rows stratified over the
M-tiles (first and last row of every 128 rows and two more) are compared
with the oracle at the GEMM bar, max |gpu - oracle| <= 1e-2 * max |oracle
row| (NVIDIA/Fuser PR #5737: eager meaning = dequantize, then linear).  The
shapes are drawn once from a fixed seed, ragged in M, N and K, with and
without bias."""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import OUT_CANARY, assert_all_written, dev, np_bits, row_tolerance_check, say, tile_rows

pytestmark = pytest.mark.gpu
TOL = 1e-2
RNG = np.random.default_rng(20261204)


def _ragged(r, lo, hi):
    return int(r.integers(lo, hi + 1))


def _k(r, steps_lo, steps_hi, even=False):
    s = int(r.integers(steps_lo, steps_hi + 1))
    if even:
        s += s % 2
    # K = whole steps of 128, or a ragged last step (K % 128 != 0, K % 16 == 0)
    return 128 * s - (16 * int(r.integers(1, 8)) if r.integers(0, 2) else 0)


CASES = []
for _ in range(2):   # 256 x 256: >= 512 tiles
    CASES.append(("256x256", _ragged(RNG, 4097, 4500), _ragged(RNG, 8193, 8700), _k(RNG, 3, 10), False))
for _ in range(2):   # 256 x 192: 16 x 14..16 tiles, fewer than 512 of 256 x 256
    CASES.append(("256x192", _ragged(RNG, 3841, 4096), _ragged(RNG, 2689, 3072), _k(RNG, 4, 20), False))
for _ in range(2):   # K-split 128 x 256: 128-256 tiles
    CASES.append(("128x256 K split", _ragged(RNG, 1500, 2048), _ragged(RNG, 3000, 4096), _k(RNG, 4, 24, even=True),
                  False))
for _ in range(2):   # split-tail single problem: 14 x 19..24 tiles of 128 x 256, under 768 of 128 x 128
    CASES.append(("split tail", _ragged(RNG, 1665, 1792), _ragged(RNG, 4700, 5900), _k(RNG, 16, 40, even=True),
                  True))


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from nvfp4_block_scaled_04_amd import ops as _ops
    return _ops


@pytest.fixture(scope="module")
def ws(ops):
    return ops.gemm_workspace("cuda")


@pytest.mark.parametrize("idx", range(len(CASES)))
def test_large_ragged(ops, ws, idx):
    path, m, n, k, use_ws = CASES[idx]
    with_bias = idx % 2 == 1
    g = torch.Generator().manual_seed(1000 + idx)
    a = torch.randn(m, k, generator=g).to(torch.bfloat16)
    w = (torch.randn(n, k, generator=g) * 0.03).to(torch.bfloat16)
    bias = torch.randn(n, generator=g).to(torch.bfloat16) if with_bias else None
    say("large ragged", path, (m, n, k), "bias", with_bias, "workspace", use_ws)
    qa, sa, ga = O.quantize(np_bits(a))
    qb, sb, gb = O.quantize(np_bits(w))
    alpha = np.float32(1.0) / (ga[0] * gb[0])
    bits = torch.full((m, n), OUT_CANARY, dtype=torch.int16, device="cuda")
    out = bits.view(torch.bfloat16)
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to("cuda")
    ops.nvfp4_gemm(t(qa), t(qb), t(sa), t(sb), torch.tensor([alpha], dtype=torch.float32, device="cuda"),
                   bias=None if bias is None else dev(bias), out=out, k=k, workspace=ws if use_ws else None)
    torch.cuda.synchronize()
    assert_all_written(bits)
    rows = tile_rows(m, 128, 4, idx)
    ref = O.gemm_rows(qa, qb, sa, sb, alpha, m, n, k, rows=rows, bias=None if bias is None else np_bits(bias))
    ratio = row_tolerance_check(out.float().cpu().numpy()[rows], ref)
    print(f"  {len(rows)} rows, worst row error / row max = {ratio:.3e}")
    assert ratio <= TOL
