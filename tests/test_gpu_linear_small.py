"""nvfp4_linear_small (the dynamic-scale NVFP4 linear for at most 16 rows in
one launch) against the three calls it stands for -- nvfp4_quantize in
DYNAMIC mode, nvfp4_alpha, nvfp4_gemm -- bit for bit (output and the
activation's gs), and against the oracle: gs bits, and every output row
within the GEMM bar of the oracle's dequantize-then-matmul (NVIDIA/Fuser PR
#5737, the scaled mm's eager meaning) of the oracle's own quantization."""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import OUT_CANARY, assert_all_written, dev, np_bits, row_tolerance_check, say

pytestmark = pytest.mark.gpu
TOL = 1e-2


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from nvfp4_block_scaled_04_amd import ops as _ops
    return _ops


def t_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def draw(m, n, k, seed, outliers=True):
    g = torch.Generator("cpu").manual_seed(seed)
    x = torch.randn(m, k, generator=g)
    if outliers:
        cols = torch.randperm(k, generator=g)[: max(1, k // 100)]
        x[:, cols] *= 20.0
    w = 0.02 * torch.randn(n, k, generator=g)
    bias = torch.randn(n, generator=g)
    return x.to(torch.bfloat16), w.to(torch.bfloat16), bias.to(torch.bfloat16)


def run_case(ops, x, w, bias=None, label=""):
    m, k = x.shape
    n = w.shape[0]
    say("linear_small", label, (m, n, k), "bias", bias is not None)
    qb, sb, gb = O.quantize(np_bits(w))
    b, b_sf = t_u8(qb), t_u8(sb)
    gsb = torch.from_numpy(gb).to("cuda")
    xd = dev(x)
    bd = None if bias is None else dev(bias)
    out_bits = torch.full((m, n), OUT_CANARY, dtype=torch.int16, device="cuda")
    gs_out = torch.zeros(1, dtype=torch.float32, device="cuda")
    ops.nvfp4_linear_small(xd, b, b_sf, gsb, bias=bd, out=out_bits.view(torch.bfloat16), gs_out=gs_out)
    # the three calls
    fa, sfa, gsa = ops.nvfp4_quantize(xd)
    alpha = ops.nvfp4_alpha(gsa, gsb)
    ref_out = ops.nvfp4_gemm(fa, b, sfa, b_sf, alpha, bias=bd)
    torch.cuda.synchronize()
    assert_all_written(out_bits)
    assert np_bits(gs_out).view(np.uint32)[0] == np_bits(gsa).view(np.uint32)[0]
    got = out_bits.cpu().numpy()
    want = ref_out.view(torch.int16).cpu().numpy()
    assert np.array_equal(got, want), f"{int((got != want).sum())} outputs differ from the three calls"
    # the oracle
    qa, sa, ga = O.quantize(np_bits(x))
    assert np_bits(gs_out).view(np.uint32)[0] == ga.view(np.uint32)[0]
    al = np.float32(1.0) / (ga[0] * gb[0])
    ref = O.gemm_rows(qa, qb, sa, sb, al, m, n, k, rows=np.arange(m),
                      bias=None if bias is None else np_bits(bias))
    ratio = row_tolerance_check(out_bits.view(torch.bfloat16).float().cpu().numpy(), ref)
    print(f"  worst row error / row max = {ratio:.3e}")
    assert ratio <= TOL


@pytest.mark.parametrize("m,n,k", [(16, 4096, 4096), (1, 16, 128), (5, 33, 256), (16, 17, 128),
                                   (3, 100, 1152), (8, 64, 2048), (16, 64, 3968), (11, 1000, 640),
                                   (16, 130, 4096)])
def test_shapes(ops, m, n, k):
    x, w, _ = draw(m, n, k, seed=m * 7 + n + k)
    run_case(ops, x, w, label="shape")


@pytest.mark.parametrize("m,n,k", [(16, 4096, 4096), (7, 50, 384)])
def test_bias(ops, m, n, k):
    x, w, bias = draw(m, n, k, seed=99 + m)
    run_case(ops, x, w, bias=bias, label="bias")


def test_zero_and_special_values(ops):
    """All-zero activation (gs from the 1e-12 clamp), then inf / NaN /
    subnormal entries (nan_to_num before the amax and the blocks)."""
    x, w, _ = draw(16, 64, 512, seed=5)
    run_case(ops, torch.zeros_like(x), w, label="zeros")
    xs = x.clone()
    xs[0, 3] = float("inf")
    xs[2, 100] = float("-inf")
    xs[5, 17] = float("nan")
    xs[9, 0:16] = torch.tensor(1e-40).to(torch.bfloat16)
    run_case(ops, xs, w, label="inf/nan/subnormal")


def test_two_calls_in_a_row(ops):
    """A second call with fewer rows and another K reuses nothing of the
    first (every LDS entry the K loop reads is written by each call)."""
    x, w, _ = draw(16, 256, 4096, seed=11)
    run_case(ops, x, w, label="first")
    x2, w2, _ = draw(3, 48, 256, seed=12)
    run_case(ops, x2, w2, label="second")


def test_unsupported_shapes_are_refused(ops):
    x, w, _ = draw(17, 64, 256, seed=3)
    qb, sb, gb = O.quantize(np_bits(w))
    gsb = torch.from_numpy(gb).to("cuda")
    with pytest.raises(RuntimeError):
        ops.nvfp4_linear_small(dev(x), t_u8(qb), t_u8(sb), gsb)
    x, w, _ = draw(4, 64, 4224, seed=4)
    qb, sb, gb = O.quantize(np_bits(w))
    gsb = torch.from_numpy(gb).to("cuda")
    with pytest.raises(RuntimeError):
        ops.nvfp4_linear_small(dev(x), t_u8(qb), t_u8(sb), gsb)
