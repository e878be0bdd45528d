"""The allocation-free entry point (nvfp4_quantize_noalloc: partial maxima in
the library's static device array) against the workspace entry point it
varies (nvfp4_quantize_ws), through the C ABI: FP4 bytes, scale bytes, gs
and alpha bit for bit, on two calls in a row -- the second on a smaller
tensor, so anything the first call left in the shared array must not leak
into it -- and a third on an fp32 tensor with the smoothing prologue."""
import numpy as np
import pytest
import torch

from gpu_util import canary, np_bits, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from nvfp4_block_scaled_04_amd import ops as _ops
    return _ops


def both(ops, x, pqs=None):
    m, k = x.shape
    gs_w = torch.full((1,), 2688.0 / 0.137, dtype=torch.float32, device="cuda")
    outs = []
    for which in ("ws", "noalloc"):
        o4, osf = canary((m, k // 2)), canary((ops.sf_size(m, k),))
        gs = torch.zeros(1, dtype=torch.float32, device="cuda")
        alpha = torch.full((1,), float("nan"), dtype=torch.float32, device="cuda")
        if which == "ws":
            ws = torch.full((ops.QUANTIZE_WS_BYTES,), 0xFF, dtype=torch.uint8, device="cuda")
            ops.nvfp4_quantize_ws(x, ws, gs, ops.GS_DYNAMIC, pre_quant_scale=pqs, gs_other=gs_w, alpha=alpha,
                                  out_fp4=o4, out_sf=osf)
        else:
            ops.nvfp4_quantize_noalloc(x, gs, gs_other=gs_w, alpha=alpha, pre_quant_scale=pqs,
                                       out_fp4=o4, out_sf=osf)
        outs.append((o4, osf, gs, alpha))
    torch.cuda.synchronize()
    (a4, asf, ag, aa), (b4, bsf, bg, ba) = outs
    assert torch.equal(a4, b4), int((a4 != b4).sum())
    assert torch.equal(asf, bsf), int((asf != bsf).sum())
    assert np_bits(ag).view(np.uint32)[0] == np_bits(bg).view(np.uint32)[0]
    assert np_bits(aa).view(np.uint32)[0] == np_bits(ba).view(np.uint32)[0]


def test_noalloc_matches_workspace_entry_point(ops):
    g = torch.Generator().manual_seed(21)
    big = (torch.randn(4100, 5120, generator=g) * 2).to(torch.bfloat16)
    big[:, 17] *= 40.0                       # the largest magnitude sits in one column
    small = (torch.randn(300, 1040, generator=g) * 0.5).to(torch.bfloat16)
    say("noalloc vs ws: large, then small")
    both(ops, big.cuda())
    both(ops, small.cuda())
    say("noalloc vs ws: fp32 with the smoothing prologue")
    x32 = torch.randn(640, 256, generator=g) * 3
    pqs = torch.exp(0.4 * torch.randn(256, generator=g)).to(torch.bfloat16)
    both(ops, x32.cuda(), pqs=pqs.cuda())
