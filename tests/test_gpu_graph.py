"""The library's launches under HIP graph capture.

The kernels clear and reduce with kernels of their own (no memset nodes, no
host synchronisation), so a captured call sequence must replay to the same
bytes as the eager calls.  Each graph is replayed several times with eager
work of the program in between (other launches on the same buffers), and
every replay is checked against the eager result."""
import numpy as np
import pytest
import torch

from nvfp4_block_scaled_04_amd import synth
from gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from nvfp4_block_scaled_04_amd import ops as _ops
    return _ops


def _capture(fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


@pytest.mark.parametrize("shape", [(16, 4096, 4096), (512, 1024, 2048), (2048, 4096, 4096)])
def test_dynamic_pipeline_replays(ops, shape):
    """Dynamic quantize (one-launch small-item and three-kernel paths), alpha, GEMM (skinny,
    K-split and tiled kernels) captured once, replayed three times."""
    m, n, k = shape
    say("graph pipeline", shape)
    d, _ = synth.dense(m=m, n=n, k=k)
    x = d.a.to("cuda")
    fw, sfw, gsw = ops.nvfp4_quantize(d.w.to("cuda"))
    fa = torch.empty(m, k // 2, dtype=torch.uint8, device="cuda")
    sfa = torch.empty(ops.sf_size(m, k), dtype=torch.uint8, device="cuda")
    gsa = torch.zeros(1, dtype=torch.float32, device="cuda")
    alpha = torch.empty(1, dtype=torch.float32, device="cuda")
    out = torch.empty(m, n, dtype=torch.bfloat16, device="cuda")

    def step():
        ops.nvfp4_quantize(x, gsa, ops.GS_DYNAMIC, out_fp4=fa, out_sf=sfa)
        ops.nvfp4_alpha(gsa, gsw, out=alpha)
        ops.nvfp4_gemm(fa, fw, sfa, sfw, alpha, out=out)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (fa, sfa, gsa, alpha, out)]
    g = _capture(step)
    for rep in range(3):
        for t in (fa, sfa, gsa, alpha, out):   # eager work between replays: scribble the outputs
            t.view(torch.uint8).fill_(0xA5 + rep)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, t, r in zip(("fp4", "scales", "gs", "alpha", "out"), (fa, sfa, gsa, alpha, out), ref):
            assert torch.equal(t.view(torch.uint8), r.view(torch.uint8)), f"replay {rep}: {name} differs"


def test_linear_small_replays(ops):
    """The one-launch decode linear captured once, replayed three times with
    its output and gs scribbled in between; every replay equals the eager
    call, which equals the three captured-apart calls (quantize, alpha, GEMM)."""
    m, n, k = 16, 4096, 4096
    say("graph linear_small", (m, n, k))
    d, _ = synth.dense(m=m, n=n, k=k)
    x = d.a.to("cuda")
    fw, sfw, gsw = ops.nvfp4_quantize(d.w.to("cuda"))
    out = torch.empty(m, n, dtype=torch.bfloat16, device="cuda")
    gs = torch.zeros(1, dtype=torch.float32, device="cuda")

    def step():
        ops.nvfp4_linear_small(x, fw, sfw, gsw, out=out, gs_out=gs)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (out, gs)]
    fa, sfa, gsa = ops.nvfp4_quantize(x)
    three = ops.nvfp4_gemm(fa, fw, sfa, sfw, ops.nvfp4_alpha(gsa, gsw))
    torch.cuda.synchronize()
    assert torch.equal(three.view(torch.uint8), ref[0].view(torch.uint8))
    assert torch.equal(gsa.view(torch.uint8), ref[1].view(torch.uint8))
    g = _capture(step)
    for rep in range(3):
        for t in (out, gs):
            t.view(torch.uint8).fill_(0xA5 + rep)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, t, r in zip(("out", "gs"), (out, gs), ref):
            assert torch.equal(t.view(torch.uint8), r.view(torch.uint8)), f"replay {rep}: {name} differs"


@pytest.mark.parametrize("ws", [False, True])
def test_moe_pipeline_replays(ops, ws):
    """silu quantize over masked experts, per-expert alpha, grouped masked
    GEMM; with ws: the silu quantize with a workspace holding h (alpha from
    the same call) and the grouped GEMM with its split-tail workspace, both
    workspaces overwritten with stale bytes between replays."""
    E, m, h, n = 4, 256, 512, 768
    say("graph moe", (E, m, h, n), "ws", ws)
    mo = synth.moe(e=E, m=m, h=h, n=n)
    x = mo.x.to("cuda")
    mask = mo.mask.to("cuda")
    fws, sfws, gsws = [], [], []
    for e in range(E):
        f_, s_, g_ = ops.nvfp4_quantize(mo.w[e].to("cuda"))
        fws.append(f_); sfws.append(s_); gsws.append(g_)
    fw, sfw, gsw = torch.stack(fws), torch.stack(sfws), torch.cat(gsws)
    fa = torch.empty(E, m, h // 2, dtype=torch.uint8, device="cuda")
    sfa = torch.empty(E, ops.sf_size(m, h), dtype=torch.uint8, device="cuda")
    gsa = torch.zeros(E, dtype=torch.float32, device="cuda")
    alpha = torch.empty(E, dtype=torch.float32, device="cuda")
    out = torch.zeros(E, m, n, dtype=torch.bfloat16, device="cuda")

    qws = ops.silu_workspace(E, m, h, "cuda") if ws else None
    gws = ops.gemm_workspace("cuda") if ws else None

    def step():
        if ws:
            ops.silu_mul_nvfp4_quantize_ws(x, qws, mask, gsa, ops.GS_DYNAMIC, gs_other=gsw, alpha=alpha,
                                           out_fp4=fa, out_sf=sfa)
        else:
            ops.silu_mul_nvfp4_quantize(x, mask, gsa, ops.GS_DYNAMIC, out_fp4=fa, out_sf=sfa)
            ops.nvfp4_alpha(gsa, gsw, out=alpha)
        ops.nvfp4_gemm_grouped_masked(fa, fw, sfa, sfw, alpha, mask, out=out, workspace=gws)

    step()
    torch.cuda.synchronize()
    valid = mo.mask.clamp(0, m).tolist()
    ref_out = out.clone()
    ref = [t.clone() for t in (sfa, gsa, alpha)]
    ref_fa = [fa[e, :valid[e]].clone() for e in range(E)]
    g = _capture(step)
    for rep in range(3):
        for t in (fa, sfa, gsa, alpha) + ((qws, gws) if ws else ()):
            t.view(torch.uint8).fill_(0x3C + rep)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, t, r in zip(("scales", "gs", "alpha"), (sfa, gsa, alpha), ref):
            assert torch.equal(t.view(torch.uint8), r.view(torch.uint8)), f"replay {rep}: {name} differs"
        for e in range(E):
            assert torch.equal(fa[e, :valid[e]], ref_fa[e]), f"replay {rep}: fp4 of expert {e} differs"
            assert torch.equal(out[e, :valid[e]].view(torch.int16), ref_out[e, :valid[e]].view(torch.int16)), \
                f"replay {rep}: output of expert {e} differs"
