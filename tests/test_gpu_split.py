"""GPU parity of the split-tail GEMM schedule (the *_ws entry points and the
grouped form, which takes the same schedule without splitting when no
workspace is given).

When the output tiles do not divide evenly over the CUs, the last ("tail")
tiles' K loops are split over the CUs and their fp32 partial tiles are added
by a second launch in a fixed order.  Bar: the GEMM bar of the other parity
tests, max |gpu - oracle| <= 1e-2 * max |oracle row| on every compared row
(flashinfer PR #1774 grouped_gemm_nt_masked; NVIDIA/Fuser PR #5737: eager
meaning = dequantize, then linear).  Every output starts as a bf16 NaN
pattern the kernels never write, so a tile that no workgroup (or no fixup)
stored fails wherever it is; every row of every case is compared, so the
split tiles are covered wherever the schedule places them.  The split result
is also checked for determinism (two calls, same bits) and against the
unsplit schedule (same bar).
"""
import numpy as np
import pytest
import torch

import oracle as O
from nvfp4_block_scaled_04_amd import synth
from gpu_util import OUT_CANARY, assert_all_written, dev, np_bits, row_tolerance_check, say

pytestmark = pytest.mark.gpu
TOL = 1e-2


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from nvfp4_block_scaled_04_amd import ops as _ops
    return _ops


@pytest.fixture(scope="module")
def ws(ops):
    return ops.gemm_workspace("cuda")


def oq(x_cpu, **kw):
    return O.quantize(np_bits(x_cpu), **kw)


def t_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def canary_out(*shape):
    bits = torch.full(shape, OUT_CANARY, dtype=torch.int16, device="cuda")
    return bits, bits.view(torch.bfloat16)


@pytest.mark.parametrize("m,n,k", [
    (1664, 5120, 8192),   # 13 x 20 = 260 tiles of 128 x 256: 4 tail tiles, each split 8 ways
    (1100, 8200, 4000),   # 9 x 33 = 297 tiles, ragged M and N, K % 128 != 0: 41 tail tiles in 4 parts
])
def test_dense_split(ops, ws, m, n, k):
    g = torch.Generator().manual_seed(m + n + k)
    a = torch.randn(m, k, generator=g).to(torch.bfloat16)
    w = (torch.randn(n, k, generator=g) * 0.02).to(torch.bfloat16)
    say("split dense", (m, n, k))
    qa, sa, ga = oq(a)
    qb, sb, gb = oq(w)
    alpha = torch.tensor([np.float32(1.0) / (ga[0] * gb[0])], dtype=torch.float32, device="cuda")
    args = (t_u8(qa), t_u8(qb), t_u8(sa), t_u8(sb), alpha)
    bits, out = canary_out(m, n)
    ops.nvfp4_gemm(*args, out=out, workspace=ws)
    torch.cuda.synchronize()
    assert_all_written(bits)
    bits2, out2 = canary_out(m, n)
    ops.nvfp4_gemm(*args, out=out2, workspace=ws)
    plain = ops.nvfp4_gemm(*args)
    torch.cuda.synchronize()
    assert torch.equal(bits, bits2), "two calls of the split schedule differ"
    ref = O.gemm_rows(qa, qb, sa, sb, float(alpha.item()), m, n, k)
    got = out.float().cpu().numpy()
    ratio = row_tolerance_check(got, ref)
    print(f"  worst row error / row max = {ratio:.3e}")
    assert ratio <= TOL
    assert row_tolerance_check(got, plain.double().cpu().numpy()) <= TOL


def test_svdquant_split(ops, ws):
    """SVDQuant form (rank 32, bias) on 1664 x 5120 x 2048: 13 x 20 = 260
    tiles of 128 x 256, the 4 tail tiles split in two; the LoRA-up term
    enters the first part only, alpha and bias the launch adding the parts.
    Every row against the oracle."""
    m, n, k, r = 1664, 5120, 2048, 32
    g = torch.Generator().manual_seed(17)
    a = torch.randn(m, k, generator=g).to(torch.bfloat16)
    w = (torch.randn(n, k, generator=g) * 0.05).to(torch.bfloat16)
    say("split svdquant", (m, n, k), r)
    qa, sa, ga = oq(a)
    qb, sb, gb = oq(w)
    alpha = np.float32(1.0) / (ga[0] * gb[0])
    d = torch.randn(m, r, generator=g).to(torch.bfloat16)
    l1 = (torch.randn(n, r, generator=g) / float(alpha) * 1e-2).to(torch.bfloat16)
    bias = torch.randn(n, generator=g).to(torch.bfloat16)
    bits, out = canary_out(m, n)
    ops.nvfp4_gemm_svdquant(t_u8(qa), t_u8(qb), t_u8(sa), t_u8(sb),
                            torch.tensor([alpha], dtype=torch.float32, device="cuda"),
                            dev(d), dev(l1), bias=dev(bias), out=out, workspace=ws)
    torch.cuda.synchronize()
    assert_all_written(bits)
    ref = O.gemm_rows(qa, qb, sa, sb, alpha, m, n, k, bias=np_bits(bias), d=np_bits(d), l1=np_bits(l1))
    ratio = row_tolerance_check(out.float().cpu().numpy(), ref)
    print(f"  worst row error / row max = {ratio:.3e}")
    assert ratio <= TOL


def grouped_operands(E, m, n, h, mask, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(E, m, h, generator=g).to(torch.bfloat16)
    w = (torch.randn(E, n, h, generator=g) * 0.02).to(torch.bfloat16)
    mk = np.array(mask, dtype=np.int32)
    qa, sa, ga = oq(x, mask=mk)
    qb, sb, gb = oq(w)
    alpha = (np.float32(1.0) / (ga * gb)).astype(np.float32)
    return qa, sa, qb, sb, alpha, mk


def run_grouped(ops, qa, sa, qb, sb, alpha, mk, m, n, workspace):
    E = len(mk)
    bits, out = canary_out(E, m, n)
    ops.nvfp4_gemm_grouped_masked(t_u8(qa), t_u8(qb), t_u8(sa), t_u8(sb), torch.from_numpy(alpha).to("cuda"),
                                  torch.from_numpy(mk).to("cuda"), out=out, workspace=workspace)
    torch.cuda.synchronize()
    return bits.cpu()


def check_grouped(got_bits, qa, sa, qb, sb, alpha, mk, m, n, h):
    for e in range(len(mk)):
        v = int(min(max(mk[e], 0), m))
        assert bool((got_bits[e, v:] == OUT_CANARY).all()), f"expert {e}: rows >= {v} were written"
        assert not bool((got_bits[e, :v] == OUT_CANARY).any()), f"expert {e}: valid rows left unwritten"
        if v == 0:
            continue
        ref = O.gemm_rows(qa[e], qb[e], sa[e], sb[e], alpha[e], m, n, h, rows=np.arange(v))
        got = got_bits[e, :v].view(torch.bfloat16).float().numpy()
        ratio = row_tolerance_check(got, ref)
        assert ratio <= TOL, (e, ratio)


@pytest.mark.parametrize("n,h,mask", [
    (5120, 2048, [512] * 8),                             # 640 tiles: 2 whole rounds, 128 tail tiles in 2 parts
    (5120, 2048, [1, 0, 0, 0, 0, 0, 0, 0]),              # 20 tiles, each split in 2 (of 16 K steps)
    (5000, 2000, [0, 1, 129, 255, 256, 300, 512, 7]),    # ragged N, K % 128 != 0, 44 tail tiles in 2 parts
    (5000, 400, [0, 1, 129, 255, 256, 300, 512, 7]),     # K too short to split: tail tiles whole
    (5120, 512, [0] * 8),                                # nothing to compute
])
def test_grouped_split(ops, ws, n, h, mask):
    """Every valid row of every expert with and without the workspace, the
    split result deterministic."""
    E, m = 8, 512
    say("split grouped", (E, m, n, h), mask)
    ops_args = grouped_operands(E, m, n, h, mask, seed=n + h + sum(mask))
    got = run_grouped(ops, *ops_args, m, n, ws)
    again = run_grouped(ops, *ops_args, m, n, ws)
    assert torch.equal(got, again), "two calls of the split schedule differ"
    check_grouped(got, *ops_args, m, n, h)
    check_grouped(run_grouped(ops, *ops_args, m, n, None), *ops_args, m, n, h)


def test_moe_workload_split(ops, ws):
    """The routed-expert workload (E = 8, 512 rows, 5120 x 8192, silu
    quantized activation): 300 live tiles, 44 of them split; every valid
    row of every expert."""
    mo = synth.moe()
    say("split moe workload", mo.mask.tolist())
    qa, sa, ga = O.quantize(np_bits(mo.x), prologue=O.PRO_SILU, mask=mo.mask.numpy())
    qbs, sbs, gbs = [], [], []
    for e in range(mo.e):
        q, s, g_ = oq(mo.w[e])
        qbs.append(q); sbs.append(s); gbs.append(g_[0])
    qb, sb, gb = np.stack(qbs), np.stack(sbs), np.array(gbs, np.float32)
    alpha = (np.float32(1.0) / (ga * gb)).astype(np.float32)
    mk = mo.mask.numpy().astype(np.int32)
    got = run_grouped(ops, qa, sa, qb, sb, alpha, mk, mo.m, mo.n, ws)
    check_grouped(got, qa, sa, qb, sb, alpha, mk, mo.m, mo.n, mo.h)


def test_split_in_graph(ops, ws):
    """The split schedule (main launch and the launch adding partials)
    captured in a HIP graph: every replay, with eager work and
    synchronisation between replays, equals the eager result bit for bit."""
    E, m, n, h = 8, 512, 5120, 2048
    mask = [238, 86, 178, 67, 107, 342, 221, 296]
    say("split grouped in a graph", (E, m, n, h), mask)
    qa, sa, qb, sb, alpha, mk = grouped_operands(E, m, n, h, mask, seed=1)
    a, b, asf, bsf = t_u8(qa), t_u8(qb), t_u8(sa), t_u8(sb)
    al, mkd = torch.from_numpy(alpha).to("cuda"), torch.from_numpy(mk).to("cuda")
    ref = ops.nvfp4_gemm_grouped_masked(a, b, asf, bsf, al, mkd, out=torch.zeros(E, m, n, dtype=torch.bfloat16,
                                                                                  device="cuda"), workspace=ws)
    out = torch.zeros(E, m, n, dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ops.nvfp4_gemm_grouped_masked(a, b, asf, bsf, al, mkd, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        ops.nvfp4_gemm_grouped_masked(a, b, asf, bsf, al, mkd, out=out, workspace=ws)
    for rep in range(3):
        out.zero_()
        ws.fill_(0x5A)   # the partials must be rewritten by every replay
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        for e in range(E):
            v = mask[e]
            assert torch.equal(out[e, :v].view(torch.int16), ref[e, :v].view(torch.int16)), f"replay {rep} expert {e}"
