"""GPU parity of the block-scaled GEMMs against the oracle.

Bar: for every compared row, max |gpu - oracle| <= 1e-2 * max |oracle row|
(bf16 output against the fp64-accumulated oracle).  Both sides consume the
same NVFP4 bytes, produced by the oracle.

Every output buffer starts filled with a bf16 NaN pattern the kernels never
write (0x7FA5).  After each call the whole buffer is checked on the device:
no element of a valid row may still hold it (so a tile that the launch never
wrote fails, wherever it is), and rows that must not be written (masked
experts) must hold nothing else.  Rows compared with the oracle: every row
up to the dense workload's 2048; for the prefill and SVDQuant workloads 512
rows stratified over the M-tiles of the launch (16 per 256-row tile, 16 per
128-row tile), each tile's first and last row included; every valid row of
every expert for the routed-expert workload.
"""
import numpy as np
import pytest
import torch

import oracle as O
from nvfp4_block_scaled_04_amd import synth
from gpu_util import (OUT_CANARY, assert_all_written, dev, np_bits, row_tolerance_check, say,
                      svdquant_lora_pieces, tile_rows)

pytestmark = pytest.mark.gpu
TOL = 1e-2


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from nvfp4_block_scaled_04_amd import ops as _ops
    return _ops


def oq(x_cpu, **kw):
    """Oracle quantization of a CPU tensor -> (fp4, sf, gs)."""
    return O.quantize(np_bits(x_cpu), **kw)


def t_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def sample_rows(m, n_samples, seed):
    if m <= n_samples:
        return np.arange(m)
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(m, n_samples - 2, replace=False).tolist()) | {0, m - 1}
    return np.array(sorted(rows))


def gemm_case(ops, a_cpu, w_cpu, bias=None, rows=None, label=""):
    m, k = a_cpu.shape
    n = w_cpu.shape[0]
    say("gemm", label, (m, n, k), "bias", bias is not None)
    qa, sa, ga = oq(a_cpu)
    qb, sb, gb = oq(w_cpu)
    alpha = np.float32(1.0) / (ga[0] * gb[0])
    out_bits = torch.full((m, n), OUT_CANARY, dtype=torch.int16, device="cuda")
    out = out_bits.view(torch.bfloat16)
    ops.nvfp4_gemm(t_u8(qa), t_u8(qb), t_u8(sa), t_u8(sb),
                   torch.tensor([alpha], dtype=torch.float32, device="cuda"),
                   bias=None if bias is None else dev(bias), out=out, k=k)
    torch.cuda.synchronize()
    assert_all_written(out_bits)
    if rows is None:
        rows = np.arange(m)
    ref = O.gemm_rows(qa, qb, sa, sb, alpha, m, n, k, rows=rows,
                      bias=None if bias is None else np_bits(bias))
    got = out.float().cpu().numpy()[rows]
    ratio = row_tolerance_check(got, ref)
    print(f"  worst row error / row max = {ratio:.3e}")
    assert ratio <= TOL
    return ratio


@pytest.mark.parametrize("m,n,k", [(1, 1, 16), (16, 33, 48), (127, 64, 128), (129, 257, 400),
                                   (200, 96, 1024), (64, 130, 80), (300, 500, 256),
                                   (16, 4096, 4096), (64, 300, 4000), (33, 17, 2064), (7, 1000, 16)])
def test_ragged_shapes(ops, m, n, k):
    g = torch.Generator().manual_seed(m * 7 + n * 3 + k)
    a = (torch.randn(m, k, generator=g) * 2).to(torch.bfloat16)
    w = (torch.randn(n, k, generator=g) * 0.02).to(torch.bfloat16)
    gemm_case(ops, a, w, label="ragged")


@pytest.mark.parametrize("shape", [(130, 70, 256), (256, 256, 384)])
def test_bias(ops, shape):
    m, n, k = shape
    g = torch.Generator().manual_seed(5)
    a = torch.randn(m, k, generator=g).to(torch.bfloat16)
    w = (torch.randn(n, k, generator=g) * 0.05).to(torch.bfloat16)
    bias = (torch.randn(n, generator=g) * 0.1).to(torch.bfloat16)
    gemm_case(ops, a, w, bias=bias, label="bias")


@pytest.mark.parametrize("m,n,k", [
    (4100, 8200, 272),   # 256x256 tiles (3-stage), ragged M and N, K % 128 != 0
    (1024, 8320, 400),   # 128x256 tiles, K % 128 != 0
    (200, 32800, 128),   # 128x256 tiles, a single partial tile row
    (3000, 4200, 144),   # 128x128 tiles (at least three per CU), ragged
    (1100, 4100, 400),   # 128x256 tiles split over two K groups, ragged M, N and K
    (640, 8000, 512),    # 128x256 tiles split over two K groups, ragged N
    (4000, 3000, 2992),  # 256x192 tiles (16 x 16: one per CU), ragged M, N and K
])
def test_tile_shapes(ops, m, n, k):
    """Each workgroup tile shape the launcher picks, with ragged edges."""
    g = torch.Generator().manual_seed(m + n + k)
    a = torch.randn(m, k, generator=g).to(torch.bfloat16)
    w = (torch.randn(n, k, generator=g) * 0.02).to(torch.bfloat16)
    rows = sample_rows(m, 160, 5) if m > 1024 else None
    if rows is not None:
        rows = np.unique(np.concatenate([rows, np.arange(m - 8, m), np.arange(250, 262)]))
    gemm_case(ops, a, w, rows=rows, label="tile shape")


def test_tiny_workload(ops):
    t = synth.tiny()
    gemm_case(ops, t.a, t.w, label="tiny fp32 workload")


def test_256x256_tile_order_every_row(ops):
    """4096 x 8192 gives 16 x 32 = 512 tiles of 256 x 256, the launch the
    prefill shape takes: the XCD remap hands each XCD 64 consecutive tiles and
    the order walks bands of 8 tile rows.  Every row is compared."""
    g = torch.Generator().manual_seed(9)
    a = torch.randn(4096, 1024, generator=g).to(torch.bfloat16)
    w = (torch.randn(8192, 1024, generator=g) * 0.02).to(torch.bfloat16)
    gemm_case(ops, a, w, label="256x256 tiles, 512 of them, every row")


def test_dense_workload(ops):
    d, a16 = synth.dense()
    gemm_case(ops, d.a, d.w, label="dense 2048x4096x4096, every row")
    gemm_case(ops, a16, d.w, label="decode 16x4096x4096")


def test_prefill_workload(ops):
    """8192 x 16384 x 5120 (32 x 64 tiles of 256 x 256): 16 rows of each of
    the 32 M-tiles, every column, and the canary check over all outputs."""
    p = synth.prefill()
    rows = tile_rows(p.m, 256, 16, 3)
    assert len(rows) == 512
    gemm_case(ops, p.a, p.w, rows=rows, label="prefill 8192x16384x5120, 512 rows over 32 M-tiles")


def test_svdquant_workload(ops):
    s = synth.svdquant()
    say("svdquant full workload")
    qa, sa, ga = oq(s.x, prologue=O.PRO_SMOOTH, pqs=np_bits(s.pqs))
    qb, sb, gb = oq(s.w)
    alpha = np.float32(1.0) / (ga[0] * gb[0])
    d, l1 = svdquant_lora_pieces(s, alpha)
    out_bits = torch.full((s.m, s.n), OUT_CANARY, dtype=torch.int16, device="cuda")
    out = out_bits.view(torch.bfloat16)
    ops.nvfp4_gemm_svdquant(t_u8(qa), t_u8(qb), t_u8(sa), t_u8(sb),
                            torch.tensor([alpha], dtype=torch.float32, device="cuda"),
                            dev(d), dev(l1), bias=dev(s.bias), out=out)
    torch.cuda.synchronize()
    assert_all_written(out_bits)
    rows = tile_rows(s.m, 128, 16, 4)   # 16 rows of every 128-row band (each 256-row tile gets 32)
    assert len(rows) == 512
    ref = O.gemm_rows(qa, qb, sa, sb, alpha, s.m, s.n, s.k, rows=rows, bias=np_bits(s.bias),
                      d=np_bits(d), l1=np_bits(l1))
    ratio = row_tolerance_check(out.float().cpu().numpy()[rows], ref)
    print(f"  worst row error / row max = {ratio:.3e}")
    assert ratio <= TOL


@pytest.mark.parametrize("r,m,n,k", [(32, 150, 90, 192), (64, 150, 90, 192), (128, 150, 90, 192),
                                     (64, 40, 200, 272),    # small M: the skinny kernel
                                     (64, 1100, 4100, 400),   # tiles split over two K groups
                                     (32, 4000, 3000, 2992)])  # 256x192 tiles, ragged M, N and K
def test_svdquant_ranks_and_ragged(ops, r, m, n, k):
    g = torch.Generator().manual_seed(r + m)
    a = torch.randn(m, k, generator=g).to(torch.bfloat16)
    w = (torch.randn(n, k, generator=g) * 0.05).to(torch.bfloat16)
    say("svdquant ragged", m, n, k, r)
    qa, sa, ga = oq(a)
    qb, sb, gb = oq(w)
    alpha = np.float32(1.0) / (ga[0] * gb[0])
    d = torch.randn(m, r, generator=g).to(torch.bfloat16)
    l1 = (torch.randn(n, r, generator=g) / float(alpha) * 1e-2).to(torch.bfloat16)
    bias = torch.randn(n, generator=g).to(torch.bfloat16)
    out = ops.nvfp4_gemm_svdquant(t_u8(qa), t_u8(qb), t_u8(sa), t_u8(sb),
                                  torch.tensor([alpha], dtype=torch.float32, device="cuda"),
                                  dev(d), dev(l1), bias=dev(bias))
    torch.cuda.synchronize()
    ref = O.gemm_rows(qa, qb, sa, sb, alpha, m, n, k, bias=np_bits(bias), d=np_bits(d),
                      l1=np_bits(l1))
    assert row_tolerance_check(out.float().cpu().numpy(), ref) <= TOL


def test_svdquant_zero_residual(ops):
    """All-zero FP4 weight: the output is alpha * d @ l1^T + bias alone."""
    g = torch.Generator().manual_seed(77)
    m, n, k, r = 64, 96, 128, 32
    a = torch.randn(m, k, generator=g).to(torch.bfloat16)
    qa, sa, _ = oq(a)
    qb = np.zeros((n, k // 2), np.uint8)
    sb = np.zeros(O.sf_size(n, k), np.uint8)
    d = torch.randn(m, r, generator=g).to(torch.bfloat16)
    l1 = torch.randn(n, r, generator=g).to(torch.bfloat16)
    bias = torch.randn(n, generator=g).to(torch.bfloat16)
    say("svdquant zero residual")
    out = ops.nvfp4_gemm_svdquant(t_u8(qa), t_u8(qb), t_u8(sa), t_u8(sb),
                                  torch.tensor([0.5], dtype=torch.float32, device="cuda"),
                                  dev(d), dev(l1), bias=dev(bias))
    torch.cuda.synchronize()
    ref = 0.5 * (d.double() @ l1.double().T) + bias.double()
    assert row_tolerance_check(out.float().cpu().numpy(), ref.numpy()) <= TOL


def grouped_case(ops, E, m, n, h, mask, rows_per_expert=None, seed=0):
    say("grouped masked", (E, m, n, h), mask)
    g = torch.Generator().manual_seed(seed)
    x = (torch.randn(E, m, h, generator=g)).to(torch.bfloat16)
    w = (torch.randn(E, n, h, generator=g) * 0.02).to(torch.bfloat16)
    mk = np.array(mask, dtype=np.int32)
    qa, sa, ga = oq(x, mask=mk)
    qb, sb, gb = oq(w)
    alpha = (np.float32(1.0) / (ga * gb)).astype(np.float32)
    out = torch.full((E, m, n), OUT_CANARY, dtype=torch.int16, device="cuda")
    ops.nvfp4_gemm_grouped_masked(t_u8(qa), t_u8(qb), t_u8(sa), t_u8(sb),
                                  torch.from_numpy(alpha).to("cuda"), torch.from_numpy(mk).to("cuda"),
                                  out=out.view(torch.bfloat16))
    torch.cuda.synchronize()
    got_all = out.cpu()
    for e in range(E):
        v = int(min(max(mk[e], 0), m))
        assert bool((got_all[e, v:] == OUT_CANARY).all()), f"expert {e}: rows >= {v} were written"
        assert not bool((got_all[e, :v] == OUT_CANARY).any()), f"expert {e}: valid rows left unwritten"
        if v == 0:
            continue
        rows = np.arange(v) if rows_per_expert is None else sample_rows(v, rows_per_expert, e)
        ref = O.gemm_rows(qa[e], qb[e], sa[e], sb[e], alpha[e], m, n, h, rows=rows)
        got = got_all[e].view(torch.bfloat16).float().numpy()[rows]
        ratio = row_tolerance_check(got, ref)
        assert ratio <= TOL, (e, ratio)


@pytest.mark.parametrize("mask", [[0, 1, 130, 256], [256, 256, 256, 256], [7, 0, 129, 64]])
def test_grouped_masked_small(ops, mask):
    grouped_case(ops, 4, 256, 96, 128, mask, seed=sum(mask))


@pytest.mark.parametrize("n,h,mask", [
    (5000, 400, [0, 1, 129, 255, 256, 300, 512, 7]),   # ragged N, K % 128 != 0
    (5120, 512, [512, 384, 100, 0, 64, 65, 511, 200]),
])
def test_grouped_masked_eight_experts(ops, n, h, mask):
    """Eight experts of 512 rows (the routed-expert launch, 128 x 256 tiles),
    masks from 0 to full: every valid row of every expert against the oracle,
    masked rows untouched."""
    grouped_case(ops, 8, 512, n, h, mask, seed=n + h)


@pytest.mark.parametrize("mask", [[0, 17, 48], [48, 48, 5]])
def test_grouped_masked_few_rows(ops, mask):
    """m <= 64 per expert: the skinny kernel, masks inside and at the edge."""
    grouped_case(ops, 3, 48, 100, 144, mask, seed=3 + sum(mask))


@pytest.mark.parametrize("m,n,k,with_bias", [(1, 1, 16, False), (7, 1000, 272, True), (16, 4096, 4096, False),
                                             (33, 130, 2064, True), (64, 300, 400, False), (100, 257, 128, True)])
def test_w4a16(ops, m, n, k, with_bias):
    """Weight-only GEMM (bf16 activation x NVFP4 weight) against the oracle:
    one or several 16-row tiles, ragged N, K % 128 != 0, bias; the 16 x 4096
    x 4096 case is the decode shape."""
    g = torch.Generator().manual_seed(m * 31 + n + k)
    a = (torch.randn(m, k, generator=g) * 2).to(torch.bfloat16)
    w = (torch.randn(n, k, generator=g) * 0.02).to(torch.bfloat16)
    bias = (torch.randn(n, generator=g) * 0.1).to(torch.bfloat16) if with_bias else None
    say("w4a16", (m, n, k), "bias", with_bias)
    qb, sb, gb = oq(w)
    alpha = np.float32(1.0) / gb[0]
    out = torch.full((m, n), OUT_CANARY, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    ops.nvfp4_gemm_w4a16(dev(a), t_u8(qb), t_u8(sb), torch.tensor([alpha], dtype=torch.float32, device="cuda"),
                         bias=None if bias is None else dev(bias), out=out)
    torch.cuda.synchronize()
    ref = O.gemm_w4a16_rows(np_bits(a), qb, sb, alpha, m, n, k,
                            bias=None if bias is None else np_bits(bias))
    got = out.float().cpu().numpy()
    ratio = row_tolerance_check(got, ref)
    print(f"  worst row error / row max = {ratio:.3e}")
    assert ratio <= TOL


def test_w4a16_reduces_to_nvfp4(ops):
    """With the activation equal to its own NVFP4 dequantization (exact in
    bf16), the weight-only GEMM and the NVFP4 x NVFP4 GEMM sum the same exact
    products; their bf16 outputs agree to accumulation-order rounding."""
    from test_oracle_gemm import dequant_torch   # decode written from the format definitions
    g = torch.Generator().manual_seed(5)
    m, n, k = 48, 384, 1024
    a = torch.randn(m, k, generator=g).to(torch.bfloat16)
    w = (torch.randn(n, k, generator=g) * 0.02).to(torch.bfloat16)
    say("w4a16 vs nvfp4", (m, n, k))
    qa, sa, ga = oq(a)
    qb, sb, gb = oq(w)
    a_dq = dequant_torch(qa, sa, m, k)
    a_dq_bf16 = a_dq.to(torch.bfloat16)
    assert torch.equal(a_dq_bf16.double(), a_dq), "dequantized values are exact in bf16"
    alpha = torch.tensor([np.float32(1.0) / gb[0]], dtype=torch.float32, device="cuda")
    o1 = ops.nvfp4_gemm_w4a16(dev(a_dq_bf16), t_u8(qb), t_u8(sb), alpha)
    o2 = ops.nvfp4_gemm(t_u8(qa), t_u8(qb), t_u8(sa), t_u8(sb), alpha, k=k)
    torch.cuda.synchronize()
    assert row_tolerance_check(o1.float().cpu().numpy(), o2.double().cpu().numpy()) <= TOL


def test_moe_workload(ops):
    mo = synth.moe()
    say("moe full workload", mo.mask.tolist())
    qa, sa, ga = O.quantize(np_bits(mo.x), prologue=O.PRO_SILU, mask=mo.mask.numpy())
    qbs, sbs, gbs = [], [], []
    for e in range(mo.e):
        q, s, g_ = oq(mo.w[e])
        qbs.append(q); sbs.append(s); gbs.append(g_[0])
    qb, sb, gb = np.stack(qbs), np.stack(sbs), np.array(gbs, np.float32)
    alpha = (np.float32(1.0) / (ga * gb)).astype(np.float32)
    out = torch.full((mo.e, mo.m, mo.n), OUT_CANARY, dtype=torch.int16, device="cuda")
    mk = mo.mask.numpy()
    ops.nvfp4_gemm_grouped_masked(t_u8(qa), t_u8(qb), t_u8(sa), t_u8(sb),
                                  torch.from_numpy(alpha).to("cuda"), dev(mo.mask),
                                  out=out.view(torch.bfloat16))
    torch.cuda.synchronize()
    got_all = out.cpu()
    for e in range(mo.e):
        v = int(mk[e])
        assert bool((got_all[e, v:] == OUT_CANARY).all()), f"expert {e}: rows >= {v} were written"
        if v == 0:
            continue
        assert not bool((got_all[e, :v] == OUT_CANARY).any()), f"expert {e}: valid rows left unwritten"
        rows = np.arange(v)   # every valid row
        ref = O.gemm_rows(qa[e], qb[e], sa[e], sb[e], alpha[e], mo.m, mo.n, mo.h, rows=rows)
        got = got_all[e].view(torch.bfloat16).float().numpy()[rows]
        assert row_tolerance_check(got, ref) <= TOL, e


def test_end_to_end_dynamic_pipeline(ops):
    """The bench's step: dynamic activation quantize, alpha on the device,
    GEMM; compared with the oracle's own quantize + GEMM."""
    d, _ = synth.dense(m=512, n=1024, k=2048)
    say("pipeline", (d.m, d.n, d.k))
    qb, sb, gb = oq(d.w)
    x = dev(d.a)
    fa, sfa, gsa = ops.nvfp4_quantize(x)
    gsb = torch.from_numpy(gb).to("cuda")
    alpha = ops.nvfp4_alpha(gsa, gsb)
    out = ops.nvfp4_gemm(fa, t_u8(qb), sfa, t_u8(sb), alpha)
    torch.cuda.synchronize()
    qa, sa, ga = oq(d.a)
    ref_alpha = np.float32(1.0) / (ga[0] * gb[0])
    assert np_bits(alpha).view(np.uint32)[0] == np.array([ref_alpha]).view(np.uint32)[0]
    rows = sample_rows(d.m, 64, 9)
    ref = O.gemm_rows(qa, qb, sa, sb, ref_alpha, d.m, d.n, d.k, rows=rows)
    assert row_tolerance_check(out.float().cpu().numpy()[rows], ref) <= TOL


def test_every_scale_code_k16(ops):
    """K = 16 (one block): out[m, n] = alpha * dec(sa[m]) * dec(sb[n]) *
    sum_j e2m1(a) e2m1(b), so every output element depends on one pair of
    scale codes.  Rows and columns walk all 127 finite ue4m3 codes, including
    the subnormals, and each element is compared on its own (relative 2^-7,
    one bf16 ulp: the two sides may round alpha * acc differently before the
    bf16 rounding), so a code decoded wrongly anywhere in the staging -- off
    by at least one e4m3 step, 1/8 -- fails here even where the row tolerance
    would hide it."""
    m = n = 254
    k = 16
    rng = np.random.default_rng(11)
    qa = rng.integers(0, 256, size=(m, k // 2), dtype=np.uint8)
    qb = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    sa = np.zeros(O.sf_size(m, k), np.uint8)
    sb = np.zeros(O.sf_size(n, k), np.uint8)
    for r in range(m):
        sa[O.sf_offset(r, 0, k)] = r % 127
    for r in range(n):
        sb[O.sf_offset(r, 0, k)] = (r * 5 + 3) % 127
    alpha = np.float32(0.75)
    say("every scale code, k=16", (m, n, k))
    out = ops.nvfp4_gemm(t_u8(qa), t_u8(qb), t_u8(sa), t_u8(sb),
                         torch.tensor([alpha], dtype=torch.float32, device="cuda"), k=k)
    torch.cuda.synchronize()
    ref = O.gemm_rows(qa, qb, sa, sb, alpha, m, n, k)
    got = out.float().cpu().numpy()
    err = np.abs(got - ref)
    assert np.all(err <= np.abs(ref) * 2.0 ** -7), float((err / np.maximum(np.abs(ref), 1e-30)).max())
