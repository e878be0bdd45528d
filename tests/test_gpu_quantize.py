"""GPU parity of the quantizers against the oracle: FP4 bytes, scale bytes
and global scales must be bit-identical.  Outputs start filled with a canary
byte so that unwritten padding and masked rows are caught.

In DYNAMIC mode, items of at most 65536 elements (32768 with the silu
prologue) are quantized in one launch (each workgroup of the tiled pass
recomputes the item's amax); larger ones take the amax pass, the finish and
the quantize pass.  The cases below cover each prologue and masking form on
both sides of that line."""
import numpy as np
import pytest
import torch

import oracle as O
from nvfp4_block_scaled_04_amd import synth
from gpu_util import CANARY, canary, dev, np_bits, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from nvfp4_block_scaled_04_amd import ops as _ops
    return _ops


def run_single(ops, x_cpu, mode, gs=None, pqs=None):
    """Quantize [m,k] on the GPU and with the oracle; compare everything."""
    m, k = x_cpu.shape
    say("quantize", tuple(x_cpu.shape), x_cpu.dtype, "mode", mode, "pqs", pqs is not None)
    x = dev(x_cpu)
    gs_d = torch.tensor([0.0 if gs is None else gs], dtype=torch.float32, device="cuda")
    o4 = canary((m, k // 2))
    osf = canary((ops.sf_size(m, k),))
    pq_d = None if pqs is None else dev(pqs)
    ops.nvfp4_quantize(x, gs_d, mode, pre_quant_scale=pq_d, out_fp4=o4, out_sf=osf)
    torch.cuda.synchronize()
    xin = np_bits(x_cpu)
    q, sf, g = O.quantize(xin, prologue=O.PRO_SMOOTH if pqs is not None else O.PRO_NONE,
                          pqs=None if pqs is None else np_bits(pqs),
                          gs=None if gs is None else np.array([gs], np.float32),
                          gs_mode=mode)
    assert np.array_equal(np_bits(gs_d).view(np.uint32), g.view(np.uint32)), (np_bits(gs_d), g)
    gq, gsf = np_bits(o4), np_bits(osf)
    bad = np.argwhere(gq != q)
    assert len(bad) == 0, f"{len(bad)} FP4 bytes differ, first at {bad[:3].tolist()}"
    bad = np.argwhere(gsf != sf)
    assert len(bad) == 0, f"{len(bad)} scale bytes differ, first at {bad[:3].tolist()}"
    return o4, osf, gs_d


# ---- single tensor -------------------------------------------------------------

@pytest.mark.parametrize("m,k", [(1, 16), (16, 64), (127, 48), (129, 80), (128, 256), (300, 1040),
                                 (257, 4096),
                                 (8200, 4112)])   # wide quantize tiles (4 swizzle tiles), ragged both ways
def test_bf16_dynamic_ragged(ops, m, k):
    g = torch.Generator().manual_seed(m * 1000 + k)
    x = (torch.randn(m, k, generator=g) * 3).to(torch.bfloat16)
    run_single(ops, x, ops.GS_DYNAMIC)


@pytest.mark.parametrize("gs", [384.0, 1.0, 1e-3, 7.25e4])
@pytest.mark.parametrize("m,k", [(200, 320), (600, 1024)])
def test_bf16_static(ops, gs, m, k):
    g = torch.Generator().manual_seed(7)
    x = torch.randn(m, k, generator=g).to(torch.bfloat16)
    run_single(ops, x, ops.GS_STATIC, gs=gs)


def test_fp32_dynamic_tiled(ops):
    g = torch.Generator().manual_seed(8)
    x = torch.randn(300, 1040, generator=g) * 5
    run_single(ops, x, ops.GS_DYNAMIC)


def test_tiny_workload_fp32(ops):
    t = synth.tiny()
    run_single(ops, t.a, ops.GS_DYNAMIC)
    run_single(ops, t.w, ops.GS_DYNAMIC)


def test_worked_example(ops):
    x = torch.tensor([[7, -3.5, 1.75, 0.875, 0.4375, 0.21875, 0, -7, 5, 2.5, 1.25, 0.625, 3, -1.5,
                       0.75, -0.1, 0.3, -0.15, 0.05, 0.1, 0.2, -0.3, 0.0, 0.01, 0.075, -0.025, 0.125,
                       0.28, -0.2, 0.06, 0.03, -0.0]], dtype=torch.float32)
    o4, osf, gs = run_single(ops, x, ops.GS_DYNAMIC)
    assert bytes(np_bits(o4)[0]) == bytes.fromhex("D723 01F0 4612 B581 D742 F600 9374 2E81".replace(" ", ""))


@pytest.mark.parametrize("m,k", [(64, 128), (640, 256)])
def test_nonfinite_and_denormal_inputs(ops, m, k):
    g = torch.Generator().manual_seed(3)
    x = torch.randn(m, k, generator=g)
    x[0, 5] = float("nan")
    x[1, 17] = float("inf")
    x[2, 33] = float("-inf")
    x[3, :16] = 1e-40            # fp32 denormals
    x[4, 16:32] = -0.0
    x[5, :] = 0.0
    run_single(ops, x.clone(), ops.GS_DYNAMIC)
    xb = x.to(torch.bfloat16)
    xb[6, 40] = float("nan")
    run_single(ops, xb, ops.GS_DYNAMIC)
    # without the non-finite values: denormal and zero rows only
    x2 = torch.randn(m, k, generator=g) * 1e-38
    run_single(ops, x2.to(torch.bfloat16), ops.GS_DYNAMIC)


@pytest.mark.parametrize("m", [100, 300])
def test_smooth_prologue(ops, m):
    s = synth.svdquant(m=m, n=64, k=320)
    run_single(ops, s.x, ops.GS_DYNAMIC, pqs=s.pqs)
    run_single(ops, s.x.float(), ops.GS_DYNAMIC, pqs=s.pqs)


def test_repeat_is_identical(ops):
    g = torch.Generator().manual_seed(11)
    x = dev(torch.randn(1024, 2048, generator=g).to(torch.bfloat16))
    say("repeat identity")
    a = ops.nvfp4_quantize(x)
    b = ops.nvfp4_quantize(x)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def lora_fragments(split, r, k):
    """The oracle's split weight [2, r, k] laid out as the prepared weight
    the header describes: fragment (h, t, s) of 64 lanes x 8 elements, lane l
    holding rank 16 t + l % 16 at columns 32 s + 8 (l / 16) .. + 7, zero
    past k."""
    ns = (k + 31) // 32
    pad = np.zeros((2, r, ns * 32), dtype=np.uint16)
    pad[:, :, :k] = split
    out = np.zeros((2, r // 16, ns, 64, 8), dtype=np.uint16)
    for lane in range(64):
        ranks = np.arange(r // 16) * 16 + lane % 16
        for sl in range(ns):
            c0 = 32 * sl + 8 * (lane // 16)
            out[:, :, sl, lane, :] = pad[:, ranks, c0:c0 + 8]
    return out.ravel()


@pytest.mark.parametrize("m,k,r,dynamic", [(4096, 3072, 32, False), (100, 400, 64, True), (17, 272, 32, True),
                                          (300, 4096, 128, True), (130, 96, 96, False),
                                          (200, 8192, 32, True),     # K past the old 4096 limit: 8 chunks
                                          (130, 5136, 64, False),    # 5 chunks and one block
                                          (64, 1024, 96, True), (40, 1040, 128, False)])
@pytest.mark.parametrize("prepared", [False, True])
def test_quantize_lora_down(ops, m, k, r, dynamic, prepared):
    """Smooth quantize with the LoRA-down projection fused: the FP4 and scale
    bytes and gs must equal the oracle's smooth quantization exactly, and
    d = (x * pqs) @ L2^T must meet the GEMM bar against the oracle's fp64
    projection (every product is exact in the kernel; only fp32 accumulation
    and the bf16 output round).  The first case is the SVDQuant workload's
    activation.  prepared: through nvfp4_quantize_lora_down_prepared, with
    the weight from nvfp4_lora_down_prepare (bit-exact against the oracle's
    split)."""
    from gpu_util import row_tolerance_check
    s = synth.svdquant(m=m, n=64, k=k, r=r)
    l2 = s.l2.to(torch.bfloat16)
    say("quantize + lora-down", (m, k, r), "dynamic", dynamic, "prepared", prepared)
    mode = ops.GS_DYNAMIC if dynamic else ops.GS_STATIC
    gs_static = None if dynamic else np.float32(2688.0 / 7.5)
    gs_d = torch.tensor([0.0 if gs_static is None else gs_static], dtype=torch.float32, device="cuda")
    o4 = canary((m, k // 2))
    osf = canary((ops.sf_size(m, k),))
    d = torch.full((m, r), 0x7FA5, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    if prepared:
        w = torch.full((ops.lora_prepared_numel(r, k),), 0x7FA5, dtype=torch.int16,
                       device="cuda").view(torch.bfloat16)
        ops.nvfp4_lora_down_prepare(dev(s.pqs), dev(l2), out=w)
        torch.cuda.synchronize()
        ref_w = lora_fragments(O.lora_weight_split(np_bits(s.pqs), np_bits(l2)), r, k)
        bad = np.argwhere(np_bits(w) != ref_w)
        assert len(bad) == 0, f"{len(bad)} prepared weight elements differ, first at {bad[:3].tolist()}"
        ops.nvfp4_quantize_lora_down_prepared(dev(s.x), dev(s.pqs), w, r, gs_d, mode, out_fp4=o4, out_sf=osf,
                                              d=d)
    else:
        ops.nvfp4_quantize_lora_down(dev(s.x), dev(s.pqs), dev(l2), gs_d, mode, out_fp4=o4, out_sf=osf, d=d)
    torch.cuda.synchronize()
    q, sf, g = O.quantize(np_bits(s.x), prologue=O.PRO_SMOOTH, pqs=np_bits(s.pqs),
                          gs=None if gs_static is None else np.array([gs_static], np.float32), gs_mode=mode)
    assert np.array_equal(np_bits(gs_d).view(np.uint32), g.view(np.uint32)), (np_bits(gs_d), g)
    bad = np.argwhere(np_bits(o4) != q)
    assert len(bad) == 0, f"{len(bad)} FP4 bytes differ, first at {bad[:3].tolist()}"
    bad = np.argwhere(np_bits(osf) != sf)
    assert len(bad) == 0, f"{len(bad)} scale bytes differ, first at {bad[:3].tolist()}"
    ref = O.lora_down(np_bits(s.x), np_bits(s.pqs), np_bits(l2))
    ratio = row_tolerance_check(d.float().cpu().numpy(), ref)
    print(f"  d: worst row error / row max = {ratio:.3e}")
    assert ratio <= 1e-2


# ---- batched / masked / silu -------------------------------------------------------

def run_batched(ops, x_cpu, mask, mode, silu=False, gs=None, ws=False):
    """ws: through the *_ws entry point, with a workspace of stale bytes and a
    gs_other, so that alpha is checked too; ws == "h": the silu workspace
    with room for h (silu evaluated once, by the amax pass)."""
    b, m, kin = x_cpu.shape
    K = kin // 2 if silu else kin
    say("batched", tuple(x_cpu.shape), "silu", silu, "mask", None if mask is None else mask.tolist(),
        "mode", mode, "ws", ws)
    x = dev(x_cpu)
    mk = None if mask is None else dev(mask)
    gs_d = torch.zeros(b, dtype=torch.float32, device="cuda") if gs is None else dev(gs.clone())
    o4 = canary((b, m, K // 2))
    osf = canary((b, ops.sf_size(m, K)))
    if ws:
        mkws = ops.silu_workspace if ws == "h" else ops.batched_workspace
        w = mkws(b, m, K, "cuda").fill_(0x5A)
        go = (torch.rand(b, generator=torch.Generator().manual_seed(b + m + K)) * 500 + 1).to(torch.float32)
        al = torch.full((b,), float("nan"), dtype=torch.float32, device="cuda")
        fn = ops.silu_mul_nvfp4_quantize_ws if silu else ops.nvfp4_quantize_masked_batched_ws
        fn(x, w, mk, gs_d, mode, gs_other=dev(go), alpha=al, out_fp4=o4, out_sf=osf)
    elif silu:
        ops.silu_mul_nvfp4_quantize(x, mk, gs_d, mode, out_fp4=o4, out_sf=osf)
    else:
        ops.nvfp4_quantize_masked_batched(x, mk, gs_d, mode, out_fp4=o4, out_sf=osf)
    torch.cuda.synchronize()
    fill = np.full((b, m, K // 2), CANARY, dtype=np.uint8)
    q, sf, g = O.quantize(np_bits(x_cpu), prologue=O.PRO_SILU if silu else O.PRO_NONE,
                          mask=None if mask is None else mask.numpy(),
                          gs=None if gs is None else gs.numpy(), gs_mode=mode, out_fp4=fill)
    assert np.array_equal(np_bits(gs_d).view(np.uint32), g.view(np.uint32)), (np_bits(gs_d), g)
    if ws:
        want = (np.float32(1.0) / (g.astype(np.float32) * go.numpy())).astype(np.float32)
        assert np.array_equal(np_bits(al).view(np.uint32), want.view(np.uint32)), (np_bits(al), want)
    gq, gsf = np_bits(o4), np_bits(osf)
    bad = np.argwhere(gq != q)
    assert len(bad) == 0, f"{len(bad)} FP4 bytes differ, first at {bad[:3].tolist()}"
    bad = np.argwhere(gsf != sf)
    assert len(bad) == 0, f"{len(bad)} scale bytes differ, first at {bad[:3].tolist()}"


@pytest.mark.parametrize("silu", [False, True])
@pytest.mark.parametrize("mask,k", [(None, 512), ([0, 1, 129, 200], 512), ([200, 0, 7, 130], 2048),
                                    ([5, 0, 0, 77], 96), ([0, 0, 0, 0], 512)])
def test_batched_ws(ops, silu, mask, k):
    """The *_ws batched forms: the quantize pass reduces each item's partial
    maxima from the workspace (two launches; the small items' one-launch path
    too) and writes alpha; bytes, gs and alpha equal the oracle's."""
    g = torch.Generator().manual_seed(41 + k)
    x = (torch.randn(4, 200, 2 * k if silu else k, generator=g) *
         torch.tensor([1.0, 10.0, 0.1, 3.0])[:, None, None])
    mk = None if mask is None else torch.tensor(mask, dtype=torch.int32)
    run_batched(ops, x.to(torch.bfloat16), mk, ops.GS_DYNAMIC, silu=silu, ws=True)


@pytest.mark.parametrize("mask,k", [(None, 512), ([0, 1, 129, 200], 512), ([200, 0, 7, 130], 2048),
                                    ([0, 0, 0, 0], 512), ([200, 200, 200, 200], 1040)])
def test_silu_ws_h(ops, mask, k):
    """silu_mul_nvfp4_quantize_ws with room for h: the amax pass stores h =
    bf16(silu(g) * u) of the valid rows and the quantize pass reads it back
    as a bf16 input; the workspace starts as stale bytes, so a row the amax
    pass did not store and the quantize pass read would show.  Bytes, gs and
    alpha equal the oracle's."""
    g = torch.Generator().manual_seed(43 + k)
    x = (torch.randn(4, 200, 2 * k, generator=g) * torch.tensor([1.0, 10.0, 0.1, 3.0])[:, None, None])
    mk = None if mask is None else torch.tensor(mask, dtype=torch.int32)
    run_batched(ops, x.to(torch.bfloat16), mk, ops.GS_DYNAMIC, silu=True, ws="h")


def test_silu_ws_size_boundary(ops):
    """A workspace one byte short of NVFP4_SILU_WS_BYTES takes the path that
    evaluates silu in both passes; exactly that size keeps h.  Both give the
    same bytes, gs and alpha."""
    g = torch.Generator().manual_seed(47)
    b, m, k = 3, 300, 512
    x = dev(torch.randn(b, m, 2 * k, generator=g).to(torch.bfloat16))
    mk = dev(torch.tensor([300, 17, 129], dtype=torch.int32))
    go = dev((torch.rand(b, generator=g) * 100 + 1).to(torch.float32))
    say("silu ws size boundary", (b, m, k))
    outs = []
    for nbytes in (ops.silu_ws_bytes(b, m, k) - 1, ops.silu_ws_bytes(b, m, k)):
        w = torch.full((nbytes,), 0x5A, dtype=torch.uint8, device="cuda")
        o4 = canary((b, m, k // 2))
        osf = canary((b, ops.sf_size(m, k)))
        r = ops.silu_mul_nvfp4_quantize_ws(x, w, mk, None, ops.GS_DYNAMIC, gs_other=go, out_fp4=o4, out_sf=osf)
        torch.cuda.synchronize()
        outs.append([t.clone() for t in r])
    for u, v in zip(*outs):
        assert torch.equal(u.view(torch.uint8), v.view(torch.uint8))


def test_batched_ws_static(ops):
    g = torch.Generator().manual_seed(42)
    x = torch.randn(3, 130, 768, generator=g).to(torch.bfloat16)
    run_batched(ops, x, torch.tensor([130, 64, 1], dtype=torch.int32), ops.GS_STATIC,
                gs=torch.tensor([100.0, 250.0, 3.0]), ws=True)


@pytest.mark.parametrize("ws", [True, "h"])
def test_moe_workload_ws(ops, ws):
    mo = synth.moe(h=8192, n=64)
    run_batched(ops, mo.x, mo.mask, ops.GS_DYNAMIC, silu=True, ws=ws)


@pytest.mark.parametrize("mask", [None, [0, 1, 129, 200], [200, 200, 200, 200], [5, 0, 0, 77]])
@pytest.mark.parametrize("k", [96, 512])
def test_masked_batched(ops, mask, k):
    g = torch.Generator().manual_seed(21)
    x = (torch.randn(4, 200, k, generator=g) * torch.tensor([1.0, 10.0, 0.1, 3.0])[:, None, None])
    mk = None if mask is None else torch.tensor(mask, dtype=torch.int32)
    run_batched(ops, x.to(torch.bfloat16), mk, ops.GS_DYNAMIC)


@pytest.mark.parametrize("k", [64, 768])
def test_masked_batched_static(ops, k):
    g = torch.Generator().manual_seed(22)
    x = torch.randn(3, 130, k, generator=g).to(torch.bfloat16)
    run_batched(ops, x, torch.tensor([130, 64, 1], dtype=torch.int32), ops.GS_STATIC,
                gs=torch.tensor([100.0, 250.0, 3.0]))


def test_mask_out_of_range_is_clamped(ops):
    g = torch.Generator().manual_seed(23)
    x = torch.randn(2, 40, 32, generator=g).to(torch.bfloat16)
    run_batched(ops, x, torch.tensor([-5, 1000], dtype=torch.int32), ops.GS_DYNAMIC)


@pytest.mark.parametrize("mask", [[64, 0, 17], [1, 64, 33]])
@pytest.mark.parametrize("h", [96, 1024])
def test_silu_masked(ops, mask, h):
    g = torch.Generator().manual_seed(31)
    x = (torch.randn(3, 64, 2 * h, generator=g) * 2).to(torch.bfloat16)
    run_batched(ops, x, torch.tensor(mask, dtype=torch.int32), ops.GS_DYNAMIC, silu=True)


def test_silu_every_bf16_gate(ops):
    """Every bf16 gate value g (65536 codes, NaN/inf included) paired with
    three up values; one item per (g, u) so that the DYNAMIC global scale of
    the item exposes |h| = |bf16(silu(g)*u)| exactly, and the bytes are
    compared as well."""
    codes = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    gate = codes.view(torch.bfloat16)
    for u in (1.0, -1.375, 0.0078125 * 3.1):
        ub = torch.tensor(u).to(torch.bfloat16)
        for half in range(2):   # items per call stay below the 65535 grid limit
            x = torch.empty(32768, 1, 32, dtype=torch.bfloat16)
            x[:, 0, :16] = gate[half * 32768:(half + 1) * 32768, None]
            x[:, 0, 16:] = ub
            run_batched(ops, x, None, ops.GS_DYNAMIC, silu=True)


@pytest.mark.parametrize("b,m,h", [(16, 128, 512), (16, 64, 256)])
def test_silu_random_pairs(ops, b, m, h):
    """Up to one million (gate, up) pairs: gates uniform over the finite bf16
    bit patterns (every binade), up values N(0,1) times random powers of two.
    The kernel decides most products of silu(g) and u on a fast fp32 path
    and only the ones next to a bf16 rounding boundary exactly; every byte
    must still equal the oracle's."""
    rng = np.random.default_rng(2024 + m)
    bits = rng.integers(0, 65536, size=(b, m, h), dtype=np.uint32).astype(np.uint16)
    finite = (bits & 0x7F80) != 0x7F80
    bits = np.where(finite, bits, bits & 0x807F)   # non-finite patterns -> small values
    gate = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    up = torch.from_numpy(rng.standard_normal((b, m, h)).astype(np.float32) *
                          np.exp2(rng.integers(-20, 21, size=(b, m, h))).astype(np.float32)).to(torch.bfloat16)
    x = torch.cat([gate, up], dim=-1).contiguous()
    run_batched(ops, x, None, ops.GS_DYNAMIC, silu=True)


# ---- workload sizes ------------------------------------------------------------

def test_dense_workload_full(ops):
    d, a16 = synth.dense()
    run_single(ops, d.a, ops.GS_DYNAMIC)
    run_single(ops, d.w, ops.GS_DYNAMIC)
    run_single(ops, a16, ops.GS_DYNAMIC)


def test_prefill_workload_full(ops):
    p = synth.prefill()
    run_single(ops, p.a, ops.GS_DYNAMIC)
    run_single(ops, p.w, ops.GS_DYNAMIC)


def test_svdquant_workload_full(ops):
    s = synth.svdquant()
    run_single(ops, s.x, ops.GS_DYNAMIC, pqs=s.pqs)
    run_single(ops, s.w, ops.GS_DYNAMIC)


def test_moe_workload_full(ops):
    mo = synth.moe(h=8192, n=64)   # the down-proj weights are exercised in the GEMM tests
    run_batched(ops, mo.x, mo.mask, ops.GS_DYNAMIC, silu=True)


@pytest.mark.parametrize("m,k,dtype,dynamic,smooth", [
    (16, 4096, torch.bfloat16, True, False),     # one-launch dynamic path
    (37, 96, torch.float32, True, True),         # one-launch, fp32 input, smooth prologue
    (1024, 4096, torch.bfloat16, True, False),   # amax, finish, quantize pass
    (300, 512, torch.bfloat16, False, True),     # static gs
])
def test_quantize_alpha(ops, m, k, dtype, dynamic, smooth):
    """nvfp4_quantize_alpha writes the bytes nvfp4_quantize writes, and alpha =
    1 / (gs * gs_other) bit for bit as nvfp4_alpha and fp32 arithmetic give it."""
    say("quantize_alpha", (m, k), dtype, "dynamic" if dynamic else "static", "smooth" if smooth else "")
    g = torch.Generator().manual_seed(m + k)
    x = (torch.randn(m, k, generator=g) * 3).to(dtype).cuda()
    pqs = torch.exp(0.3 * torch.randn(k, generator=g)).to(torch.bfloat16).cuda() if smooth else None
    mode = ops.GS_DYNAMIC if dynamic else ops.GS_STATIC
    gs0 = torch.full((1,), 2688.0 / 11.0, dtype=torch.float32, device="cuda")
    gs_w = torch.full((1,), 2688.0 / 0.137, dtype=torch.float32, device="cuda")
    q1, sf1, gs1 = ops.nvfp4_quantize(x, gs0.clone(), mode, pre_quant_scale=pqs)
    q2, sf2, gs2, alpha = ops.nvfp4_quantize_alpha(x, gs_w, gs0.clone(), mode, pre_quant_scale=pqs)
    want = ops.nvfp4_alpha(gs2, gs_w)
    torch.cuda.synchronize()
    assert torch.equal(q1, q2) and torch.equal(sf1, sf2)
    assert np_bits(gs1).view(np.uint32)[0] == np_bits(gs2).view(np.uint32)[0]
    a = np_bits(alpha).view(np.uint32)[0]
    assert a == np_bits(want).view(np.uint32)[0]
    host = np.float32(1.0) / (np_bits(gs2)[0] * np_bits(gs_w)[0])
    assert a == np.array([host], dtype=np.float32).view(np.uint32)[0]


def _nonfinite(x):
    x[0, 5] = float("nan")
    x[1, 17] = float("inf")
    x[2, 33] = float("-inf")
    x[4, 16:32] = -0.0
    return x


@pytest.mark.parametrize("m,k,dtype,case", [
    (640, 256, torch.float32, "nonfinite"),
    (640, 256, torch.bfloat16, "nonfinite"),
    (300, 1040, torch.bfloat16, "plain"),
    (8200, 4112, torch.bfloat16, "plain"),      # ragged both ways, more than one amax chunk per workgroup
    (300, 320, torch.bfloat16, "smooth"),
    (300, 320, torch.float32, "smooth"),
    (16, 4096, torch.bfloat16, "plain"),        # small: the one-launch path (workspace unused)
    (300, 512, torch.bfloat16, "static"),
])
def test_quantize_ws(ops, m, k, dtype, case):
    """nvfp4_quantize_ws: the partial maxima in the caller's workspace (filled
    with a NaN pattern beforehand), the quantize pass reducing them itself.
    FP4 and scale bytes and gs equal to the oracle's, alpha = 1 / (gs *
    gs_other) bit for bit; the same bytes without alpha."""
    say("quantize_ws", (m, k), dtype, case)
    g = torch.Generator().manual_seed(m * 3 + k)
    x = torch.randn(m, k, generator=g) * 3
    if case == "nonfinite":
        x = _nonfinite(x)
    x = x.to(dtype)
    pqs = torch.exp(0.4 * torch.randn(k, generator=g)).to(torch.bfloat16) if case == "smooth" else None
    static = case == "static"
    mode = ops.GS_STATIC if static else ops.GS_DYNAMIC
    gs_in = 2688.0 / 9.5
    ws = torch.full((ops.QUANTIZE_WS_BYTES,), 0xFF, dtype=torch.uint8, device="cuda")
    gs_w = torch.full((1,), 2688.0 / 0.137, dtype=torch.float32, device="cuda")
    o4, osf = canary((m, k // 2)), canary((ops.sf_size(m, k),))
    gs_d = torch.tensor([gs_in], dtype=torch.float32, device="cuda")
    _, _, _, alpha = ops.nvfp4_quantize_ws(dev(x), ws, gs_d, mode, pre_quant_scale=None if pqs is None else dev(pqs),
                                           gs_other=gs_w, out_fp4=o4, out_sf=osf)
    o4b, osfb = canary((m, k // 2)), canary((ops.sf_size(m, k),))
    gs_b = torch.tensor([gs_in], dtype=torch.float32, device="cuda")
    ops.nvfp4_quantize_ws(dev(x), ws, gs_b, mode, pre_quant_scale=None if pqs is None else dev(pqs),
                          out_fp4=o4b, out_sf=osfb)
    torch.cuda.synchronize()
    q, sf, gsv = O.quantize(np_bits(x), prologue=O.PRO_SMOOTH if pqs is not None else O.PRO_NONE,
                            pqs=None if pqs is None else np_bits(pqs),
                            gs=np.array([gs_in], np.float32) if static else None,
                            gs_mode=O.STATIC if static else O.DYNAMIC)
    for a4, asf, ag in ((o4, osf, gs_d), (o4b, osfb, gs_b)):
        assert np_bits(ag).view(np.uint32)[0] == gsv.view(np.uint32)[0]
        assert np.array_equal(np_bits(a4), q), int((np_bits(a4) != q).sum())
        assert np.array_equal(np_bits(asf), sf), int((np_bits(asf) != sf).sum())
    want = np.float32(1.0) / (gsv[0] * np_bits(gs_w)[0])
    assert np_bits(alpha).view(np.uint32)[0] == np.array([want], np.float32).view(np.uint32)[0]


def test_quantize_ws_prefill_and_reuse(ops):
    """The prefill activation through the workspace path, then a smaller
    tensor through the same workspace: both bit-exact with the oracle."""
    p = synth.prefill()
    ws = torch.full((ops.QUANTIZE_WS_BYTES,), 0xFF, dtype=torch.uint8, device="cuda")
    for x in (p.a, p.a[:1000, :2048].contiguous()):
        m, k = x.shape
        say("quantize_ws reuse", (m, k))
        o4, osf = canary((m, k // 2)), canary((ops.sf_size(m, k),))
        _, _, gs, _ = ops.nvfp4_quantize_ws(dev(x), ws, out_fp4=o4, out_sf=osf)
        torch.cuda.synchronize()
        q, sf, gv = O.quantize(np_bits(x))
        assert np_bits(gs).view(np.uint32)[0] == gv.view(np.uint32)[0]
        assert np.array_equal(np_bits(o4), q)
        assert np.array_equal(np_bits(osf), sf)
