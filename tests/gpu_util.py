"""Helpers shared by the GPU parity tests (not collected: no test_ prefix)."""
import sys

import numpy as np
import torch

CANARY = 0xA5
OUT_CANARY = 0x7FA5  # a bf16 NaN pattern the GEMM kernels never write


def say(*a):
    """Name the case before the GPU step runs (flushed, so a fault still
    leaves the case in the log)."""
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def dev(t):
    return t.contiguous().to("cuda")


def np_bits(t):
    """numpy raw bits of a CPU or device tensor."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def canary(shape, device="cuda"):
    return torch.full(shape, CANARY, dtype=torch.uint8, device=device)


def bf16_from_bits(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)


def row_tolerance_check(gpu, ref, tol=1e-2):
    """Acceptance bar for the GEMM: for every row, max |gpu - oracle| <=
    tol * max |oracle row|.  Returns the worst ratio."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(gpu - ref).max(axis=-1)
    scale = np.abs(ref).max(axis=-1)
    scale = np.where(scale == 0, 1.0, scale)
    ratio = err / scale
    return float(ratio.max())


def assert_all_written(out_bits):
    """No element of an (all valid) GEMM output may still hold OUT_CANARY;
    out_bits is the output viewed as int16, checked on its device."""
    left = int((out_bits == OUT_CANARY).sum().item())
    if left:
        idx = torch.nonzero(out_bits == OUT_CANARY)[:4].tolist()
        raise AssertionError(f"{left} outputs never written, first at {idx}")


def tile_rows(m, bm, per_tile, seed):
    """Rows stratified over the M-tiles of height bm: per tile its first and
    last row and per_tile - 2 others drawn from a seeded generator."""
    rng = np.random.default_rng(seed)
    rows = []
    for t0 in range(0, m, bm):
        t1 = min(m, t0 + bm)
        inner = np.arange(t0 + 1, t1 - 1)
        k = min(len(inner), per_tile - 2)
        rows += [t0, t1 - 1] + (rng.choice(inner, k, replace=False).tolist() if k > 0 else [])
    return np.array(sorted(set(rows)))


def svdquant_lora_pieces(s, alpha):
    """The caller-side pieces of the SVDQuant GEMM for a synth.svdquant()
    draw (flashinfer mm_nvfp4_svdquant puts them on the caller):
    d = bf16((x * pqs) @ L2^T), the LoRA-down output (plain torch CPU fp32
    matmul, then bf16), and l1 = bf16(l1_raw / alpha), the LoRA-up weight
    with 1/alpha folded in so that the epilogue's alpha * acc restores it."""
    xs = s.x.float() * s.pqs.float()
    d = (xs @ s.l2.t()).to(torch.bfloat16)
    l1 = (s.l1_raw / float(alpha)).to(torch.bfloat16)
    return d, l1
