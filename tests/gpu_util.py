"""Helpers shared by the GPU parity tests (not collected: no test_ prefix)."""
import sys

import numpy as np
import torch

CANARY = 0xA5


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
