"""Seeded synthetic inputs shaped like the workloads on the pages.

This module holds no arithmetic of the method (no scale, no encoding, no
GEMM): it only draws random tensors with torch's CPU generator and casts them
to bf16 with torch's own round-to-nearest-even.  Tests, the bench and the
smoke check use it to feed both the oracle and the HIP path the same bytes.

Workloads (their sizes follow the pages' use cases; the values are synthetic,
no dataset or checkpoint is involved):
  * tiny      -- fp32 A[128,256], B[256,256] ~ N(0,1), 4 A columns x50.
  * dense     -- NVFP4 linear: bf16 A[2048,4096] ~ N(0,1) with 1% of channels
                 x20, weight [4096,4096] ~ N(0,0.02); decode variant M=16.
  * moe       -- Llama4-style routed experts: E=8, gate|up [512,16384] bf16,
                 valid rows per expert uniform in [0,512], down-proj weight
                 [8,5120,8192] ~ N(0,0.02).
  * moe_swiglu -- the same experts one step earlier: hidden states
                 [8,512,5120] bf16 ~ N(0,1) against gate|up weights
                 [8,16384,5120] ~ N(0,0.02) (gate rows, then up rows), valid
                 rows per expert uniform in [0,512].
  * svdquant  -- video-diffusion linear: bf16 X[4096,3072], pre_quant_scale
                 lognormal(0,0.5), weight [3072,3072], rank-32 LoRA pieces,
                 bias [3072].
  * prefill   -- bf16 A[8192,5120] with 0.5% outlier channels x30, weight
                 [16384,5120] (fused gate+up).
Outlier channels stand in for the activation outliers that motivate
pre_quant_scale smoothing on the pages.
"""
from dataclasses import dataclass

import torch


def _gen(seed):
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return g


def _bf16(t):
    return t.to(torch.bfloat16)


def _outlier_cols(k, frac, g):
    n = int(round(frac * k))
    return torch.randperm(k, generator=g)[:n]


@dataclass
class Dense:
    a: torch.Tensor          # [M, K] bf16 (or fp32 for the tiny case)
    w: torch.Tensor          # [N, K] bf16 (or fp32)
    m: int
    n: int
    k: int


def tiny(seed=0, m=128, n=256, k=256, n_outliers=4, scale=50.0):
    """fp32 activation and weight, N(0,1); n_outliers A columns scaled."""
    g = _gen(seed)
    a = torch.randn(m, k, generator=g, dtype=torch.float32)
    w = torch.randn(n, k, generator=g, dtype=torch.float32)
    cols = torch.randperm(k, generator=g)[:n_outliers]
    a[:, cols] *= scale
    return Dense(a, w, m, n, k)


def dense(seed=0, m=2048, n=4096, k=4096, outlier_frac=0.01, outlier_scale=20.0, decode_m=16):
    """bf16 activation with outlier channels, bf16 weight ~ N(0, 0.02).
    Returns (Dense, decode activation [decode_m, k] with the same channels)."""
    g = _gen(seed)
    a = torch.randn(m, k, generator=g, dtype=torch.float32)
    cols = _outlier_cols(k, outlier_frac, g)
    a[:, cols] *= outlier_scale
    w = 0.02 * torch.randn(n, k, generator=g, dtype=torch.float32)
    a16 = torch.randn(decode_m, k, generator=g, dtype=torch.float32)
    a16[:, cols] *= outlier_scale
    return Dense(_bf16(a), _bf16(w), m, n, k), _bf16(a16)


def prefill(seed=0, m=8192, n=16384, k=5120, outlier_frac=0.005, outlier_scale=30.0):
    g = _gen(seed)
    a = torch.randn(m, k, generator=g, dtype=torch.float32)
    cols = _outlier_cols(k, outlier_frac, g)
    a[:, cols] *= outlier_scale
    w = 0.02 * torch.randn(n, k, generator=g, dtype=torch.float32)
    return Dense(_bf16(a), _bf16(w), m, n, k)


@dataclass
class MoE:
    x: torch.Tensor          # [E, m, 2h] bf16, gate | up
    mask: torch.Tensor       # [E] int32 valid rows
    w: torch.Tensor          # [E, N, h] bf16 down-proj
    e: int
    m: int
    h: int
    n: int


def moe(seed=0, e=8, m=512, h=8192, n=5120, mask_lo=0, mask=None):
    """Routed-expert down projection input: valid rows per expert uniform in
    [mask_lo, m] (inclusive) unless given."""
    g = _gen(seed)
    x = torch.randn(e, m, 2 * h, generator=g, dtype=torch.float32)
    if mask is None:
        mk = torch.randint(mask_lo, m + 1, (e,), generator=g, dtype=torch.int32)
    else:
        mk = torch.as_tensor(mask, dtype=torch.int32)
    w = torch.empty(e, n, h, dtype=torch.float32)
    for i in range(e):  # per expert, to bound peak host memory
        w[i] = 0.02 * torch.randn(n, h, generator=g, dtype=torch.float32)
    return MoE(_bf16(x), mk, _bf16(w), e, m, h, n)


def expert_mask(seed=0, e=8, m=512, lo=0):
    """Valid rows per expert, uniform in [lo, m] (inclusive)."""
    return torch.randint(lo, m + 1, (e,), generator=_gen(seed), dtype=torch.int32)


@dataclass
class MoESwiGLU:
    x: torch.Tensor          # [E, m, hidden] bf16 expert inputs
    mask: torch.Tensor       # [E] int32 valid rows
    w: torch.Tensor          # [E, 2h, hidden] bf16, gate rows then up rows
    e: int
    m: int
    h: int
    hidden: int


def moe_swiglu(seed=0, e=8, m=512, h=8192, hidden=5120, mask=None):
    """Routed-expert gate_up projection input (the step before the silu_and_mul
    quantize of the moe workload)."""
    g = _gen(seed)
    mk = expert_mask(seed + 1, e, m) if mask is None else torch.as_tensor(mask, dtype=torch.int32)
    x = _bf16(torch.randn(e, m, hidden, generator=g, dtype=torch.float32))
    w = torch.empty(e, 2 * h, hidden, dtype=torch.bfloat16)
    for i in range(e):  # per expert, to bound peak host memory
        w[i] = _bf16(0.02 * torch.randn(2 * h, hidden, generator=g, dtype=torch.float32))
    return MoESwiGLU(x, mk, w, e, m, h, hidden)


@dataclass
class SVDQ:
    x: torch.Tensor          # [M, K] bf16
    pqs: torch.Tensor        # [K] bf16
    w: torch.Tensor          # [N, K] bf16
    l2: torch.Tensor         # [r, K] fp32 LoRA-down weight
    l1_raw: torch.Tensor     # [N, r] fp32 LoRA-up weight before 1/alpha
    bias: torch.Tensor       # [N] bf16
    m: int
    n: int
    k: int
    r: int


def svdquant(seed=0, m=4096, n=3072, k=3072, r=32):
    g = _gen(seed)
    x = torch.randn(m, k, generator=g, dtype=torch.float32)
    pqs = torch.exp(0.5 * torch.randn(k, generator=g, dtype=torch.float32))
    w = 0.02 * torch.randn(n, k, generator=g, dtype=torch.float32)
    l2 = 0.02 * torch.randn(r, k, generator=g, dtype=torch.float32)
    l1_raw = 0.02 * torch.randn(n, r, generator=g, dtype=torch.float32)
    bias = 0.1 * torch.randn(n, generator=g, dtype=torch.float32)
    return SVDQ(_bf16(x), _bf16(pqs), _bf16(w), l2, l1_raw, _bf16(bias), m, n, k, r)


def bits(t: torch.Tensor):
    """numpy view of a CPU tensor's raw bits (bf16 -> uint16, fp32 -> float32)."""
    t = t.contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    if t.dtype == torch.float32:
        return t.numpy()
    if t.dtype == torch.int32:
        return t.numpy()
    if t.dtype == torch.uint8:
        return t.numpy()
    raise TypeError(t.dtype)
