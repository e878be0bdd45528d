"""Thin Python binding of libnvfp4_amd.so (include/nvfp4.h).

Argument marshalling only: torch supplies device memory and the current HIP
stream; every step of the computation runs in the library's kernels.  Outputs
left as None are allocated here with torch (the C ABI never allocates).
Importing this module loads the library and raises if it is missing: there is
no fallback path.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnvfp4_amd.so")

EXPORTS = (
    "nvfp4_quantize",
    "nvfp4_quantize_lora_down",
    "nvfp4_quantize_masked_batched",
    "silu_mul_nvfp4_quantize",
    "nvfp4_gemm",
    "nvfp4_gemm_grouped_masked",
    "nvfp4_gemm_grouped_masked_silu_quantize",
    "nvfp4_gemm_svdquant",
    "nvfp4_gemm_w4a16",
    "nvfp4_alpha",
    "mxfp4_quantize",
    "mxfp4_gemm",
)

STATUS = {
    0: "ok", 1: "null pointer", 2: "bad shape", 3: "pointer not 16-byte aligned",
    4: "rank must be a positive multiple of 32", 5: "unknown dtype",
    6: "unsupported argument", 7: "kernel launch failed",
}

GS_STATIC, GS_DYNAMIC = 0, 1


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m nvfp4_block_scaled_04_amd.build` "
            "(or __graft_entry__.build()); there is no CPU fallback")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    sig = {
        "nvfp4_quantize": [vp, i32, i64, i64, vp, vp, i32, vp, vp, vp],
        "nvfp4_quantize_lora_down": [vp, i64, i64, vp, vp, i64, vp, i32, vp, vp, vp, vp],
        "nvfp4_quantize_masked_batched": [vp, i64, i64, i64, vp, vp, i32, vp, vp, vp],
        "silu_mul_nvfp4_quantize": [vp, i64, i64, i64, vp, vp, i32, vp, vp, vp],
        "nvfp4_gemm": [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, vp],
        "nvfp4_gemm_grouped_masked": [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, vp],
        "nvfp4_gemm_grouped_masked_silu_quantize": [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, vp, vp, vp],
        "nvfp4_gemm_svdquant": [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, vp],
        "nvfp4_gemm_w4a16": [vp, vp, vp, vp, vp, vp, i64, i64, i64, vp],
        "nvfp4_alpha": [vp, vp, vp, i64, vp],
        "mxfp4_quantize": [vp, i32, i64, i64, vp, vp, vp],
        "mxfp4_gemm": [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, vp],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    return lib


_lib = _load()


def lib():
    return _lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(rc, name):
    if rc != 0:
        raise RuntimeError(f"{name}: {STATUS.get(rc, rc)} (status {rc})")


def sf_size(rows, k):
    """pad_up(rows,128) * pad_up(k/16,4): bytes of a swizzled scale buffer."""
    return (rows + 127) // 128 * 128 * ((k // 16 + 3) // 4 * 4)


def _need(t, name):
    if not (t.is_cuda and t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous device tensor")


# ---- quantization -------------------------------------------------------------

def nvfp4_quantize(x, global_scale=None, gs_mode=GS_DYNAMIC, pre_quant_scale=None,
                   out_fp4=None, out_sf=None):
    """x: [m, k] bf16 or fp32 -> (fp4 [m, k/2] uint8, sf [sf_size] uint8, gs [1] fp32)."""
    _need(x, "x")
    m, k = x.shape
    dt = {torch.bfloat16: 0, torch.float32: 1}.get(x.dtype)
    if dt is None:
        raise ValueError("x must be bf16 or fp32")
    dev = x.device
    if global_scale is None:
        global_scale = torch.zeros(1, dtype=torch.float32, device=dev)
    if out_fp4 is None:
        out_fp4 = torch.empty(m, k // 2, dtype=torch.uint8, device=dev)
    if out_sf is None:
        out_sf = torch.empty(sf_size(m, k), dtype=torch.uint8, device=dev)
    rc = _lib.nvfp4_quantize(_ptr(x), dt, m, k, _ptr(pre_quant_scale), _ptr(global_scale),
                             gs_mode, _ptr(out_fp4), _ptr(out_sf), _stream(dev))
    _check(rc, "nvfp4_quantize")
    return out_fp4, out_sf, global_scale


def nvfp4_quantize_lora_down(x, pre_quant_scale, l2, global_scale=None, gs_mode=GS_DYNAMIC,
                             out_fp4=None, out_sf=None, d=None):
    """Smooth NVFP4 quantize of bf16 x [m, k] (pre_quant_scale [k] bf16) and the
    SVDQuant LoRA-down d = bf16((x * pqs) @ l2^T), l2 [r, k] bf16, in one read
    of x.  Returns (fp4 [m, k/2], sf, global_scale [1], d [m, r])."""
    for t, name in ((x, "x"), (pre_quant_scale, "pre_quant_scale"), (l2, "l2")):
        _need(t, name)
    m, k = x.shape
    r = l2.shape[0]
    dev_ = x.device
    if global_scale is None:
        global_scale = torch.zeros(1, dtype=torch.float32, device=dev_)
    if out_fp4 is None:
        out_fp4 = torch.empty(m, k // 2, dtype=torch.uint8, device=dev_)
    if out_sf is None:
        out_sf = torch.empty(sf_size(m, k), dtype=torch.uint8, device=dev_)
    if d is None:
        d = torch.empty(m, r, dtype=torch.bfloat16, device=dev_)
    rc = _lib.nvfp4_quantize_lora_down(_ptr(x), m, k, _ptr(pre_quant_scale), _ptr(l2), r, _ptr(global_scale),
                                       gs_mode, _ptr(out_fp4), _ptr(out_sf), _ptr(d), _stream(dev_))
    _check(rc, "nvfp4_quantize_lora_down")
    return out_fp4, out_sf, global_scale, d


def nvfp4_quantize_masked_batched(x, mask=None, global_scale=None, gs_mode=GS_DYNAMIC,
                                  out_fp4=None, out_sf=None):
    """x: [b, m, k] bf16 -> (fp4 [b, m, k/2], sf [b, sf_size], gs [b])."""
    _need(x, "x")
    b, m, k = x.shape
    dev = x.device
    if global_scale is None:
        global_scale = torch.zeros(b, dtype=torch.float32, device=dev)
    if out_fp4 is None:
        out_fp4 = torch.empty(b, m, k // 2, dtype=torch.uint8, device=dev)
    if out_sf is None:
        out_sf = torch.empty(b, sf_size(m, k), dtype=torch.uint8, device=dev)
    rc = _lib.nvfp4_quantize_masked_batched(_ptr(x), b, m, k, _ptr(mask), _ptr(global_scale),
                                            gs_mode, _ptr(out_fp4), _ptr(out_sf), _stream(dev))
    _check(rc, "nvfp4_quantize_masked_batched")
    return out_fp4, out_sf, global_scale


def silu_mul_nvfp4_quantize(x, mask=None, global_scale=None, gs_mode=GS_DYNAMIC,
                            out_fp4=None, out_sf=None):
    """x: [b, m, 2h] bf16 (gate | up) -> (fp4 [b, m, h/2], sf [b, sf_size(m, h)], gs [b])."""
    _need(x, "x")
    b, m, k2 = x.shape
    h = k2 // 2
    dev = x.device
    if global_scale is None:
        global_scale = torch.zeros(b, dtype=torch.float32, device=dev)
    if out_fp4 is None:
        out_fp4 = torch.empty(b, m, h // 2, dtype=torch.uint8, device=dev)
    if out_sf is None:
        out_sf = torch.empty(b, sf_size(m, h), dtype=torch.uint8, device=dev)
    rc = _lib.silu_mul_nvfp4_quantize(_ptr(x), b, m, k2, _ptr(mask), _ptr(global_scale), gs_mode,
                                      _ptr(out_fp4), _ptr(out_sf), _stream(dev))
    _check(rc, "silu_mul_nvfp4_quantize")
    return out_fp4, out_sf, global_scale


# ---- GEMM -----------------------------------------------------------------------

def nvfp4_gemm(a, b, a_sf, b_sf, alpha, bias=None, out=None, k=None):
    """a: [m, k/2], b: [n, k/2] packed FP4 -> out [m, n] bf16 = alpha*(a@b^T) (+bias)."""
    m, n = a.shape[0], b.shape[0]
    k = a.shape[1] * 2 if k is None else k
    if out is None:
        out = torch.empty(m, n, dtype=torch.bfloat16, device=a.device)
    rc = _lib.nvfp4_gemm(_ptr(a), _ptr(b), _ptr(a_sf), _ptr(b_sf), _ptr(alpha), _ptr(bias),
                         _ptr(out), m, n, k, _stream(a.device))
    _check(rc, "nvfp4_gemm")
    return out


def nvfp4_gemm_grouped_masked(a, b, a_sf, b_sf, alpha, mask, out=None):
    """a: [E, m, k/2], b: [E, n, k/2] -> out [E, m, n] bf16, rows >= mask[e] untouched."""
    E, m, kb = a.shape
    n = b.shape[1]
    if out is None:
        out = torch.empty(E, m, n, dtype=torch.bfloat16, device=a.device)
    rc = _lib.nvfp4_gemm_grouped_masked(_ptr(a), _ptr(b), _ptr(a_sf), _ptr(b_sf), _ptr(alpha),
                                        _ptr(mask), _ptr(out), E, m, n, kb * 2, _stream(a.device))
    _check(rc, "nvfp4_gemm_grouped_masked")
    return out


def nvfp4_gemm_grouped_masked_silu_quantize(a, b, a_sf, b_sf, alpha, mask, global_scale,
                                            out_fp4=None, out_sf=None):
    """a: [E, m, k/2], b: [E, 2h, k/2] (gate rows, then up rows), global_scale:
    [E] static scales of the output -> (fp4 [E, m, h/2], sf [E, sf_size(m, h)])
    of silu(gate) * up of the grouped masked GEMM; rows >= mask[e] of fp4
    untouched."""
    E, m, kb = a.shape
    n2 = b.shape[1]
    h = n2 // 2
    dev = a.device
    if out_fp4 is None:
        out_fp4 = torch.empty(E, m, h // 2, dtype=torch.uint8, device=dev)
    if out_sf is None:
        out_sf = torch.empty(E, sf_size(m, h), dtype=torch.uint8, device=dev)
    rc = _lib.nvfp4_gemm_grouped_masked_silu_quantize(
        _ptr(a), _ptr(b), _ptr(a_sf), _ptr(b_sf), _ptr(alpha), _ptr(mask), _ptr(global_scale),
        E, m, n2, kb * 2, _ptr(out_fp4), _ptr(out_sf), _stream(dev))
    _check(rc, "nvfp4_gemm_grouped_masked_silu_quantize")
    return out_fp4, out_sf


def nvfp4_gemm_svdquant(a, b, a_sf, b_sf, alpha, d, l1, bias=None, out=None):
    """out = alpha*(a@b^T + d@l1^T) (+bias); l1 pre-divided by alpha by the caller."""
    m, n = a.shape[0], b.shape[0]
    k = a.shape[1] * 2
    r = d.shape[1]
    if out is None:
        out = torch.empty(m, n, dtype=torch.bfloat16, device=a.device)
    rc = _lib.nvfp4_gemm_svdquant(_ptr(a), _ptr(b), _ptr(a_sf), _ptr(b_sf), _ptr(alpha), _ptr(d),
                                  _ptr(l1), _ptr(bias), _ptr(out), m, n, k, r, _stream(a.device))
    _check(rc, "nvfp4_gemm_svdquant")
    return out


def nvfp4_gemm_w4a16(a, b, b_sf, alpha, bias=None, out=None):
    """a: [m, k] bf16 activation, b: [n, k/2] packed FP4 weight ->
    out [m, n] bf16 = alpha*(a @ dequant(b)^T) (+bias), alpha = 1/weight gs."""
    _need(a, "a")
    m, k = a.shape
    n = b.shape[0]
    if out is None:
        out = torch.empty(m, n, dtype=torch.bfloat16, device=a.device)
    rc = _lib.nvfp4_gemm_w4a16(_ptr(a), _ptr(b), _ptr(b_sf), _ptr(alpha), _ptr(bias), _ptr(out), m, n, k,
                               _stream(a.device))
    _check(rc, "nvfp4_gemm_w4a16")
    return out


def nvfp4_alpha(gs_a, gs_b, out=None):
    """alpha = 1 / (gs_a * gs_b) elementwise on the device."""
    if out is None:
        out = torch.empty_like(gs_a)
    rc = _lib.nvfp4_alpha(_ptr(gs_a), _ptr(gs_b), _ptr(out), gs_a.numel(), _stream(gs_a.device))
    _check(rc, "nvfp4_alpha")
    return out


# ---- MX setting (32-element blocks, ue8m0 scales) --------------------------------

def sf_size_mx(rows, k):
    """pad_up(rows,128) * pad_up(k/32,4): bytes of a swizzled MX scale buffer."""
    return (rows + 127) // 128 * 128 * ((k // 32 + 3) // 4 * 4)


def mxfp4_quantize(x, out_fp4=None, out_sf=None):
    """x: [m, k] bf16 or fp32 -> (fp4 [m, k/2] uint8, sf [sf_size_mx(m, k)] uint8)."""
    _need(x, "x")
    m, k = x.shape
    dt = {torch.bfloat16: 0, torch.float32: 1}.get(x.dtype)
    if dt is None:
        raise ValueError("x must be bf16 or fp32")
    dev = x.device
    if out_fp4 is None:
        out_fp4 = torch.empty(m, k // 2, dtype=torch.uint8, device=dev)
    if out_sf is None:
        out_sf = torch.empty(sf_size_mx(m, k), dtype=torch.uint8, device=dev)
    rc = _lib.mxfp4_quantize(_ptr(x), dt, m, k, _ptr(out_fp4), _ptr(out_sf), _stream(dev))
    _check(rc, "mxfp4_quantize")
    return out_fp4, out_sf


def mxfp4_gemm(a, b, a_sf, b_sf, alpha=None, bias=None, out=None):
    """a: [m, k/2], b: [n, k/2] MXFP4 -> out [m, n] bf16 = alpha*(a@b^T) (+bias)."""
    m, n = a.shape[0], b.shape[0]
    k = a.shape[1] * 2
    if out is None:
        out = torch.empty(m, n, dtype=torch.bfloat16, device=a.device)
    rc = _lib.mxfp4_gemm(_ptr(a), _ptr(b), _ptr(a_sf), _ptr(b_sf), _ptr(alpha), _ptr(bias), _ptr(out),
                         m, n, k, _stream(a.device))
    _check(rc, "mxfp4_gemm")
    return out
