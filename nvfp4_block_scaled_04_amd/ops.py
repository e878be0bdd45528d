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
    "nvfp4_quantize_alpha",
    "nvfp4_quantize_ws",
    "nvfp4_quantize_noalloc",
    "nvfp4_quantize_lora_down",
    "nvfp4_lora_down_prepare",
    "nvfp4_quantize_lora_down_prepared",
    "nvfp4_quantize_masked_batched",
    "nvfp4_quantize_masked_batched_ws",
    "silu_mul_nvfp4_quantize",
    "silu_mul_nvfp4_quantize_ws",
    "nvfp4_gemm",
    "nvfp4_gemm_grouped_masked",
    "nvfp4_gemm_grouped_masked_silu_quantize",
    "nvfp4_gemm_svdquant",
    "nvfp4_gemm_ws",
    "nvfp4_gemm_grouped_masked_ws",
    "nvfp4_gemm_svdquant_ws",
    "nvfp4_gemm_w4a16",
    "nvfp4_linear_small",
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
        "nvfp4_quantize_alpha": [vp, i32, i64, i64, vp, vp, i32, vp, vp, vp, vp, vp],
        "nvfp4_quantize_ws": [vp, i32, i64, i64, vp, vp, i32, vp, vp, vp, vp, vp, i64, vp],
        "nvfp4_quantize_noalloc": [vp, i32, i64, i64, vp, vp, i32, vp, vp, vp, vp, vp],
        "nvfp4_quantize_lora_down": [vp, i64, i64, vp, vp, i64, vp, i32, vp, vp, vp, vp],
        "nvfp4_lora_down_prepare": [vp, vp, i64, i64, vp, vp],
        "nvfp4_quantize_lora_down_prepared": [vp, i64, i64, vp, vp, i64, vp, i32, vp, vp, vp, vp],
        "nvfp4_quantize_masked_batched": [vp, i64, i64, i64, vp, vp, i32, vp, vp, vp],
        "silu_mul_nvfp4_quantize": [vp, i64, i64, i64, vp, vp, i32, vp, vp, vp],
        "nvfp4_quantize_masked_batched_ws": [vp, i64, i64, i64, vp, vp, i32, vp, vp, vp, vp, vp, i64, vp],
        "silu_mul_nvfp4_quantize_ws": [vp, i64, i64, i64, vp, vp, i32, vp, vp, vp, vp, vp, i64, vp],
        "nvfp4_gemm": [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, vp],
        "nvfp4_gemm_grouped_masked": [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, vp],
        "nvfp4_gemm_grouped_masked_silu_quantize": [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, vp, vp, vp],
        "nvfp4_gemm_svdquant": [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, vp],
        "nvfp4_gemm_ws": [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, vp, i64, vp],
        "nvfp4_gemm_grouped_masked_ws": [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, vp, i64, vp],
        "nvfp4_gemm_svdquant_ws": [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, vp, i64, vp],
        "nvfp4_gemm_w4a16": [vp, vp, vp, vp, vp, vp, i64, i64, i64, vp],
        "nvfp4_linear_small": [vp, i64, i64, vp, vp, vp, vp, vp, i64, vp, vp],
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
    if not (isinstance(t, torch.Tensor) and t.is_cuda and t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous device tensor")


BYTES = "bytes"  # any one-byte dtype (uint8, float4_e2m1fn_x2, float8 scale types)
F32, BF16, I32 = (torch.float32,), (torch.bfloat16,), (torch.int32,)


def _dev(t, name, dtype, numel, device):
    """t must be a contiguous tensor on `device` of a dtype in `dtype` (or of
    one byte, for BYTES) holding at least `numel` elements: the library reads
    or writes that many through the raw pointer, so anything else raises here,
    before any launch.  One short-circuit test on the common path (these
    checks run on every eager call); the slow path only words the error."""
    try:
        if (t.is_cuda and t.is_contiguous() and t.numel() >= numel and t.get_device() == device.index
                and (t.element_size() == 1 if dtype is BYTES else t.dtype in dtype)):
            return t
    except AttributeError:
        pass
    _need(t, name)
    if dtype is BYTES and t.element_size() != 1:
        raise ValueError(f"{name} must have a one-byte dtype, got {t.dtype}")
    if dtype is not BYTES and t.dtype not in dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    raise ValueError(f"{name} holds {t.numel()} elements, the call needs {numel}")


def _opt(t, name, dtype, numel, device):
    return None if t is None else _dev(t, name, dtype, numel, device)


def _dims(t, name, nd):
    _need(t, name)
    if t.dim() != nd:
        raise ValueError(f"{name} must have {nd} dimensions, got shape {tuple(t.shape)}")


# ---- quantization -------------------------------------------------------------

def nvfp4_quantize(x, global_scale=None, gs_mode=GS_DYNAMIC, pre_quant_scale=None,
                   out_fp4=None, out_sf=None):
    """x: [m, k] bf16 or fp32 -> (fp4 [m, k/2] uint8, sf [sf_size] uint8, gs [1] fp32)."""
    _dims(x, "x", 2)
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
    _opt(pre_quant_scale, "pre_quant_scale", BF16, k, dev)
    _dev(global_scale, "global_scale", F32, 1, dev)
    _dev(out_fp4, "out_fp4", BYTES, m * (k // 2), dev)
    _dev(out_sf, "out_sf", BYTES, sf_size(m, k), dev)
    rc = _lib.nvfp4_quantize(_ptr(x), dt, m, k, _ptr(pre_quant_scale), _ptr(global_scale),
                             gs_mode, _ptr(out_fp4), _ptr(out_sf), _stream(dev))
    _check(rc, "nvfp4_quantize")
    return out_fp4, out_sf, global_scale


def nvfp4_quantize_alpha(x, gs_other, global_scale=None, gs_mode=GS_DYNAMIC, pre_quant_scale=None,
                         out_fp4=None, out_sf=None, alpha=None):
    """nvfp4_quantize that also writes alpha [1] = 1 / (gs * gs_other[0]) from
    the same launch (gs_other: the weight's global scale [1] fp32).  Returns
    (fp4, sf, gs, alpha)."""
    _dims(x, "x", 2)
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
    if alpha is None:
        alpha = torch.empty(1, dtype=torch.float32, device=dev)
    _opt(pre_quant_scale, "pre_quant_scale", BF16, k, dev)
    _dev(global_scale, "global_scale", F32, 1, dev)
    _dev(gs_other, "gs_other", F32, 1, dev)
    _dev(alpha, "alpha", F32, 1, dev)
    _dev(out_fp4, "out_fp4", BYTES, m * (k // 2), dev)
    _dev(out_sf, "out_sf", BYTES, sf_size(m, k), dev)
    rc = _lib.nvfp4_quantize_alpha(_ptr(x), dt, m, k, _ptr(pre_quant_scale), _ptr(global_scale), gs_mode,
                                   _ptr(gs_other), _ptr(alpha), _ptr(out_fp4), _ptr(out_sf), _stream(dev))
    _check(rc, "nvfp4_quantize_alpha")
    return out_fp4, out_sf, global_scale, alpha


QUANTIZE_WS_BYTES = 4096   # NVFP4_QUANTIZE_WS_BYTES


def quantize_workspace(device):
    """A workspace for nvfp4_quantize_ws (caller-owned device memory)."""
    return torch.empty(QUANTIZE_WS_BYTES, dtype=torch.uint8, device=device)


def nvfp4_quantize_ws(x, workspace, global_scale=None, gs_mode=GS_DYNAMIC, pre_quant_scale=None,
                      gs_other=None, alpha=None, out_fp4=None, out_sf=None):
    """nvfp4_quantize with a caller workspace ([QUANTIZE_WS_BYTES] bytes on the
    device) for the DYNAMIC mode's partial maxima: two launches instead of
    three.  With gs_other ([1] fp32, the weight's global scale) it also writes
    alpha = 1 / (gs * gs_other[0]) (allocated when None).  Returns (fp4, sf,
    gs, alpha or None)."""
    _dims(x, "x", 2)
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
    if gs_other is not None and alpha is None:
        alpha = torch.empty(1, dtype=torch.float32, device=dev)
    if (gs_other is None) != (alpha is None):
        raise ValueError("gs_other and alpha go together")
    _opt(pre_quant_scale, "pre_quant_scale", BF16, k, dev)
    _dev(global_scale, "global_scale", F32, 1, dev)
    _opt(gs_other, "gs_other", F32, 1, dev)
    _opt(alpha, "alpha", F32, 1, dev)
    _dev(out_fp4, "out_fp4", BYTES, m * (k // 2), dev)
    _dev(out_sf, "out_sf", BYTES, sf_size(m, k), dev)
    _dev(workspace, "workspace", BYTES, QUANTIZE_WS_BYTES, dev)
    rc = _lib.nvfp4_quantize_ws(_ptr(x), dt, m, k, _ptr(pre_quant_scale), _ptr(global_scale), gs_mode,
                                _ptr(gs_other), _ptr(alpha), _ptr(out_fp4), _ptr(out_sf), _ptr(workspace),
                                workspace.numel(), _stream(dev))
    _check(rc, "nvfp4_quantize_ws")
    return out_fp4, out_sf, global_scale, alpha


def nvfp4_quantize_noalloc(x, global_scale, gs_other=None, alpha=None, gs_mode=GS_DYNAMIC, pre_quant_scale=None,
                           out_fp4=None, out_sf=None):
    """nvfp4_quantize_ws with the library's static scratch array in place of
    a workspace: every output must be given (nothing is allocated here).
    Returns (fp4, sf, gs, alpha)."""
    _dims(x, "x", 2)
    m, k = x.shape
    dt = {torch.bfloat16: 0, torch.float32: 1}.get(x.dtype)
    if dt is None:
        raise ValueError("x must be bf16 or fp32")
    if out_fp4 is None or out_sf is None:
        raise ValueError("nvfp4_quantize_noalloc allocates nothing: pass out_fp4 and out_sf")
    if (gs_other is None) != (alpha is None):
        raise ValueError("gs_other and alpha go together")
    dev = x.device
    _opt(pre_quant_scale, "pre_quant_scale", BF16, k, dev)
    _dev(global_scale, "global_scale", F32, 1, dev)
    _opt(gs_other, "gs_other", F32, 1, dev)
    _opt(alpha, "alpha", F32, 1, dev)
    _dev(out_fp4, "out_fp4", BYTES, m * (k // 2), dev)
    _dev(out_sf, "out_sf", BYTES, sf_size(m, k), dev)
    rc = _lib.nvfp4_quantize_noalloc(_ptr(x), dt, m, k, _ptr(pre_quant_scale), _ptr(global_scale), gs_mode,
                                     _ptr(gs_other), _ptr(alpha), _ptr(out_fp4), _ptr(out_sf), _stream(dev))
    _check(rc, "nvfp4_quantize_noalloc")
    return out_fp4, out_sf, global_scale, alpha


def _lora_down(fn, name, x, pre_quant_scale, w, r, global_scale, gs_mode, out_fp4, out_sf, d):
    m, k = x.shape
    dev_ = x.device
    _dev(x, "x", BF16, m * k, dev_)
    _dev(pre_quant_scale, "pre_quant_scale", BF16, k, dev_)
    if global_scale is None:
        global_scale = torch.zeros(1, dtype=torch.float32, device=dev_)
    if out_fp4 is None:
        out_fp4 = torch.empty(m, k // 2, dtype=torch.uint8, device=dev_)
    if out_sf is None:
        out_sf = torch.empty(sf_size(m, k), dtype=torch.uint8, device=dev_)
    if d is None:
        d = torch.empty(m, r, dtype=torch.bfloat16, device=dev_)
    _dev(global_scale, "global_scale", F32, 1, dev_)
    _dev(out_fp4, "out_fp4", BYTES, m * (k // 2), dev_)
    _dev(out_sf, "out_sf", BYTES, sf_size(m, k), dev_)
    _dev(d, "d", BF16, m * r, dev_)
    rc = fn(_ptr(x), m, k, _ptr(pre_quant_scale), _ptr(w), r, _ptr(global_scale), gs_mode, _ptr(out_fp4),
            _ptr(out_sf), _ptr(d), _stream(dev_))
    _check(rc, name)
    return out_fp4, out_sf, global_scale, d


def nvfp4_quantize_lora_down(x, pre_quant_scale, l2, global_scale=None, gs_mode=GS_DYNAMIC,
                             out_fp4=None, out_sf=None, d=None):
    """Smooth NVFP4 quantize of bf16 x [m, k] (pre_quant_scale [k] bf16) and the
    SVDQuant LoRA-down d = bf16((x * pqs) @ l2^T), l2 [r, k] bf16, in one read
    of x.  Returns (fp4 [m, k/2], sf, global_scale [1], d [m, r])."""
    _dims(x, "x", 2)
    _dims(l2, "l2", 2)
    m, k = x.shape
    r = l2.shape[0]
    if l2.shape[1] != k:
        raise ValueError(f"l2 must be [r, {k}], got {tuple(l2.shape)}")
    _dev(l2, "l2", BF16, r * k, x.device)
    return _lora_down(_lib.nvfp4_quantize_lora_down, "nvfp4_quantize_lora_down", x, pre_quant_scale, l2, r,
                      global_scale, gs_mode, out_fp4, out_sf, d)


def lora_prepared_numel(r, k):
    """bf16 elements of the prepared LoRA-down weight (NVFP4_LORA_PREPARED_ELEMS):
    hi and lo, r ranks, k rounded up to 32 columns."""
    return 2 * r * ((k + 31) // 32 * 32)


def nvfp4_lora_down_prepare(pre_quant_scale, l2, out=None):
    """The LoRA-down weight with the smoothing folded in, pqs[:, None] * L2^T,
    as the exact sum of two bf16 halves (hi = bf16(pqs * l2), lo = bf16(pqs *
    l2 - hi)), in the fused kernel's MFMA operand order (nvfp4.h gives it):
    returns a flat bf16 tensor of lora_prepared_numel(r, k) elements for
    nvfp4_quantize_lora_down_prepared.  A weight transform: run it once."""
    _dims(l2, "l2", 2)
    r, k = l2.shape
    dev_ = l2.device
    _dev(l2, "l2", BF16, r * k, dev_)
    _dev(pre_quant_scale, "pre_quant_scale", BF16, k, dev_)
    n = lora_prepared_numel(r, k)
    if out is None:
        out = torch.empty(n, dtype=torch.bfloat16, device=dev_)
    _dev(out, "out", BF16, n, dev_)
    rc = _lib.nvfp4_lora_down_prepare(_ptr(pre_quant_scale), _ptr(l2), r, k, _ptr(out), _stream(dev_))
    _check(rc, "nvfp4_lora_down_prepare")
    return out


def nvfp4_quantize_lora_down_prepared(x, pre_quant_scale, w_prepared, r, global_scale=None, gs_mode=GS_DYNAMIC,
                                      out_fp4=None, out_sf=None, d=None):
    """nvfp4_quantize_lora_down with the rank-r weight from
    nvfp4_lora_down_prepare in place of l2: the same quantized bytes, and
    d = bf16(x @ (hi + lo)^T).  Returns (fp4, sf, global_scale, d)."""
    _dims(x, "x", 2)
    m, k = x.shape
    _dev(w_prepared, "w_prepared", BF16, lora_prepared_numel(r, k), x.device)
    return _lora_down(_lib.nvfp4_quantize_lora_down_prepared, "nvfp4_quantize_lora_down_prepared", x,
                      pre_quant_scale, w_prepared, r, global_scale, gs_mode, out_fp4, out_sf, d)


def nvfp4_quantize_masked_batched(x, mask=None, global_scale=None, gs_mode=GS_DYNAMIC,
                                  out_fp4=None, out_sf=None):
    """x: [b, m, k] bf16 -> (fp4 [b, m, k/2], sf [b, sf_size], gs [b])."""
    _dims(x, "x", 3)
    b, m, k = x.shape
    dev = x.device
    _dev(x, "x", BF16, b * m * k, dev)
    if global_scale is None:
        global_scale = torch.zeros(b, dtype=torch.float32, device=dev)
    if out_fp4 is None:
        out_fp4 = torch.empty(b, m, k // 2, dtype=torch.uint8, device=dev)
    if out_sf is None:
        out_sf = torch.empty(b, sf_size(m, k), dtype=torch.uint8, device=dev)
    _opt(mask, "mask", I32, b, dev)
    _dev(global_scale, "global_scale", F32, b, dev)
    _dev(out_fp4, "out_fp4", BYTES, b * m * (k // 2), dev)
    _dev(out_sf, "out_sf", BYTES, b * sf_size(m, k), dev)
    rc = _lib.nvfp4_quantize_masked_batched(_ptr(x), b, m, k, _ptr(mask), _ptr(global_scale),
                                            gs_mode, _ptr(out_fp4), _ptr(out_sf), _stream(dev))
    _check(rc, "nvfp4_quantize_masked_batched")
    return out_fp4, out_sf, global_scale


def silu_mul_nvfp4_quantize(x, mask=None, global_scale=None, gs_mode=GS_DYNAMIC,
                            out_fp4=None, out_sf=None):
    """x: [b, m, 2h] bf16 (gate | up) -> (fp4 [b, m, h/2], sf [b, sf_size(m, h)], gs [b])."""
    _dims(x, "x", 3)
    b, m, k2 = x.shape
    h = k2 // 2
    dev = x.device
    _dev(x, "x", BF16, b * m * k2, dev)
    if global_scale is None:
        global_scale = torch.zeros(b, dtype=torch.float32, device=dev)
    if out_fp4 is None:
        out_fp4 = torch.empty(b, m, h // 2, dtype=torch.uint8, device=dev)
    if out_sf is None:
        out_sf = torch.empty(b, sf_size(m, h), dtype=torch.uint8, device=dev)
    _opt(mask, "mask", I32, b, dev)
    _dev(global_scale, "global_scale", F32, b, dev)
    _dev(out_fp4, "out_fp4", BYTES, b * m * (h // 2), dev)
    _dev(out_sf, "out_sf", BYTES, b * sf_size(m, h), dev)
    rc = _lib.silu_mul_nvfp4_quantize(_ptr(x), b, m, k2, _ptr(mask), _ptr(global_scale), gs_mode,
                                      _ptr(out_fp4), _ptr(out_sf), _stream(dev))
    _check(rc, "silu_mul_nvfp4_quantize")
    return out_fp4, out_sf, global_scale


def batched_ws_bytes(b, m, k):
    """NVFP4_BATCHED_WS_BYTES(b, m, k): workspace of the batched *_ws quantizers
    (k: the quantized width)."""
    return 4096 + 4 * b * ((m + 127) // 128) * ((k + 63) // 64)


def batched_workspace(b, m, k, device):
    """A workspace for nvfp4_quantize_masked_batched_ws / silu_mul_nvfp4_quantize_ws
    (caller-owned device memory)."""
    return torch.empty(batched_ws_bytes(b, m, k), dtype=torch.uint8, device=device)


def silu_ws_bytes(b, m, k):
    """NVFP4_SILU_WS_BYTES(b, m, k): a silu_mul_nvfp4_quantize_ws workspace that
    also holds h (silu evaluated once); k = k2 / 2."""
    return (batched_ws_bytes(b, m, k) + 255) // 256 * 256 + 2 * b * m * k


def silu_workspace(b, m, k, device):
    """A silu_mul_nvfp4_quantize_ws workspace with room for h (caller-owned)."""
    return torch.empty(silu_ws_bytes(b, m, k), dtype=torch.uint8, device=device)


def _batched_ws(fn, x, b, m, k_in, k, workspace, mask, global_scale, gs_mode, gs_other, alpha, out_fp4, out_sf):
    dev = x.device
    _dev(x, "x", BF16, b * m * k_in, dev)
    if global_scale is None:
        global_scale = torch.zeros(b, dtype=torch.float32, device=dev)
    if out_fp4 is None:
        out_fp4 = torch.empty(b, m, k // 2, dtype=torch.uint8, device=dev)
    if out_sf is None:
        out_sf = torch.empty(b, sf_size(m, k), dtype=torch.uint8, device=dev)
    if alpha is not None and gs_other is None:
        raise ValueError("alpha needs gs_other")
    if gs_other is not None and alpha is None:
        alpha = torch.empty(b, dtype=torch.float32, device=dev)
    _opt(mask, "mask", I32, b, dev)
    _dev(global_scale, "global_scale", F32, b, dev)
    _opt(gs_other, "gs_other", F32, b, dev)
    _opt(alpha, "alpha", F32, b, dev)
    _dev(out_fp4, "out_fp4", BYTES, b * m * (k // 2), dev)
    _dev(out_sf, "out_sf", BYTES, b * sf_size(m, k), dev)
    if gs_mode == GS_DYNAMIC:
        _dev(workspace, "workspace", BYTES, batched_ws_bytes(b, m, k), dev)
    wsb = workspace.numel() if workspace is not None else 0
    rc = getattr(_lib, fn)(_ptr(x), b, m, k_in, _ptr(mask), _ptr(global_scale), gs_mode, _ptr(gs_other),
                           _ptr(alpha), _ptr(out_fp4), _ptr(out_sf), _ptr(workspace), wsb, _stream(dev))
    _check(rc, fn)
    return out_fp4, out_sf, global_scale, alpha


def nvfp4_quantize_masked_batched_ws(x, workspace, mask=None, global_scale=None, gs_mode=GS_DYNAMIC,
                                     gs_other=None, alpha=None, out_fp4=None, out_sf=None):
    """nvfp4_quantize_masked_batched with a workspace ([batched_ws_bytes(b, m, k)]
    bytes) and, given gs_other [b], alpha [b] = 1 / (gs * gs_other) from the same
    call -> (fp4, sf, gs, alpha or None)."""
    _dims(x, "x", 3)
    b, m, k = x.shape
    return _batched_ws("nvfp4_quantize_masked_batched_ws", x, b, m, k, k, workspace, mask, global_scale,
                       gs_mode, gs_other, alpha, out_fp4, out_sf)


def silu_mul_nvfp4_quantize_ws(x, workspace, mask=None, global_scale=None, gs_mode=GS_DYNAMIC,
                               gs_other=None, alpha=None, out_fp4=None, out_sf=None):
    """silu_mul_nvfp4_quantize with a workspace (at least batched_ws_bytes(b, m, h)
    bytes; silu_ws_bytes(b, m, h) or more: silu evaluated once) and, given
    gs_other [b], alpha [b] from the same call -> (fp4, sf, gs, alpha or None)."""
    _dims(x, "x", 3)
    b, m, k2 = x.shape
    return _batched_ws("silu_mul_nvfp4_quantize_ws", x, b, m, k2, k2 // 2, workspace, mask, global_scale,
                       gs_mode, gs_other, alpha, out_fp4, out_sf)


# ---- GEMM -----------------------------------------------------------------------

def _operands(a, b, a_sf, b_sf, E, m, n, k, dev, sfsz):
    """Packed FP4 operands (E items of [m|n, k/2]) and their scale buffers."""
    if b.shape[-1] != a.shape[-1]:
        raise ValueError(f"a and b must have the same bytes per row, got {a.shape[-1]} and {b.shape[-1]}")
    _dev(a, "a", BYTES, E * m * (k // 2), dev)
    _dev(b, "b", BYTES, E * n * (k // 2), dev)
    _dev(a_sf, "a_sf", BYTES, E * sfsz(m, k), dev)
    _dev(b_sf, "b_sf", BYTES, E * sfsz(n, k), dev)


GEMM_WS_BYTES = 33554432   # NVFP4_GEMM_WS_BYTES


def gemm_workspace(device):
    """A workspace for the split-tail GEMM schedule (caller-owned device memory)."""
    return torch.empty(GEMM_WS_BYTES, dtype=torch.uint8, device=device)


def _ws_args(workspace, dev):
    if workspace is None:
        return []
    _dev(workspace, "workspace", BYTES, GEMM_WS_BYTES, dev)
    return [_ptr(workspace), workspace.numel()]


def nvfp4_gemm(a, b, a_sf, b_sf, alpha, bias=None, out=None, k=None, workspace=None):
    """a: [m, k/2], b: [n, k/2] packed FP4 -> out [m, n] bf16 = alpha*(a@b^T) (+bias).
    With a workspace ([GEMM_WS_BYTES] bytes) the call is nvfp4_gemm_ws."""
    _dims(a, "a", 2)
    _dims(b, "b", 2)
    m, n = a.shape[0], b.shape[0]
    if k is not None and k != a.shape[1] * 2:
        raise ValueError(f"k = {k} does not match a's {a.shape[1]} bytes per row")
    k = a.shape[1] * 2
    dev = a.device
    if out is None:
        out = torch.empty(m, n, dtype=torch.bfloat16, device=dev)
    _operands(a, b, a_sf, b_sf, 1, m, n, k, dev, sf_size)
    _dev(alpha, "alpha", F32, 1, dev)
    _opt(bias, "bias", BF16, n, dev)
    _dev(out, "out", BF16, m * n, dev)
    ws = _ws_args(workspace, dev)
    f = _lib.nvfp4_gemm_ws if ws else _lib.nvfp4_gemm
    rc = f(_ptr(a), _ptr(b), _ptr(a_sf), _ptr(b_sf), _ptr(alpha), _ptr(bias),
           _ptr(out), m, n, k, *ws, _stream(a.device))
    _check(rc, "nvfp4_gemm_ws" if ws else "nvfp4_gemm")
    return out


def nvfp4_gemm_grouped_masked(a, b, a_sf, b_sf, alpha, mask, out=None, workspace=None):
    """a: [E, m, k/2], b: [E, n, k/2] -> out [E, m, n] bf16, rows >= mask[e] untouched.
    With a workspace ([GEMM_WS_BYTES] bytes) the call is nvfp4_gemm_grouped_masked_ws."""
    _dims(a, "a", 3)
    _dims(b, "b", 3)
    E, m, kb = a.shape
    n = b.shape[1]
    dev = a.device
    if b.shape[0] != E:
        raise ValueError(f"b must hold {E} experts, got {b.shape[0]}")
    if out is None:
        out = torch.empty(E, m, n, dtype=torch.bfloat16, device=dev)
    _operands(a, b, a_sf, b_sf, E, m, n, kb * 2, dev, sf_size)
    _dev(alpha, "alpha", F32, E, dev)
    _dev(mask, "mask", I32, E, dev)
    _dev(out, "out", BF16, E * m * n, dev)
    ws = _ws_args(workspace, dev)
    f = _lib.nvfp4_gemm_grouped_masked_ws if ws else _lib.nvfp4_gemm_grouped_masked
    rc = f(_ptr(a), _ptr(b), _ptr(a_sf), _ptr(b_sf), _ptr(alpha),
           _ptr(mask), _ptr(out), E, m, n, kb * 2, *ws, _stream(a.device))
    _check(rc, "nvfp4_gemm_grouped_masked_ws" if ws else "nvfp4_gemm_grouped_masked")
    return out


def nvfp4_gemm_grouped_masked_silu_quantize(a, b, a_sf, b_sf, alpha, mask, global_scale,
                                            out_fp4=None, out_sf=None):
    """a: [E, m, k/2], b: [E, 2h, k/2] (gate rows, then up rows), global_scale:
    [E] static scales of the output -> (fp4 [E, m, h/2], sf [E, sf_size(m, h)])
    of silu(gate) * up of the grouped masked GEMM; rows >= mask[e] of fp4
    untouched."""
    _dims(a, "a", 3)
    _dims(b, "b", 3)
    E, m, kb = a.shape
    n2 = b.shape[1]
    h = n2 // 2
    dev = a.device
    if b.shape[0] != E:
        raise ValueError(f"b must hold {E} experts, got {b.shape[0]}")
    _operands(a, b, a_sf, b_sf, E, m, n2, kb * 2, dev, sf_size)
    _dev(alpha, "alpha", F32, E, dev)
    _dev(mask, "mask", I32, E, dev)
    _dev(global_scale, "global_scale", F32, E, dev)
    if out_fp4 is None:
        out_fp4 = torch.empty(E, m, h // 2, dtype=torch.uint8, device=dev)
    if out_sf is None:
        out_sf = torch.empty(E, sf_size(m, h), dtype=torch.uint8, device=dev)
    _dev(out_fp4, "out_fp4", BYTES, E * m * (h // 2), dev)
    _dev(out_sf, "out_sf", BYTES, E * sf_size(m, h), dev)
    rc = _lib.nvfp4_gemm_grouped_masked_silu_quantize(
        _ptr(a), _ptr(b), _ptr(a_sf), _ptr(b_sf), _ptr(alpha), _ptr(mask), _ptr(global_scale),
        E, m, n2, kb * 2, _ptr(out_fp4), _ptr(out_sf), _stream(dev))
    _check(rc, "nvfp4_gemm_grouped_masked_silu_quantize")
    return out_fp4, out_sf


def nvfp4_gemm_svdquant(a, b, a_sf, b_sf, alpha, d, l1, bias=None, out=None, workspace=None):
    """out = alpha*(a@b^T + d@l1^T) (+bias); l1 pre-divided by alpha by the caller.
    With a workspace ([GEMM_WS_BYTES] bytes) the call is nvfp4_gemm_svdquant_ws."""
    _dims(a, "a", 2)
    _dims(b, "b", 2)
    _dims(d, "d", 2)
    m, n = a.shape[0], b.shape[0]
    k = a.shape[1] * 2
    r = d.shape[1]
    dev = a.device
    if out is None:
        out = torch.empty(m, n, dtype=torch.bfloat16, device=dev)
    _operands(a, b, a_sf, b_sf, 1, m, n, k, dev, sf_size)
    _dev(alpha, "alpha", F32, 1, dev)
    _dev(d, "d", BF16, m * r, dev)
    _dev(l1, "l1", BF16, n * r, dev)
    _opt(bias, "bias", BF16, n, dev)
    _dev(out, "out", BF16, m * n, dev)
    ws = _ws_args(workspace, dev)
    f = _lib.nvfp4_gemm_svdquant_ws if ws else _lib.nvfp4_gemm_svdquant
    rc = f(_ptr(a), _ptr(b), _ptr(a_sf), _ptr(b_sf), _ptr(alpha), _ptr(d),
           _ptr(l1), _ptr(bias), _ptr(out), m, n, k, r, *ws, _stream(a.device))
    _check(rc, "nvfp4_gemm_svdquant_ws" if ws else "nvfp4_gemm_svdquant")
    return out


def nvfp4_gemm_w4a16(a, b, b_sf, alpha, bias=None, out=None):
    """a: [m, k] bf16 activation, b: [n, k/2] packed FP4 weight ->
    out [m, n] bf16 = alpha*(a @ dequant(b)^T) (+bias), alpha = 1/weight gs."""
    _dims(a, "a", 2)
    _dims(b, "b", 2)
    m, k = a.shape
    n = b.shape[0]
    dev = a.device
    if b.shape[1] * 2 != k:
        raise ValueError(f"b must be [n, {k // 2}] packed FP4, got {tuple(b.shape)}")
    if out is None:
        out = torch.empty(m, n, dtype=torch.bfloat16, device=dev)
    _dev(a, "a", BF16, m * k, dev)
    _dev(b, "b", BYTES, n * (k // 2), dev)
    _dev(b_sf, "b_sf", BYTES, sf_size(n, k), dev)
    _dev(alpha, "alpha", F32, 1, dev)
    _opt(bias, "bias", BF16, n, dev)
    _dev(out, "out", BF16, m * n, dev)
    rc = _lib.nvfp4_gemm_w4a16(_ptr(a), _ptr(b), _ptr(b_sf), _ptr(alpha), _ptr(bias), _ptr(out), m, n, k,
                               _stream(a.device))
    _check(rc, "nvfp4_gemm_w4a16")
    return out


def nvfp4_linear_small(x, b, b_sf, gs_b, bias=None, out=None, gs_out=None):
    """x: [m, k] bf16 (m <= 16), b: [n, k/2] packed FP4 weight with its scales
    and global scale gs_b -> out [m, n] bf16: the dynamic quantization of x,
    alpha = 1/(gs*gs_b) and the NVFP4 GEMM in one launch (bit for bit the
    three calls).  gs_out, if given, receives the activation's global scale."""
    _dims(x, "x", 2)
    _dims(b, "b", 2)
    m, k = x.shape
    n = b.shape[0]
    dev = x.device
    if b.shape[1] * 2 != k:
        raise ValueError(f"b must be [n, {k // 2}] packed FP4, got {tuple(b.shape)}")
    if out is None:
        out = torch.empty(m, n, dtype=torch.bfloat16, device=dev)
    _dev(x, "x", BF16, m * k, dev)
    _dev(b, "b", BYTES, n * (k // 2), dev)
    _dev(b_sf, "b_sf", BYTES, sf_size(n, k), dev)
    _dev(gs_b, "gs_b", F32, 1, dev)
    _opt(bias, "bias", BF16, n, dev)
    _opt(gs_out, "gs_out", F32, 1, dev)
    _dev(out, "out", BF16, m * n, dev)
    rc = _lib.nvfp4_linear_small(_ptr(x), m, k, _ptr(b), _ptr(b_sf), _ptr(gs_b), _ptr(bias), _ptr(out), n,
                                 _ptr(gs_out), _stream(dev))
    _check(rc, "nvfp4_linear_small")
    return out


def nvfp4_alpha(gs_a, gs_b, out=None):
    """alpha = 1 / (gs_a * gs_b) elementwise on the device."""
    _need(gs_a, "gs_a")
    dev = gs_a.device
    if out is None:
        out = torch.empty_like(gs_a)
    _dev(gs_a, "gs_a", F32, 1, dev)
    _dev(gs_b, "gs_b", F32, gs_a.numel(), dev)
    _dev(out, "out", F32, gs_a.numel(), dev)
    rc = _lib.nvfp4_alpha(_ptr(gs_a), _ptr(gs_b), _ptr(out), gs_a.numel(), _stream(gs_a.device))
    _check(rc, "nvfp4_alpha")
    return out


# ---- MX setting (32-element blocks, ue8m0 scales) --------------------------------

def sf_size_mx(rows, k):
    """pad_up(rows,128) * pad_up(k/32,4): bytes of a swizzled MX scale buffer."""
    return (rows + 127) // 128 * 128 * ((k // 32 + 3) // 4 * 4)


def mxfp4_quantize(x, out_fp4=None, out_sf=None):
    """x: [m, k] bf16 or fp32 -> (fp4 [m, k/2] uint8, sf [sf_size_mx(m, k)] uint8)."""
    _dims(x, "x", 2)
    m, k = x.shape
    dt = {torch.bfloat16: 0, torch.float32: 1}.get(x.dtype)
    if dt is None:
        raise ValueError("x must be bf16 or fp32")
    dev = x.device
    if out_fp4 is None:
        out_fp4 = torch.empty(m, k // 2, dtype=torch.uint8, device=dev)
    if out_sf is None:
        out_sf = torch.empty(sf_size_mx(m, k), dtype=torch.uint8, device=dev)
    _dev(out_fp4, "out_fp4", BYTES, m * (k // 2), dev)
    _dev(out_sf, "out_sf", BYTES, sf_size_mx(m, k), dev)
    rc = _lib.mxfp4_quantize(_ptr(x), dt, m, k, _ptr(out_fp4), _ptr(out_sf), _stream(dev))
    _check(rc, "mxfp4_quantize")
    return out_fp4, out_sf


def mxfp4_gemm(a, b, a_sf, b_sf, alpha=None, bias=None, out=None):
    """a: [m, k/2], b: [n, k/2] MXFP4 -> out [m, n] bf16 = alpha*(a@b^T) (+bias)."""
    _dims(a, "a", 2)
    _dims(b, "b", 2)
    m, n = a.shape[0], b.shape[0]
    k = a.shape[1] * 2
    dev = a.device
    if out is None:
        out = torch.empty(m, n, dtype=torch.bfloat16, device=dev)
    _operands(a, b, a_sf, b_sf, 1, m, n, k, dev, sf_size_mx)
    _opt(alpha, "alpha", F32, 1, dev)
    _opt(bias, "bias", BF16, n, dev)
    _dev(out, "out", BF16, m * n, dev)
    rc = _lib.mxfp4_gemm(_ptr(a), _ptr(b), _ptr(a_sf), _ptr(b_sf), _ptr(alpha), _ptr(bias), _ptr(out),
                         m, n, k, _stream(a.device))
    _check(rc, "mxfp4_gemm")
    return out
