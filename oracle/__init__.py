"""CPU oracle for NVFP4 quantization and the block-scaled FP4 GEMM.

TEST INFRASTRUCTURE ONLY: tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this package; the product path never does.  The
arithmetic lives in nvfp4_oracle.c (plain C, gcc); this module only marshals
numpy arrays through ctypes.  See nvfp4_oracle.c for the passages each step
follows and the readings taken where the pages are silent.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None

PRO_NONE, PRO_SMOOTH, PRO_SILU = 0, 1, 2
STATIC, DYNAMIC = 0, 1


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB) or (
            os.path.getmtime(_build.LIB) < os.path.getmtime(_build.SRC)
        ):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        u8p = ctypes.POINTER(ctypes.c_uint8)
        L.nvo_bf16_to_f32.restype = ctypes.c_float
        L.nvo_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.nvo_f32_to_bf16.restype = ctypes.c_uint16
        L.nvo_f32_to_bf16.argtypes = [ctypes.c_float]
        L.nvo_e2m1_value.restype = ctypes.c_double
        L.nvo_e2m1_value.argtypes = [ctypes.c_uint8]
        L.nvo_e2m1_encode.restype = ctypes.c_uint8
        L.nvo_e2m1_encode.argtypes = [ctypes.c_float]
        L.nvo_ue4m3_value.restype = ctypes.c_double
        L.nvo_ue4m3_value.argtypes = [ctypes.c_uint8]
        L.nvo_ue4m3_encode.restype = ctypes.c_uint8
        L.nvo_ue4m3_encode.argtypes = [ctypes.c_float]
        L.nvo_silu.restype = ctypes.c_float
        L.nvo_silu.argtypes = [ctypes.c_float]
        L.nvo_global_scale.restype = ctypes.c_float
        L.nvo_global_scale.argtypes = [ctypes.c_float]
        L.nvo_sf_size.restype = ctypes.c_int64
        L.nvo_sf_size.argtypes = [ctypes.c_int64, ctypes.c_int64]
        L.nvo_sf_offset.restype = ctypes.c_int64
        L.nvo_sf_offset.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64]
        L.nvo_quantize.restype = ctypes.c_int
        L.nvo_quantize.argtypes = [
            ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
            u8p, u8p,
        ]
        L.nvo_gemm_rows.restype = ctypes.c_int
        L.nvo_gemm_rows.argtypes = [
            u8p, u8p, u8p, u8p, ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
        ]
        L.nvo_gemm_w4a16_rows.restype = ctypes.c_int
        L.nvo_gemm_w4a16_rows.argtypes = [
            ctypes.c_void_p, u8p, u8p, ctypes.c_float, ctypes.c_void_p, ctypes.c_int64,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
        ]
        L.nvo_f64_to_bf16_via_f32.restype = None
        L.nvo_f64_to_bf16_via_f32.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64]
        L.nvo_ue8m0_value.restype = ctypes.c_double
        L.nvo_ue8m0_value.argtypes = [ctypes.c_uint8]
        L.nvo_sf_size_mx.restype = ctypes.c_int64
        L.nvo_sf_size_mx.argtypes = [ctypes.c_int64, ctypes.c_int64]
        L.nvo_sf_offset_mx.restype = ctypes.c_int64
        L.nvo_sf_offset_mx.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64]
        L.nvo_quantize_mx.restype = ctypes.c_int
        L.nvo_quantize_mx.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, u8p, u8p]
        L.nvo_gemm_mx_rows.restype = ctypes.c_int
        L.nvo_gemm_mx_rows.argtypes = [
            u8p, u8p, u8p, u8p, ctypes.c_float, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
        ]
        L.nvo_num_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _u8(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))


def _vp(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


# ---- scalar codecs (vectorised by plain loops; small inputs only) ----------

def bf16_to_f32(h):
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16(f):
    L = lib()
    f = np.asarray(f, dtype=np.float32).ravel()
    return np.array([L.nvo_f32_to_bf16(float(v)) for v in f], dtype=np.uint16)


def e2m1_value(code):
    return lib().nvo_e2m1_value(int(code))


def e2m1_encode(v):
    return lib().nvo_e2m1_encode(float(np.float32(v)))


def ue4m3_value(code):
    return lib().nvo_ue4m3_value(int(code))


def ue4m3_encode(v):
    return lib().nvo_ue4m3_encode(float(np.float32(v)))


def silu(g):
    return np.float32(lib().nvo_silu(float(np.float32(g))))


def global_scale(amax):
    return np.float32(lib().nvo_global_scale(float(np.float32(amax))))


def sf_size(rows, k):
    return lib().nvo_sf_size(rows, k)


def sf_offset(r, c, k):
    return lib().nvo_sf_offset(r, c, k)


def num_threads():
    return lib().nvo_num_threads()


# ---- tensors ----------------------------------------------------------------

def quantize(x, *, prologue=PRO_NONE, pqs=None, mask=None, gs=None, gs_mode=DYNAMIC,
             out_fp4=None):
    """Quantize x: numpy uint16 (bf16 bits) or float32 of shape [m, k] or
    [b, m, k].  Returns (fp4 [b?, m, K/2] uint8, sf [b?, sf_size] uint8,
    gs [b] float32).  out_fp4 may be given pre-filled (rows >= mask stay)."""
    x = np.ascontiguousarray(x)
    squeeze = x.ndim == 2
    x3 = x[None] if squeeze else x
    b, m, k_in = x3.shape
    if x3.dtype == np.uint16:
        x_dtype = 0
    elif x3.dtype == np.float32:
        x_dtype = 1
    else:
        raise TypeError("x must be bf16 bits (uint16) or float32")
    K = k_in // 2 if prologue == PRO_SILU else k_in
    if gs is None:
        gs = np.zeros(b, dtype=np.float32)
    gs = np.ascontiguousarray(np.asarray(gs, dtype=np.float32).reshape(b)).copy()
    if out_fp4 is None:
        out_fp4 = np.zeros((b, m, K // 2), dtype=np.uint8)
    else:
        out_fp4 = np.ascontiguousarray(out_fp4.reshape(b, m, K // 2)).copy()
    sfsz = sf_size(m, K)
    out_sf = np.zeros((b, sfsz), dtype=np.uint8)
    if pqs is not None:
        pqs = np.ascontiguousarray(pqs, dtype=np.uint16)
    if mask is not None:
        mask = np.ascontiguousarray(mask, dtype=np.int32)
    rc = lib().nvo_quantize(_vp(x3), x_dtype, b, m, k_in, prologue, _vp(pqs), _vp(mask),
                            _vp(gs), gs_mode, _u8(out_fp4), _u8(out_sf))
    if rc != 0:
        raise ValueError(f"oracle quantize rejected the arguments (status {rc})")
    if squeeze:
        return out_fp4[0], out_sf[0], gs
    return out_fp4, out_sf, gs


def gemm_rows(a, b, a_sf, b_sf, alpha, m, n, k, rows=None, bias=None, d=None, l1=None):
    """fp64 alpha*(Adq @ Bdq^T + d @ l1^T) + bias for the given A rows."""
    a = np.ascontiguousarray(a, dtype=np.uint8)
    b = np.ascontiguousarray(b, dtype=np.uint8)
    a_sf = np.ascontiguousarray(a_sf, dtype=np.uint8)
    b_sf = np.ascontiguousarray(b_sf, dtype=np.uint8)
    if rows is None:
        rows = np.arange(m, dtype=np.int64)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    r = 0
    if d is not None:
        d = np.ascontiguousarray(d, dtype=np.uint16)
        l1 = np.ascontiguousarray(l1, dtype=np.uint16)
        r = d.shape[-1]
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.uint16)
    out = np.zeros((len(rows), n), dtype=np.float64)
    rc = lib().nvo_gemm_rows(_u8(a), _u8(b), _u8(a_sf), _u8(b_sf), float(np.float32(alpha)),
                             _vp(bias), _vp(d), _vp(l1), r, m, n, k, _vp(rows), len(rows),
                             _vp(out))
    if rc != 0:
        raise ValueError(f"oracle gemm rejected the arguments (status {rc})")
    return out


def lora_down(x_bf16, pqs_bf16, l2_bf16):
    """SVDQuant's LoRA-down projection of the smoothed activation ([SVD]
    flashinfer mm_nvfp4_svdquant: d = x @ (pqs[:, None] * L2^T), i.e. the
    activation times pre_quant_scale, against the rank-r down weight):
    d[i, p] = sum_k (x[i,k] * pqs[k]) * l2[p,k] in fp64, not rounded.
    x_bf16: uint16 [m, k]; pqs_bf16: uint16 [k]; l2_bf16: uint16 [r, k]."""
    x = bf16_to_f32(np.asarray(x_bf16, dtype=np.uint16)).astype(np.float64)
    p = bf16_to_f32(np.asarray(pqs_bf16, dtype=np.uint16)).astype(np.float64)
    l2 = bf16_to_f32(np.asarray(l2_bf16, dtype=np.uint16)).astype(np.float64)
    return (x * p[None, :]) @ l2.T


def lora_weight_split(pqs_bf16, l2_bf16):
    """The LoRA-down weight with the smoothing folded in ([SVD] flashinfer
    mm_nvfp4_svdquant, parameter d: the factor pqs[:, None] * L2^T), each
    product p = pqs[k] * l2[j, k] written as two bf16 halves that sum to it
    exactly: hi = bf16(p) (round to nearest even) and lo = bf16(p - hi).  The
    fp32 product of two bf16 values is exact (two 8-bit significands), and so
    is p - hi (at most 8 significant bits remain), for products in fp32's
    normal range.  pqs_bf16: uint16 [k]; l2_bf16: uint16 [r, k].  Returns
    uint16 [2, r, k]: the hi rows, then the lo rows."""
    l2 = bf16_to_f32(np.asarray(l2_bf16, dtype=np.uint16))
    p = l2 * bf16_to_f32(np.asarray(pqs_bf16, dtype=np.uint16))[None, :]
    hi = f32_to_bf16(p).reshape(p.shape)
    lo = f32_to_bf16(p - bf16_to_f32(hi)).reshape(p.shape)
    return np.stack([hi, lo])


def gemm_w4a16_rows(a_bf16, b, b_sf, alpha, m, n, k, rows=None, bias=None):
    """fp64 alpha * (A @ Bdq^T) + bias for the given rows of the bf16
    activation A ([NVF] f16a_nvfp4weight_scaled_mm); a_bf16: uint16 bit
    patterns [m, k]; alpha = 1 / the weight's global scale."""
    a_bf16 = np.ascontiguousarray(a_bf16, dtype=np.uint16)
    b = np.ascontiguousarray(b, dtype=np.uint8)
    b_sf = np.ascontiguousarray(b_sf, dtype=np.uint8)
    if rows is None:
        rows = np.arange(m, dtype=np.int64)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.uint16)
    out = np.zeros((len(rows), n), dtype=np.float64)
    rc = lib().nvo_gemm_w4a16_rows(_vp(a_bf16), _u8(b), _u8(b_sf), float(np.float32(alpha)), _vp(bias),
                                   m, n, k, _vp(rows), len(rows), _vp(out))
    if rc != 0:
        raise ValueError(f"oracle weight-only gemm rejected the arguments (status {rc})")
    return out


def f64_to_bf16_via_f32(v):
    """bf16 bit patterns of fp64 values rounded to fp32, then to bf16 (the
    bf16 output of an fp32-accumulated GEMM)."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.zeros(v.shape, dtype=np.uint16)
    lib().nvo_f64_to_bf16_via_f32(_vp(v), _vp(out), v.size)
    return out


def gemm_silu_quantize(a, b, a_sf, b_sf, alpha, gs, mask, m, n2, k):
    """Front half of a routed-expert SwiGLU ([FI] grouped_gemm_nt_masked over
    experts, then silu_and_mul_scaled_nvfp4_experts_quantize with a given
    per-expert global scale), composed from its two steps:
      h[e] = bf16(fp32(alpha[e] * Adq[e] @ Bdq[e]^T))  on the valid rows, [m, n2]
      (fp4, sf) = silu_and_mul quantize of h (gate = columns [0, n2/2), up =
                  the rest), STATIC global scale gs[e], rows >= mask[e] masked.
    a: [E, m, k/2], b: [E, n2, k/2] packed e2m1; a_sf, b_sf: [E, sf bytes];
    alpha, gs: [E] float32; mask: [E] int32.  Returns (fp4 [E, m, n2/4] with
    masked rows zero, sf [E, sf_size(m, n2/2)])."""
    E = len(alpha)
    mask = np.asarray(mask, dtype=np.int32).reshape(E)
    h = np.zeros((E, m, n2), dtype=np.uint16)
    for e in range(E):
        valid = int(min(max(mask[e], 0), m))
        if valid == 0:
            continue
        v = gemm_rows(a[e], b[e], a_sf[e], b_sf[e], alpha[e], m, n2, k, rows=np.arange(valid))
        h[e, :valid] = f64_to_bf16_via_f32(v)
    fp4, sf, _ = quantize(h, prologue=PRO_SILU, mask=mask, gs=gs, gs_mode=STATIC)
    return fp4, sf


# ---- MX variant (ue8m0 scale per 32 elements) ---------------------------------

def ue8m0_value(code):
    return lib().nvo_ue8m0_value(int(code))


def sf_size_mx(rows, k):
    return lib().nvo_sf_size_mx(rows, k)


def sf_offset_mx(r, c, k):
    return lib().nvo_sf_offset_mx(r, c, k)


def quantize_mx(x):
    """MXFP4 quantization of x (uint16 bf16 bits or float32, [m, k], k % 32
    == 0): returns (fp4 [m, k/2] uint8, sf [sf_size_mx(m, k)] uint8)."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        x_dtype = 0
    elif x.dtype == np.float32:
        x_dtype = 1
    else:
        raise TypeError("x must be bf16 bits (uint16) or float32")
    m, k = x.shape
    out_fp4 = np.zeros((m, k // 2), dtype=np.uint8)
    out_sf = np.zeros(sf_size_mx(m, k), dtype=np.uint8)
    rc = lib().nvo_quantize_mx(_vp(x), x_dtype, m, k, _u8(out_fp4), _u8(out_sf))
    if rc != 0:
        raise ValueError(f"oracle MX quantize rejected the arguments (status {rc})")
    return out_fp4, out_sf


def gemm_mx_rows(a, b, a_sf, b_sf, alpha, m, n, k, rows=None, bias=None):
    """fp64 alpha * (Adq @ Bdq^T) + bias for the given A rows, MX operands."""
    a = np.ascontiguousarray(a, dtype=np.uint8)
    b = np.ascontiguousarray(b, dtype=np.uint8)
    a_sf = np.ascontiguousarray(a_sf, dtype=np.uint8)
    b_sf = np.ascontiguousarray(b_sf, dtype=np.uint8)
    if rows is None:
        rows = np.arange(m, dtype=np.int64)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.uint16)
    out = np.zeros((len(rows), n), dtype=np.float64)
    rc = lib().nvo_gemm_mx_rows(_u8(a), _u8(b), _u8(a_sf), _u8(b_sf), float(np.float32(alpha)), _vp(bias),
                                m, n, k, _vp(rows), len(rows), _vp(out))
    if rc != 0:
        raise ValueError(f"oracle MX gemm rejected the arguments (status {rc})")
    return out
