"""The C-ABI library loads, exports every entry point include/nvfp4.h declares,
and rejects bad arguments before enqueuing anything (CPU only: every call
here fails validation, so no HIP work is started and no pointer is touched).
"""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4.h")
LIB = os.path.join(ROOT, "nvfp4_block_scaled_04_amd", "libnvfp4_amd.so")

OK, NULLP, SHAPE, MISAL, RANK, DTYPE, UNSUP = 0, 1, 2, 3, 4, 5, 6
P = 0x10000  # a 16-byte aligned address that is never dereferenced here


def declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^int\s+(\w+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} not built; run __graft_entry__.build()")
    L = ctypes.CDLL(LIB)
    return L


def test_header_declares_the_entry_points():
    assert declared() == sorted([
        "nvfp4_alpha", "nvfp4_gemm", "nvfp4_gemm_grouped_masked",
        "nvfp4_gemm_grouped_masked_silu_quantize", "nvfp4_gemm_svdquant",
        "nvfp4_gemm_ws", "nvfp4_gemm_grouped_masked_ws", "nvfp4_gemm_svdquant_ws",
        "nvfp4_gemm_w4a16", "nvfp4_linear_small", "nvfp4_quantize_lora_down",
        "nvfp4_lora_down_prepare", "nvfp4_quantize_lora_down_prepared",
        "nvfp4_quantize", "nvfp4_quantize_alpha", "nvfp4_quantize_ws", "nvfp4_quantize_noalloc",
        "nvfp4_quantize_masked_batched", "nvfp4_quantize_masked_batched_ws",
        "silu_mul_nvfp4_quantize", "silu_mul_nvfp4_quantize_ws",
        "mxfp4_quantize", "mxfp4_gemm",
    ])


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (\w+)$", out, flags=re.M))
    for name in declared():
        assert name in exported, name
        assert getattr(lib, name)


def test_binding_names_match_header():
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "ops_src", os.path.join(ROOT, "nvfp4_block_scaled_04_amd", "ops.py"))
    src = open(spec.origin).read()
    exports = re.search(r"EXPORTS = \((.*?)\)", src, flags=re.S).group(1)
    names = sorted(re.findall(r'"(\w+)"', exports))
    assert names == declared()


def call(lib, name, *args):
    f = getattr(lib, name)
    f.restype = ctypes.c_int
    conv = []
    for a in args:
        if isinstance(a, float):
            conv.append(ctypes.c_float(a))
        else:
            conv.append(ctypes.c_int64(a) if a is not None else ctypes.c_void_p(None))
    return f(*conv)


def q(lib, x=P, dt=0, m=128, k=256, pqs=None, gs=P, mode=1, o=P, s=P):
    return lib.nvfp4_quantize(ctypes.c_void_p(x), ctypes.c_int(dt), ctypes.c_int64(m),
                              ctypes.c_int64(k), ctypes.c_void_p(pqs), ctypes.c_void_p(gs),
                              ctypes.c_int(mode), ctypes.c_void_p(o), ctypes.c_void_p(s),
                              ctypes.c_void_p(None))


def test_quantize_validation(lib):
    assert q(lib, x=None) == NULLP
    assert q(lib, gs=None) == NULLP
    assert q(lib, o=None) == NULLP
    assert q(lib, s=None) == NULLP
    assert q(lib, dt=2) == DTYPE
    assert q(lib, mode=5) == UNSUP
    assert q(lib, k=15) == SHAPE
    assert q(lib, k=24) == SHAPE
    assert q(lib, k=0) == SHAPE
    assert q(lib, m=0) == SHAPE
    assert q(lib, m=-3) == SHAPE
    assert q(lib, x=P + 8) == MISAL
    assert q(lib, o=P + 4) == MISAL
    assert q(lib, s=P + 1) == MISAL
    assert q(lib, pqs=P + 2) == MISAL
    assert q(lib, gs=P + 2) == MISAL


def qb(lib, fn, x=P, b=2, m=128, k=256, mask=None, gs=P, mode=1, o=P, s=P):
    f = getattr(lib, fn)
    return f(ctypes.c_void_p(x), ctypes.c_int64(b), ctypes.c_int64(m), ctypes.c_int64(k),
             ctypes.c_void_p(mask), ctypes.c_void_p(gs), ctypes.c_int(mode), ctypes.c_void_p(o),
             ctypes.c_void_p(s), ctypes.c_void_p(None))


@pytest.mark.parametrize("fn", ["nvfp4_quantize_masked_batched", "silu_mul_nvfp4_quantize"])
def test_batched_validation(lib, fn):
    assert qb(lib, fn, x=None) == NULLP
    assert qb(lib, fn, gs=None) == NULLP
    assert qb(lib, fn, b=0) == SHAPE
    assert qb(lib, fn, m=0) == SHAPE
    assert qb(lib, fn, k=8) == SHAPE
    assert qb(lib, fn, mode=2) == UNSUP
    assert qb(lib, fn, x=P + 2) == MISAL
    assert qb(lib, fn, mask=P + 1) == MISAL


@pytest.mark.parametrize("fn,silu", [("nvfp4_quantize_masked_batched_ws", False), ("silu_mul_nvfp4_quantize_ws", True)])
def test_batched_ws_validation(lib, fn, silu):
    """The batched checks, the optional alpha pair and, in DYNAMIC mode, the
    workspace: present, at least NVFP4_BATCHED_WS_BYTES(b, m, k), 16-byte
    aligned; STATIC mode ignores it."""
    f = getattr(lib, fn)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    f.argtypes = [vp, i64, i64, i64, vp, vp, ctypes.c_int, vp, vp, vp, vp, vp, i64, vp]
    b, m, kin = 2, 300, 128
    k = kin // 2 if silu else kin
    need = 4096 + 4 * b * ((m + 127) // 128) * ((k + 63) // 64)
    run = lambda x=P, kk=kin, mode=1, go=None, al=None, ws=P, wsb=need, mask=None: \
        f(x, b, m, kk, mask, P, mode, go, al, P, P, ws, wsb, None)
    assert run(x=None) == NULLP
    assert run(go=P) == NULLP
    assert run(al=P) == NULLP
    assert run(ws=None) == NULLP
    assert run(wsb=need - 1) == SHAPE
    assert run(ws=P + 4) == MISAL
    assert run(go=P + 2, al=P) == MISAL
    assert run(mask=P + 1) == MISAL
    assert run(mode=3) == UNSUP
    assert run(kk=40) == SHAPE
    assert run(mode=0, ws=None, kk=40) == SHAPE   # STATIC: no workspace needed (refused here for k)


def test_silu_width_rules(lib):
    fn = "silu_mul_nvfp4_quantize"
    assert qb(lib, fn, k=33) == SHAPE        # odd gate|up width
    assert qb(lib, fn, k=48) == SHAPE        # h = 24 is not a multiple of 16
    assert qb(lib, fn, k=16) == SHAPE        # h = 8


def g(lib, a=P, b=P, asf=P, bsf=P, alpha=P, bias=None, out=P, m=128, n=128, k=256):
    return lib.nvfp4_gemm(*[ctypes.c_void_p(v) for v in (a, b, asf, bsf, alpha, bias, out)],
                          ctypes.c_int64(m), ctypes.c_int64(n), ctypes.c_int64(k),
                          ctypes.c_void_p(None))


def test_gemm_validation(lib):
    for kw in ("a", "b", "asf", "bsf", "alpha", "out"):
        assert g(lib, **{kw: None}) == NULLP, kw
    assert g(lib, k=40) == SHAPE
    assert g(lib, k=0) == SHAPE
    assert g(lib, m=0) == SHAPE
    assert g(lib, n=-1) == SHAPE
    assert g(lib, a=P + 8) == MISAL
    assert g(lib, out=P + 2) == MISAL
    assert g(lib, bias=P + 2) == MISAL
    assert g(lib, alpha=P + 1) == MISAL
    # 32-bit offsets inside one FP4 matrix: 2^32 - 64 bytes is the limit
    assert g(lib, m=(1 << 20), k=8192) == UNSUP      # 4 GiB of A
    assert g(lib, n=(1 << 20) + 1, k=8192) == UNSUP
    # scale buffers (32-bit descriptors, signed per-step offsets): below 2^31 bytes
    assert g(lib, m=7, n=7, k=1 << 30) == UNSUP       # 128 rows x 2^26 blocks = 2^33 bytes
    assert g(lib, m=7, n=7, k=1 << 28) == UNSUP       # 128 x 2^24 = 2^31 bytes: the first size refused


def test_grouped_validation(lib):
    f = lib.nvfp4_gemm_grouped_masked
    args = lambda mask=P, E=4, k=256: [ctypes.c_void_p(P)] * 5 + [ctypes.c_void_p(mask), ctypes.c_void_p(P),
                                         ctypes.c_int64(E), ctypes.c_int64(64), ctypes.c_int64(64),
                                         ctypes.c_int64(k), ctypes.c_void_p(None)]
    assert f(*args(mask=None)) == NULLP
    assert f(*args(E=0)) == SHAPE
    assert f(*args(k=17)) == SHAPE
    assert f(*args(mask=P + 2)) == MISAL


GEMM_WS = 33554432  # NVFP4_GEMM_WS_BYTES


def test_gemm_ws_validation(lib):
    """The workspace forms keep every check of the plain calls, and refuse a
    workspace that is too small or misaligned; NULL selects the plain
    schedule (here refused for another argument, so nothing launches)."""
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    f = lib.nvfp4_gemm_ws
    f.argtypes = [vp] * 7 + [i64] * 3 + [vp, i64, vp]
    run = lambda a=P, out=P, m=128, k=256, ws=P, wsb=GEMM_WS: f(a, P, P, P, P, None, out, m, 128, k, ws, wsb, None)
    assert run(a=None) == NULLP
    assert run(k=40) == SHAPE
    assert run(m=0) == SHAPE
    assert run(out=P + 2) == MISAL
    assert run(wsb=GEMM_WS - 1) == SHAPE
    assert run(ws=P + 8) == MISAL
    assert run(ws=None, k=40) == SHAPE
    assert run(m=(1 << 20), k=8192) == UNSUP
    fg = lib.nvfp4_gemm_grouped_masked_ws
    fg.argtypes = [vp] * 7 + [i64] * 4 + [vp, i64, vp]
    rung = lambda mask=P, E=4, k=256, ws=P, wsb=GEMM_WS: fg(P, P, P, P, P, mask, P, E, 64, 64, k, ws, wsb, None)
    assert rung(mask=None) == NULLP
    assert rung(E=0) == SHAPE
    assert rung(k=17) == SHAPE
    assert rung(mask=P + 2) == MISAL
    assert rung(wsb=1 << 20) == SHAPE
    assert rung(ws=P + 4) == MISAL
    fs = lib.nvfp4_gemm_svdquant_ws
    fs.argtypes = [vp] * 9 + [i64] * 4 + [vp, i64, vp]
    runs = lambda r=32, d=P, k=256, ws=P, wsb=GEMM_WS: fs(P, P, P, P, P, d, P, None, P, 64, 64, k, r, ws, wsb, None)
    assert runs(r=16) == RANK
    assert runs(d=None) == NULLP
    assert runs(d=P + 8) == MISAL
    assert runs(k=40) == SHAPE
    assert runs(wsb=0) == SHAPE
    assert runs(ws=P + 2) == MISAL


def test_quantize_alpha_validation(lib):
    """nvfp4_quantize's checks, plus the two alpha pointers."""
    f = lib.nvfp4_quantize_alpha
    f.restype = ctypes.c_int

    def run(x=P, dtype=0, k=64, gs_other=P, alpha=P):
        return f(ctypes.c_void_p(x), ctypes.c_int(dtype), ctypes.c_int64(32), ctypes.c_int64(k), ctypes.c_void_p(None),
                 ctypes.c_void_p(P), ctypes.c_int(1), ctypes.c_void_p(gs_other), ctypes.c_void_p(alpha),
                 ctypes.c_void_p(P), ctypes.c_void_p(P), ctypes.c_void_p(None))
    assert run(gs_other=None) == NULLP
    assert run(alpha=None) == NULLP
    assert run(x=None) == NULLP
    assert run(dtype=3) == DTYPE
    assert run(k=40) == SHAPE
    assert run(gs_other=P + 2) == MISAL
    assert run(alpha=P + 1) == MISAL


def test_quantize_ws_validation(lib):
    """nvfp4_quantize's checks, plus the optional alpha pair and, in DYNAMIC
    mode, the workspace (present, large enough, 16-byte aligned)."""
    f = lib.nvfp4_quantize_ws
    f.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    run = lambda x=P, dt=0, m=128, k=256, pqs=None, gs=P, mode=1, go=None, al=None, o=P, s=P, ws=P, wsb=4096: \
        f(x, dt, m, k, pqs, gs, mode, go, al, o, s, ws, wsb, None)
    assert run(go=P) == NULLP            # gs_other without alpha
    assert run(al=P) == NULLP            # alpha without gs_other
    assert run(ws=None) == NULLP         # DYNAMIC needs the workspace
    assert run(wsb=4095) == SHAPE        # smaller than NVFP4_QUANTIZE_WS_BYTES
    assert run(ws=P + 4) == MISAL
    assert run(x=None) == NULLP
    assert run(k=40) == SHAPE
    assert run(dt=2) == DTYPE
    assert run(mode=2) == UNSUP
    assert run(o=P + 8) == MISAL
    assert run(go=P + 2, al=P) == MISAL


def test_quantize_noalloc_validation(lib):
    """nvfp4_quantize's checks and the optional alpha pair, all refused before
    the library touches the device (no symbol lookup on a refused call)."""
    f = lib.nvfp4_quantize_noalloc
    f.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_void_p]
    run = lambda x=P, dt=0, m=128, k=256, pqs=None, gs=P, mode=1, go=None, al=None, o=P, s=P: \
        f(x, dt, m, k, pqs, gs, mode, go, al, o, s, None)
    assert run(go=P) == NULLP
    assert run(al=P) == NULLP
    assert run(x=None) == NULLP
    assert run(s=None) == NULLP
    assert run(k=40) == SHAPE
    assert run(m=0) == SHAPE
    assert run(dt=2) == DTYPE
    assert run(mode=2) == UNSUP


def test_svdquant_rank_and_alignment(lib):
    f = lib.nvfp4_gemm_svdquant

    def run(r=32, d=P, l1=P, k=256):
        return f(*[ctypes.c_void_p(P)] * 5, ctypes.c_void_p(d), ctypes.c_void_p(l1),
                 ctypes.c_void_p(None), ctypes.c_void_p(P), ctypes.c_int64(64), ctypes.c_int64(64),
                 ctypes.c_int64(k), ctypes.c_int64(r), ctypes.c_void_p(None))
    assert run(r=0) == RANK
    assert run(r=16) == RANK
    assert run(r=48) == RANK
    assert run(r=-32) == RANK
    assert run(d=None) == NULLP
    assert run(l1=None) == NULLP
    assert run(d=P + 8) == MISAL     # d must be 16-byte aligned
    assert run(k=40) == SHAPE


def test_w4a16_validation(lib):
    f = lib.nvfp4_gemm_w4a16
    f.argtypes = [ctypes.c_void_p] * 6 + [ctypes.c_int64] * 3 + [ctypes.c_void_p]
    run = lambda a=P, b=P, sf=P, alpha=P, bias=None, out=P, m=16, n=64, k=256: f(a, b, sf, alpha, bias, out, m, n, k, None)
    assert run(a=None) == NULLP
    assert run(alpha=None) == NULLP
    assert run(out=None) == NULLP
    assert run(k=40) == SHAPE
    assert run(k=8) == SHAPE
    assert run(m=0) == SHAPE
    assert run(a=P + 8) == MISAL
    assert run(bias=P + 2) == MISAL
    assert run(alpha=P + 1) == MISAL


def test_linear_small_validation(lib):
    f = lib.nvfp4_linear_small
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64] + [ctypes.c_void_p] * 5 + \
        [ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    run = lambda x=P, m=16, k=4096, b=P, sf=P, gsb=P, bias=None, out=P, n=4096, gso=None: \
        f(x, m, k, b, sf, gsb, bias, out, n, gso, None)
    assert run(x=None) == NULLP
    assert run(b=None) == NULLP
    assert run(sf=None) == NULLP
    assert run(gsb=None) == NULLP
    assert run(out=None) == NULLP
    assert run(m=0) == SHAPE
    assert run(n=0) == SHAPE
    assert run(k=40) == SHAPE
    assert run(m=17) == UNSUP        # more than 16 rows: the three calls
    assert run(k=4096 + 128) == UNSUP
    assert run(k=1040) == UNSUP      # k % 128 != 0
    assert run(x=P + 8) == MISAL
    assert run(out=P + 8) == MISAL
    assert run(bias=P + 2) == MISAL
    assert run(gsb=P + 1) == MISAL
    assert run(gso=P + 2) == MISAL


def test_lora_down_validation(lib):
    f = lib.nvfp4_quantize_lora_down
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                  ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    run = lambda x=P, m=64, k=256, pqs=P, l2=P, r=32, gs=P, mode=1, o4=P, osf=P, d=P: \
        f(x, m, k, pqs, l2, r, gs, mode, o4, osf, d, None)
    assert run(pqs=None) == NULLP
    assert run(l2=None) == NULLP
    assert run(d=None) == NULLP
    assert run(r=16) == RANK
    assert run(r=160) == RANK
    assert run(k=40) == SHAPE
    assert run(k=4112, d=P + 8) == MISAL   # any K % 16 == 0 is accepted (here refused for d's alignment)
    assert run(mode=7) == UNSUP
    assert run(l2=P + 8) == MISAL
    assert run(d=P + 8) == MISAL


def test_lora_down_prepared_validation(lib):
    f = lib.nvfp4_quantize_lora_down_prepared
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                  ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    run = lambda x=P, m=64, k=256, pqs=P, w=P, r=32, gs=P, mode=1, o4=P, osf=P, d=P: \
        f(x, m, k, pqs, w, r, gs, mode, o4, osf, d, None)
    assert run(x=None) == NULLP
    assert run(w=None) == NULLP
    assert run(r=48) == RANK
    assert run(r=0) == RANK
    assert run(k=8) == SHAPE
    assert run(m=0) == SHAPE
    assert run(mode=3) == UNSUP
    assert run(w=P + 4) == MISAL
    g = lib.nvfp4_lora_down_prepare
    g.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    prep = lambda pqs=P, l2=P, r=32, k=256, w=P: g(pqs, l2, r, k, w, None)
    assert prep(pqs=None) == NULLP
    assert prep(l2=None) == NULLP
    assert prep(w=None) == NULLP
    assert prep(r=16) == RANK
    assert prep(r=256) == RANK
    assert prep(k=0) == SHAPE
    assert prep(k=264) == SHAPE   # k % 16 != 0
    assert prep(k=1 << 31) == SHAPE
    assert prep(w=P + 2) == MISAL
    assert prep(pqs=P + 8) == MISAL


def test_alpha_validation(lib):
    f = lib.nvfp4_alpha
    assert f(ctypes.c_void_p(None), ctypes.c_void_p(P), ctypes.c_void_p(P), ctypes.c_int64(1),
             ctypes.c_void_p(None)) == NULLP
    assert f(ctypes.c_void_p(P), ctypes.c_void_p(P), ctypes.c_void_p(P), ctypes.c_int64(0),
             ctypes.c_void_p(None)) == SHAPE


def test_product_does_not_touch_oracle():
    """The library sources and the binding never name the oracle."""
    pkg = os.path.join(ROOT, "nvfp4_block_scaled_04_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".cpp", ".h")):
                txt = open(os.path.join(dirpath, fn)).read()
                assert "import oracle" not in txt and "from oracle" not in txt, fn
                assert "nvfp4_oracle" not in txt and "nvo_" not in txt, fn


def test_gemm_silu_quantize_validation(lib):
    f = lib.nvfp4_gemm_grouped_masked_silu_quantize
    f.argtypes = [ctypes.c_void_p] * 7 + [ctypes.c_int64] * 4 + [ctypes.c_void_p] * 3
    run = lambda a=P, b=P, asf=P, bsf=P, alpha=P, mask=P, gs=P, E=2, m=64, n2=128, k=256, o4=P, osf=P: \
        f(a, b, asf, bsf, alpha, mask, gs, E, m, n2, k, o4, osf, None)
    assert run(mask=None) == NULLP
    assert run(gs=None) == NULLP
    assert run(o4=None) == NULLP
    assert run(osf=None) == NULLP
    assert run(n2=127) == SHAPE        # odd
    assert run(n2=16) == SHAPE         # H = 8 < 16
    assert run(n2=48) == SHAPE         # H = 24 not a multiple of 16
    assert run(k=40) == SHAPE
    assert run(E=0) == SHAPE
    assert run(m=0) == SHAPE
    assert run(o4=P + 8) == MISAL
    assert run(osf=P + 4) == MISAL
    assert run(gs=P + 2) == MISAL
    assert run(mask=P + 1) == MISAL
    assert run(m=1 << 20, k=1 << 13) == UNSUP   # one expert's A spans 2^32 bytes


def test_mx_validation(lib):
    q = lib.mxfp4_quantize
    q.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64] + [ctypes.c_void_p] * 3
    runq = lambda x=P, dt=0, m=64, k=256, o4=P, osf=P: q(x, dt, m, k, o4, osf, None)
    assert runq(x=None) == NULLP
    assert runq(osf=None) == NULLP
    assert runq(dt=3) == DTYPE
    assert runq(k=48) == SHAPE          # not a multiple of 32
    assert runq(k=16) == SHAPE
    assert runq(m=0) == SHAPE
    assert runq(o4=P + 8) == MISAL
    g = lib.mxfp4_gemm
    g.argtypes = [ctypes.c_void_p] * 7 + [ctypes.c_int64] * 3 + [ctypes.c_void_p]
    rung = lambda a=P, b=P, asf=P, bsf=P, alpha=None, bias=None, out=P, m=64, n=64, k=256: \
        g(a, b, asf, bsf, alpha, bias, out, m, n, k, None)
    assert rung(a=None) == NULLP
    assert rung(out=None) == NULLP
    assert rung(k=48) == SHAPE
    assert rung(n=0) == SHAPE
    assert rung(alpha=P + 2) == MISAL
    assert rung(bias=P + 2) == MISAL
    assert rung(m=1 << 20, k=1 << 13) == UNSUP
    # a 2^30-wide K with 7 rows: 128 x 2^25 scale bytes = 2^32, past the
    # 32-bit descriptor the kernel would address them with
    assert rung(m=7, n=7, k=1 << 30) == UNSUP
    assert rung(m=7, n=7, k=1 << 29) == UNSUP        # 128 x 2^24 = 2^31 bytes: the first size refused



def test_quantize_noalloc_alignment_refused(lib):
    f = lib.nvfp4_quantize_noalloc
    f.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_void_p]
    assert f(P + 8, 0, 128, 256, None, P, 1, None, None, P, P, None) == MISAL
    assert f(P, 0, 128, 256, P + 4, P, 1, None, None, P, P, None) == MISAL
    assert f(P, 0, 128, 256, None, P, 1, P + 2, P, P, P, None) == MISAL


def test_workspace_size_macros_match_the_binding(tmp_path):
    """The workspace sizes the header defines (compiled with gcc) equal the
    binding's helpers, over shapes with ragged m and k."""
    from nvfp4_block_scaled_04_amd import ops
    import subprocess
    shapes = [(1, 1, 16), (8, 512, 8192), (3, 130, 1040), (4, 200, 96)]
    src = tmp_path / "ws.c"
    lines = ['#include <stdio.h>', '#include <stdint.h>', '#include "nvfp4.h"', "int main(void) {"]
    for b, m, k in shapes:
        lines.append(f'  printf("%lld %lld\\n", (long long)NVFP4_BATCHED_WS_BYTES({b}, {m}, {k}), '
                     f'(long long)NVFP4_SILU_WS_BYTES({b}, {m}, {k}));')
    lines += ["  return 0;", "}"]
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "ws"
    inc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    subprocess.run(["gcc", "-I", inc, str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    for (b, m, k), line in zip(shapes, out):
        got = [int(v) for v in line.split()]
        assert got == [ops.batched_ws_bytes(b, m, k), ops.silu_ws_bytes(b, m, k)], (b, m, k, got)


def test_prepared_lora_size_macro_matches_the_binding(tmp_path):
    """NVFP4_LORA_PREPARED_ELEMS (compiled with gcc) equals the binding's
    lora_prepared_numel, with k a multiple of 32 and not."""
    from nvfp4_block_scaled_04_amd import ops
    import subprocess
    shapes = [(32, 16), (32, 3072), (64, 1040), (96, 272), (128, 8192)]
    src = tmp_path / "lp.c"
    lines = ['#include <stdio.h>', '#include <stdint.h>', '#include "nvfp4.h"', "int main(void) {"]
    for r, k in shapes:
        lines.append(f'  printf("%lld\\n", (long long)NVFP4_LORA_PREPARED_ELEMS({r}, {k}));')
    lines += ["  return 0;", "}"]
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "lp"
    inc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    subprocess.run(["gcc", "-I", inc, str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()
    assert [int(v) for v in out] == [ops.lora_prepared_numel(r, k) for r, k in shapes]
    assert ops.lora_prepared_numel(32, 1040) == 2 * 32 * 1056
