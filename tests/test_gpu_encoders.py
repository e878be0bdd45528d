"""GPU sweep of the two hardware encoders against the oracle.

The quantize kernels encode the block scale with the gfx950 fp8 convert
(after clamping to 448) and the elements with the FP4 convert; random data
and the worked example leave their rounding at exact midpoints to chance.
Here the inputs are built so that the values reaching each encoder sit on
every rounding boundary and one fp32 ulp either side of it, and the FP4 and
scale bytes of the whole tensor must equal the oracle's bit for bit
(TensorRT-LLM NVFP4LinearMethod.create_weights: FP8 per-block scaling
factors; flashinfer mm_nvfp4_svdquant, parameter a_sf: ue4m3).

The global scale is STATIC and 1.0, so the value the scale encoder sees is
fp32(bamax / 6) for a block whose largest magnitude is bamax.  Inputs are fp32.

* Scale encoder: for every pair of neighbouring ue4m3 codes (subnormals
  m * 2^-9 included) the midpoint, its two fp32 neighbours and the lower
  code's own value; the region around and above the largest code (448, the
  converter's overflow edge at 464, far above); zero and the values around
  2^-10 (half of the smallest subnormal).  Each such value is one block: its
  first element is +-bamax (bamax found by search so that fp32(bamax / 6)
  is exactly the target), the other 15 uniform in [-bamax, bamax].
* Element encoder: for every nonzero scale code, blocks with bamax =
  6 * dec(s) (the scale is then exactly s) whose other elements x are found
  by search so that fp32(x * fp32(1 / dec(s))) is each e2m1 tie (0.25,
  0.75, 1.25, 1.75, 2.5, 3.5, 5) or one fp32 ulp either side, with both
  signs, plus -0 and a tiny negative value (codes 0x8).  Where 1 / dec(s)
  is a power of two every such value is reached exactly; for the other
  codes the product's fp32 grid may skip one, and the nearest reachable
  value is taken.

The search below only steers the inputs; the expected bytes come from the
oracle."""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import canary, np_bits, say

pytestmark = pytest.mark.gpu

F = np.float32
TIES = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from nvfp4_block_scaled_04_amd import ops as _ops
    return _ops


def ue4m3_value(c):
    """Value of ue4m3 code c from the e4m3 bit layout (bias 7, subnormals m * 2^-9)."""
    e, m = c >> 3, c & 7
    return F(m * 2.0 ** -9) if e == 0 else F((1 + m / 8) * 2.0 ** (e - 7))


def nxt(v, d):
    return np.nextafter(F(v), F(d))


def preimage(target, f, guess, exact=True):
    """An fp32 x within 16 ulps of guess with f(x) == target exactly (f is
    monotone); if there is none: None, or with exact=False the candidate
    whose f(x) is nearest the target."""
    cands = [F(guess)]
    up = dn = F(guess)
    for _ in range(16):
        up, dn = nxt(up, np.inf), nxt(dn, -np.inf)
        cands += [up, dn]
    cands = [x for x in cands if np.isfinite(x)]
    for x in cands:
        if f(x) == F(target):
            return x
    if exact:
        return None
    return min(cands, key=lambda x: abs(np.float64(f(x)) - np.float64(target)))


def div6(x):
    """fp32(x / 6): the value the scale encoder sees at global scale 1."""
    return F(F(x) / F(6.0))


def scale_targets():
    vals = [ue4m3_value(c) for c in range(127)]
    out = []
    for c in range(126):
        mid = F((np.float64(vals[c]) + np.float64(vals[c + 1])) / 2)
        out += [vals[c], nxt(mid, 0), mid, nxt(mid, np.inf)]
    out += [vals[126], nxt(448, 0), nxt(448, np.inf), F(456), F(463.9), nxt(464, 0), F(464), nxt(464, np.inf),
            F(480), F(1000.0), F(2.0 ** 100),
            F(2.0 ** -11), nxt(2.0 ** -10, 0), F(2.0 ** -10), nxt(2.0 ** -10, np.inf), F(2.0 ** -30)]
    return out


def build_blocks(seed=0):
    """The sweep's blocks [n, 16] fp32, and the (code, x * r) pairs of the
    element sweep that hit their target exactly."""
    rng = np.random.default_rng(seed)
    blocks = []
    exact_hits = set()
    # scale encoder sweep
    for i, t in enumerate(scale_targets()):
        b = preimage(t, div6, np.float64(t) * 6.0)
        assert b is not None and div6(b) == t, f"no fp32 bamax gives block scale value {t!r}"
        blk = (rng.uniform(-1.0, 1.0, 16) * np.float64(b)).astype(F)
        blk = np.clip(blk, -b, b)
        blk[0] = b if i % 2 == 0 else -b
        blocks.append(blk)
    # element encoder sweep, every nonzero scale code
    for c in range(1, 127):
        dec = ue4m3_value(c)
        bamax = F(6.0 * np.float64(dec))
        assert np.float64(bamax) == 6.0 * np.float64(dec)
        r = F(F(1.0) / dec)   # the element factor gs / dec(s) at gs = 1

        def mul(x, r=r):
            return F(F(x) * r)

        pow2 = (c & 7) == 0 or c in (1, 2, 4)   # dec(s) a power of two
        vals = []
        for t in TIES:
            for v in (nxt(t, 0), F(t), nxt(t, np.inf)):
                x = preimage(v, mul, np.float64(v) / np.float64(r), exact=pow2)
                assert x is not None, f"code {c}: no fp32 x gives x * r = {v!r}"
                if mul(x) == v:
                    exact_hits.add((c, float(v)))
                vals += [x, -x]
        vals += [F(-0.0), F(-np.float64(dec) * 2.0 ** -8)]
        for j in range(0, len(vals), 15):
            chunk = vals[j:j + 15]
            blk = np.zeros(16, F)
            blk[0] = bamax if (c + j) % 2 == 0 else -bamax
            blk[1:1 + len(chunk)] = chunk
            blocks.append(blk)
    return np.stack(blocks), exact_hits


def test_encoders_at_every_rounding_boundary(ops):
    blocks, hits = build_blocks()
    # every tie and both neighbours reached exactly on at least the 18
    # power-of-two scale codes
    for t in TIES:
        for v in (nxt(t, 0), F(t), nxt(t, np.inf)):
            assert sum(1 for c, w in hits if w == float(v)) >= 18, v
    k = 256
    per_row = k // 16
    rows = -(-len(blocks) // per_row)
    x = np.zeros((rows * per_row, 16), F)
    x[:len(blocks)] = blocks
    x = x.reshape(rows, k)
    assert np.all(np.isfinite(x))
    say("encoder sweep", x.shape, "blocks", len(blocks))
    xd = torch.from_numpy(x).to("cuda")
    gs_d = torch.tensor([1.0], dtype=torch.float32, device="cuda")
    o4 = canary((rows, k // 2))
    osf = canary((ops.sf_size(rows, k),))
    ops.nvfp4_quantize(xd, gs_d, ops.GS_STATIC, out_fp4=o4, out_sf=osf)
    torch.cuda.synchronize()
    q, sf, _ = O.quantize(x, gs=np.array([1.0], F), gs_mode=O.STATIC)
    # coverage: every ue4m3 code 0..0x7E appears as a block scale
    codes = set(np.unique(sf).tolist())
    assert set(range(0x7F)) <= codes, sorted(set(range(0x7F)) - codes)[:8]
    gq, gsf = np_bits(o4), np_bits(osf)
    bad = np.argwhere(gsf != sf)
    assert len(bad) == 0, f"{len(bad)} scale bytes differ, first at {bad[:3].tolist()}"
    bad = np.argwhere(gq != q)
    assert len(bad) == 0, f"{len(bad)} FP4 bytes differ, first at {bad[:3].tolist()}"
