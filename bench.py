"""Benchmark of the NVFP4 hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input that
is already resident in HBM: NVFP4 quantization of the bf16 activation with a
dynamic global scale (the amax pass with its partial maxima in a workspace,
then the quantize pass, which also writes gs and alpha = 1/(gs_a*gs_w); one
launch for small activations), and the block-scaled GEMM to bf16.  Weights
are quantized once before timing (same kernels, untimed).  Each step owns
its quantized outputs.  The K timed steps run as two HIP graphs replayed
back to back -- the K quantizations, then the K GEMMs -- between three HIP
events on the kernels' stream, after at least 30 ms of untimed replays of
the same graphs (the clock the chip holds under this load) and a cache
flush; the step time, the
quantize share and the GEMM's average duration all come from those events.
The same steps interleaved in one graph, and launched eagerly, are reported
for reference.

Default workload: the large prefill linear, activation [8192, 5120] bf16
(0.5% outlier channels x30) against a [16384, 5120] weight, output [8192,
16384] bf16.  Other workloads (--workload dense|decode|moe|svdquant|tiny)
are for development measurements.

Prints one JSON line.  `value` is whole-step GEMM throughput (GEMM flops per
step / step time); the quantize and GEMM kernels are also reported on their
own (the quantize pass and the whole dynamic call timed back to back over
every activation copy, next to a plain device copy for reference), and
`roofline` covers the dominant kernel (the GEMM), timed with HIP events on
the stream it runs on.  For the prefill and dense workloads, `library` times
the vendor library's GEMMs (hipBLASLt through torch: bf16, fp8, MXFP4) beside
this library's on the same shape and data, for comparison only.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
SETTLE_MS = 30.0               # untimed back-to-back replays before a timed region
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 MFMA, TFLOP/s
MFMA_FP4_PEAK_TFLOPS = 10100.0  # MI355X dense fp4 (and fp6) MFMA, TFLOP/s


def sf_size(rows, k):
    return (rows + 127) // 128 * 128 * ((k // 16 + 3) // 4 * 4)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="prefill",
                   choices=["prefill", "dense", "decode", "moe", "svdquant", "tiny"])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-library", action="store_true",
                   help="skip the comparison with the vendor library's GEMMs (prefill and dense only)")
    p.add_argument("--rotate", type=int, default=0,
                   help="activation copies cycled per step (0: enough to exceed 512 MB)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a plain elementwise copy of 256 MiB (fp32 negate, 256 MiB read + "
                        "256 MiB written) so that HBM byte counters can be scaled by a kernel of known traffic")
    return p.parse_args()


class Workload:
    """Device-resident inputs, the step closures and their algorithmic work.

    make_steps(acts, K) gives K (quantize, gemm) closure pairs; step i reads
    activation copy i % len(acts) and owns its quantized outputs, which its
    GEMM consumes (so the K quantizations and the K GEMMs can run as two
    graphs and every GEMM still reads its own step's operands).  quant(a,
    mode) quantizes into one shared output set (the pass measurements)."""


def _rotation(nbytes):
    """Copies of an nbytes buffer needed to exceed 512 MiB (twice the 256 MB
    Infinity Cache), so reads cycling through them come from HBM."""
    return max(1, -(-512 * 2 ** 20 // nbytes))


def build_workload(name, ops, synth, torch):
    w = Workload()
    w.gemm_kernel = "k_gemm (block-scaled NVFP4 GEMM)"
    w.hbm_bound = False
    w.w4a16 = None
    w.linear_small = None
    w.lora_down = w.lora_down_unprepared = None
    w.swiglu = None
    w.mx = None
    w.library = None
    w.quant_3launch = None
    w.quant_3launch_desc = ("without the workspace: amax pass, a one-workgroup finish kernel, then the "
                            "quantize pass (which writes alpha)")
    dev = "cuda"
    if name in ("prefill", "dense", "decode", "tiny"):
        if name == "prefill":
            d = synth.prefill()
            a_cpu, w_cpu = d.a, d.w
            w.desc = "prefill linear 8192x16384x5120: bf16 activation -> dynamic NVFP4 quantize -> block-scaled GEMM -> bf16"
        elif name == "dense":
            d, _ = synth.dense()
            a_cpu, w_cpu = d.a, d.w
            w.desc = "dense linear 2048x4096x4096: bf16 activation -> dynamic NVFP4 quantize -> block-scaled GEMM -> bf16"
        elif name == "decode":
            d, a16 = synth.dense()
            a_cpu, w_cpu = a16, d.w
            w.desc = ("decode linear 16x4096x4096: bf16 activation -> dynamic NVFP4 quantize -> block-scaled GEMM "
                      "-> bf16; every step reads its own weight copy (cold)")
        else:
            d = synth.tiny()
            a_cpu, w_cpu = d.a, d.w
            w.desc = "tiny 128x256x256: fp32 activation -> dynamic NVFP4 quantize -> block-scaled GEMM -> bf16"
        m, k = a_cpu.shape
        n = w_cpu.shape[0]
        fw0, sfw0, gsw = ops.nvfp4_quantize(w_cpu.to(dev))
        w.hbm_bound = name == "decode"   # 16 rows: the weight read bounds the GEMM
        w_bytes = n * k // 2 + sf_size(n, k)
        # decode: enough weight copies that the steps' weight reads come from HBM
        w.n_wcopies = _rotation(w_bytes) if w.hbm_bound else 1
        weights = [(fw0, sfw0)] + [(fw0.clone(), sfw0.clone()) for _ in range(w.n_wcopies - 1)]
        esz = a_cpu.element_size()
        w.rotate_hint = _rotation(m * k * esz)
        w.a_cpu, w.w_cpu = a_cpu, w_cpu
        w.m, w.n, w.k = m, n, k
        w.flops = 2.0 * m * n * k
        w.q_bytes = m * k * esz + m * k // 2 + sf_size(m, k)     # quantize pass
        w.amax_bytes = m * k * esz                                 # amax pass
        w.gemm_bytes = m * k // 2 + sf_size(m, k) + w_bytes + 2 * m * n
        out = torch.empty(m, n, dtype=torch.bfloat16, device=dev)
        ws = ops.quantize_workspace(dev)
        fa = torch.empty(m, k // 2, dtype=torch.uint8, device=dev)
        sfa = torch.empty(sf_size(m, k), dtype=torch.uint8, device=dev)
        gsa = torch.zeros(1, dtype=torch.float32, device=dev)
        alpha = torch.empty(1, dtype=torch.float32, device=dev)

        def quant(a, mode=ops.GS_DYNAMIC):
            # the step's call: with the workspace; DYNAMIC also writes alpha
            ops.nvfp4_quantize_ws(a, ws, gsa, mode, gs_other=gsw, alpha=alpha, out_fp4=fa, out_sf=sfa)

        def quant_3launch(a):
            ops.nvfp4_quantize_alpha(a, gsw, gsa, ops.GS_DYNAMIC, out_fp4=fa, out_sf=sfa, alpha=alpha)

        def make_steps(acts, K):
            steps = []
            for i in range(K):
                o = (torch.empty(m, k // 2, dtype=torch.uint8, device=dev),
                     torch.empty(sf_size(m, k), dtype=torch.uint8, device=dev),
                     torch.zeros(1, dtype=torch.float32, device=dev), torch.empty(1, dtype=torch.float32, device=dev))
                fw, sfw = weights[i % len(weights)]
                a = acts[i % len(acts)]

                def pre(a=a, o=o):
                    ops.nvfp4_quantize_ws(a, ws, o[2], ops.GS_DYNAMIC, gs_other=gsw, alpha=o[3],
                                          out_fp4=o[0], out_sf=o[1])

                def gemm(o=o, fw=fw, sfw=sfw):
                    ops.nvfp4_gemm(o[0], fw, o[1], sfw, o[3], out=out)
                steps.append((pre, gemm))
            return steps

        w.make_acts = lambda n_copies: [a_cpu.to(dev) for _ in range(n_copies)]
        w.make_steps, w.quant, w.quant_3launch = make_steps, quant, quant_3launch
        w.gemm0 = lambda: ops.nvfp4_gemm(fa, fw0, sfa, sfw0, alpha, out=out)
        w.cfg = {"m": m, "n": n, "k": k}
        if name == "decode":
            # weight-only form: the bf16 activation against the NVFP4 weight,
            # no activation quantization (alpha = 1 / the weight's gs); step i
            # reads weight copy i
            alpha_w = ops.nvfp4_alpha(torch.ones(1, dtype=torch.float32, device=dev), gsw)
            out_w = torch.empty(m, n, dtype=torch.bfloat16, device=dev)
            w.w4a16 = lambda a, i: ops.nvfp4_gemm_w4a16(a, weights[i % len(weights)][0], weights[i % len(weights)][1],
                                                        alpha_w, out=out_w)
            w.w4a16_bytes = w_bytes + m * k * 2 + 2 * m * n
            # the whole step in one launch (nvfp4_linear_small: the dynamic
            # quantization on chip, then the GEMM); step i reads weight copy i
            out_ls = torch.empty(m, n, dtype=torch.bfloat16, device=dev)
            gs_ls = torch.zeros(1, dtype=torch.float32, device=dev)
            w.linear_small = lambda a, i: ops.nvfp4_linear_small(a, weights[i % len(weights)][0],
                                                                 weights[i % len(weights)][1], gsw, out=out_ls,
                                                                 gs_out=gs_ls)
        w.cpu_sample = lambda O, np: cpu_baseline_dense(O, np, a_cpu, w_cpu, synth)
        if name in ("prefill", "dense"):
            w.mx = lambda acts: mx_setting(ops, torch, acts, w_cpu, dev)
            w.library = lambda acts: library_comparison(ops, torch, w, acts[0], w_cpu, dev)
        return w

    if name == "moe":
        mo = synth.moe()
        E, m, h, n = mo.e, mo.m, mo.h, mo.n
        fws, sfws, gsws = [], [], []
        for e in range(E):
            f_, s_, g_ = ops.nvfp4_quantize(mo.w[e].to(dev))
            fws.append(f_); sfws.append(s_); gsws.append(g_)
        fw = torch.stack(fws); sfw = torch.stack(sfws); gsw = torch.cat(gsws)
        del fws, sfws
        mask = mo.mask.to(dev)
        valid = int(mo.mask.clamp(0, m).sum())
        fa = torch.empty(E, m, h // 2, dtype=torch.uint8, device=dev)
        sfa = torch.empty(E, sf_size(m, h), dtype=torch.uint8, device=dev)
        gsa = torch.zeros(E, dtype=torch.float32, device=dev)
        alpha = torch.empty(E, dtype=torch.float32, device=dev)
        out = torch.empty(E, m, n, dtype=torch.bfloat16, device=dev)
        gws = ops.gemm_workspace(dev)   # partial tiles of the split-tail schedule
        qws = ops.silu_workspace(E, m, h, dev)   # the silu quantize's partial maxima and h

        def quant(x, mode=ops.GS_DYNAMIC):
            # the step's call: with the workspace; also writes alpha
            ops.silu_mul_nvfp4_quantize_ws(x, qws, mask, gsa, mode, gs_other=gsw, alpha=alpha,
                                           out_fp4=fa, out_sf=sfa)

        def quant_3launch(x):
            # without the workspace (amax, finish, quantize), then alpha in its own launch
            ops.silu_mul_nvfp4_quantize(x, mask, gsa, ops.GS_DYNAMIC, out_fp4=fa, out_sf=sfa)
            ops.nvfp4_alpha(gsa, gsw, out=alpha)

        def make_steps(acts, K):
            steps = []
            for i in range(K):
                o = (torch.empty(E, m, h // 2, dtype=torch.uint8, device=dev),
                     torch.empty(E, sf_size(m, h), dtype=torch.uint8, device=dev),
                     torch.zeros(E, dtype=torch.float32, device=dev), torch.empty(E, dtype=torch.float32, device=dev))
                x = acts[i % len(acts)]

                def pre(x=x, o=o):
                    # amax pass, then the quantize pass, which also writes gs and alpha
                    ops.silu_mul_nvfp4_quantize_ws(x, qws, mask, o[2], ops.GS_DYNAMIC, gs_other=gsw, alpha=o[3],
                                                   out_fp4=o[0], out_sf=o[1])

                def gemm(o=o):
                    ops.nvfp4_gemm_grouped_masked(o[0], fw, o[1], sfw, o[3], mask, out=out, workspace=gws)
                steps.append((pre, gemm))
            return steps

        w.desc = ("Llama4-style routed experts: E=8 gate|up [512,16384] bf16, valid rows "
                  f"{mo.mask.tolist()} -> fused silu_and_mul + NVFP4 quantize -> grouped masked GEMM vs [8,5120,8192] "
                  "(split-tail schedule with a workspace)")
        w.rotate_hint = _rotation(mo.x.numel() * 2)
        w.make_acts = lambda n_copies: [mo.x.to(dev) for _ in range(n_copies)]
        w.make_steps, w.quant, w.quant_3launch = make_steps, quant, quant_3launch
        w.quant_3launch_desc = ("without the workspace: amax pass, a finish kernel, the quantize pass, then "
                                "nvfp4_alpha (four launches)")
        w.dynamic_call_desc = ("the step's call: the amax pass evaluates silu once and stores h and the partial "
                               "maxima in the workspace, then a bf16 quantize pass over h reduces the partials "
                               "and writes gs and alpha; bytes = g|u read + h written and read back + outputs, "
                               "the same total as reading g|u in both passes")
        w.gemm0 = lambda: ops.nvfp4_gemm_grouped_masked(fa, fw, sfa, sfw, alpha, mask, out=out, workspace=gws)
        w.gemm_kernel = ("k_gemm split-tail schedule + k_gemm_fixup (block-scaled NVFP4 grouped GEMM; the two "
                         "launches together)")
        w.n_wcopies = 1
        w.flops = 2.0 * n * h * valid
        w.q_bytes = valid * 2 * h * 2 + E * m * h // 2 + E * sf_size(m, h)
        w.amax_bytes = valid * 2 * h * 2
        w.gemm_bytes = valid * h // 2 + E * sf_size(m, h) + E * n * h // 2 + E * sf_size(n, h) + 2 * valid * n
        w.m, w.n, w.k = valid, n, h
        w.cfg = {"experts": E, "m_max": m, "valid_rows": mo.mask.tolist(), "n": n, "k": h}
        w.cpu_sample = lambda O, np: cpu_baseline_moe(O, np, mo, synth)
        w.swiglu = lambda: swiglu_front_half(ops, synth, torch, mo.mask, dev)
        return w

    if name == "svdquant":
        s = synth.svdquant()
        m, n, k, r = s.m, s.n, s.k, s.r
        fw, sfw, gsw = ops.nvfp4_quantize(s.w.to(dev))
        x0 = s.x.to(dev)
        pqs = s.pqs.to(dev)
        # calibrated (static) input scale, as the smoothing pipeline uses a fixed
        # alpha to pre-divide l1; calibration = one dynamic pass, untimed
        _, _, gsa = ops.nvfp4_quantize(x0, pre_quant_scale=pqs)
        alpha = ops.nvfp4_alpha(gsa, gsw)
        al = float(alpha.item())
        l2 = s.l2.to(torch.bfloat16).to(dev)
        # the caller's LoRA-up weight with 1/alpha folded in (the fused
        # epilogue's alpha * acc restores the unscaled term)
        l1 = (s.l1_raw / al).to(torch.bfloat16).to(dev)
        bias = s.bias.to(dev)
        fa = torch.empty(m, k // 2, dtype=torch.uint8, device=dev)
        sfa = torch.empty(sf_size(m, k), dtype=torch.uint8, device=dev)
        d = torch.empty(m, r, dtype=torch.bfloat16, device=dev)
        out = torch.empty(m, n, dtype=torch.bfloat16, device=dev)

        def quant(x, mode=ops.GS_STATIC):
            ops.nvfp4_quantize(x, gsa, mode, pre_quant_scale=pqs, out_fp4=fa, out_sf=sfa)

        # the LoRA-down weight with the smoothing folded in, split into exact
        # bf16 halves in the fused kernel's operand order: a weight transform,
        # done once like the weight quantization
        wl = ops.nvfp4_lora_down_prepare(pqs, l2)

        def lora_down(x):
            # smooth quantize and the LoRA-down projection d, one read of x
            ops.nvfp4_quantize_lora_down_prepared(x, pqs, wl, r, gsa, ops.GS_STATIC, out_fp4=fa, out_sf=sfa, d=d)

        def lora_down_unprepared(x):
            ops.nvfp4_quantize_lora_down(x, pqs, l2, gsa, ops.GS_STATIC, out_fp4=fa, out_sf=sfa, d=d)

        def make_steps(acts, K):
            steps = []
            for i in range(K):
                o = (torch.empty(m, k // 2, dtype=torch.uint8, device=dev),
                     torch.empty(sf_size(m, k), dtype=torch.uint8, device=dev),
                     torch.empty(m, r, dtype=torch.bfloat16, device=dev))
                x = acts[i % len(acts)]

                def pre(x=x, o=o):
                    ops.nvfp4_quantize_lora_down_prepared(x, pqs, wl, r, gsa, ops.GS_STATIC, out_fp4=o[0],
                                                          out_sf=o[1], d=o[2])

                def gemm(o=o):
                    ops.nvfp4_gemm_svdquant(o[0], fw, o[1], sfw, alpha, o[2], l1, bias=bias, out=out)
                steps.append((pre, gemm))
            return steps

        w.lora_down, w.lora_down_unprepared = lora_down, lora_down_unprepared
        w.lora_down_bytes = m * k * 2 + k * 2 + 2 * ops.lora_prepared_numel(r, k) + m * k // 2 + sf_size(m, k) \
            + 2 * m * r
        w.lora_down_unprepared_bytes = m * k * 2 + k * 2 + r * k * 2 + m * k // 2 + sf_size(m, k) + 2 * m * r
        w.desc = ("SVDQuant linear 4096x3072x3072, r=32: smooth NVFP4 quantize (static gs) with the LoRA-down "
                  "projection fused (weight pqs * L2 prepared once) -> fused GEMM + LoRA-up + bias")
        w.rotate_hint = _rotation(m * k * 2)
        w.make_acts = lambda n_copies: [s.x.to(dev) for _ in range(n_copies)]
        w.make_steps, w.quant = make_steps, quant
        w.gemm0 = lambda: ops.nvfp4_gemm_svdquant(fa, fw, sfa, sfw, alpha, d, l1, bias=bias, out=out)
        w.n_wcopies = 1
        w.flops = 2.0 * m * n * k + 2.0 * m * n * r
        w.q_bytes = m * k * 2 + k * 2 + m * k // 2 + sf_size(m, k)
        w.amax_bytes = 0
        w.gemm_bytes = m * k // 2 + sf_size(m, k) + n * k // 2 + sf_size(n, k) + 2 * m * n + 2 * (m + n) * r + 2 * n
        w.m, w.n, w.k = m, n, k
        w.cfg = {"m": m, "n": n, "k": k, "r": r}
        w.cpu_sample = lambda O, np: cpu_baseline_svdquant(O, np, s, synth)
        return w
    raise ValueError(name)


def mx_setting(ops, torch, acts, w_cpu, dev):
    """The same linear in the MX setting (32-element blocks, ue8m0 scales):
    the weight quantized once (untimed); the activation quantize pass over
    every activation copy and the GEMM back to back, each in a HIP graph."""
    m, k = acts[0].shape
    n = w_cpu.shape[0]
    fw, sfw = ops.mxfp4_quantize(w_cpu.to(dev))
    fa = torch.empty(m, k // 2, dtype=torch.uint8, device=dev)
    sfa = torch.empty(ops.sf_size_mx(m, k), dtype=torch.uint8, device=dev)
    out = torch.empty(m, n, dtype=torch.bfloat16, device=dev)
    for a in acts:
        ops.mxfp4_quantize(a, out_fp4=fa, out_sf=sfa)
    ops.mxfp4_gemm(fa, fw, sfa, sfw, out=out)
    torch.cuda.synchronize()
    g_q = capture(torch, lambda: [ops.mxfp4_quantize(a, out_fp4=fa, out_sf=sfa) for a in acts])
    q_ms = time_graph(torch, g_q) / len(acts)
    del g_q
    reps = max(1, len(acts))
    g_g = capture(torch, lambda: [ops.mxfp4_gemm(fa, fw, sfa, sfw, out=out) for _ in range(reps)])
    g_ms = time_graph(torch, g_g) / reps
    del g_g
    q_bytes = m * k * acts[0].element_size() + m * k // 2 + ops.sf_size_mx(m, k)
    flops = 2.0 * m * n * k
    tf = flops / (g_ms * 1e-3) / 1e12
    q_gbs = q_bytes / (q_ms * 1e-3) / 1e9
    return {
        "kernels": "k_quantize_mx (one pass, no global scale) and k_gemm_mx (v_mfma_scale_f32_32x32x64, FP4 operands)",
        "quantize_pass_ms": round(q_ms, 4), "quantize_gbs": round(q_gbs, 1),
        "quantize_frac_hbm": round(q_gbs / HBM_PEAK_GBS, 4), "quantize_bytes": q_bytes,
        "gemm_ms": round(g_ms, 4), "gemm_tflops": round(tf, 2),
        "gemm_frac_fp4_mfma_peak": round(tf / MFMA_FP4_PEAK_TFLOPS, 4),
        "step_ms": round(q_ms + g_ms, 4),
        "step_tflops": round(flops / ((q_ms + g_ms) * 1e-3) / 1e12, 2),
    }


def swiglu_front_half(ops, synth, torch, mask_cpu, dev):
    """The experts' step before the moe workload's: hidden states [8,512,5120]
    (NVFP4, quantized once, untimed) against gate|up weights [8,16384,5120],
    with silu_and_mul + NVFP4 quantize of the output (static global scale,
    calibrated by one untimed dynamic pass).  Times the one-launch fused path
    and the two-launch path (grouped GEMM to bf16 h, then the silu quantize),
    each back to back in a HIP graph."""
    sw = synth.moe_swiglu(mask=mask_cpu)
    E, m, H, hid = sw.e, sw.m, sw.h, sw.hidden
    mask = sw.mask.to(dev)
    valid = int(sw.mask.clamp(0, m).sum())
    fx, sfx, gsx = ops.nvfp4_quantize_masked_batched(sw.x.to(dev), mask)
    fws, sfws, gsws = [], [], []
    for e in range(E):
        f_, s_, g_ = ops.nvfp4_quantize(sw.w[e].to(dev))
        fws.append(f_); sfws.append(s_); gsws.append(g_)
    del sw
    fw = torch.stack(fws); sfw = torch.stack(sfws); gsw = torch.cat(gsws)
    del fws, sfws
    alpha = ops.nvfp4_alpha(gsx, gsw)
    h = ops.nvfp4_gemm_grouped_masked(fx, fw, sfx, sfw, alpha, mask)
    fq = torch.empty(E, m, H // 2, dtype=torch.uint8, device=dev)
    sfq = torch.empty(E, sf_size(m, H), dtype=torch.uint8, device=dev)
    _, _, gsh = ops.silu_mul_nvfp4_quantize(h, mask, out_fp4=fq, out_sf=sfq)   # calibration
    torch.cuda.synchronize()
    reps = 4

    def fused():
        ops.nvfp4_gemm_grouped_masked_silu_quantize(fx, fw, sfx, sfw, alpha, mask, gsh, out_fp4=fq, out_sf=sfq)

    def two_launch():
        ops.nvfp4_gemm_grouped_masked(fx, fw, sfx, sfw, alpha, mask, out=h)
        ops.silu_mul_nvfp4_quantize(h, mask, gsh, ops.GS_STATIC, out_fp4=fq, out_sf=sfq)

    def gemm_only():
        ops.nvfp4_gemm_grouped_masked(fx, fw, sfx, sfw, alpha, mask, out=h)

    for fn in (fused, two_launch):
        fn()
    torch.cuda.synchronize()
    # the three graphs timed in turn, five rounds, best of each (the clock
    # drifts with the chip's power state over a run)
    graphs = {name: capture(torch, lambda fn=fn: [fn() for _ in range(reps)])
              for name, fn in (("fused", fused), ("two_launch", two_launch), ("gemm_only", gemm_only))}
    times = {name: time_graph(torch, g, reps=1) / reps for name, g in graphs.items()}
    for _ in range(4):
        for name, g in graphs.items():
            times[name] = min(times[name], time_graph(torch, g, reps=1) / reps)
    del graphs
    flops = 2.0 * valid * 2 * H * hid
    tf = flops / (times["fused"] * 1e-3) / 1e12
    return {
        "kernel": "k_gemm with the silu_and_mul + NVFP4 quantize epilogue (grouped masked gate_up GEMM)",
        "shape": f"E={E} x {m} rows (valid {mask_cpu.tolist()}) x gate|up {2 * H} x hidden {hid}",
        "fused_ms": round(times["fused"], 5),
        "two_launch_ms": round(times["two_launch"], 5),
        "gemm_to_bf16_ms": round(times["gemm_only"], 5),
        "fused_tflops": round(tf, 2),
        "fused_frac_f16_mfma_peak": round(tf / MFMA_F16_PEAK_TFLOPS, 4),
        "flops_per_launch": flops,
        "bf16_h_bytes_not_written_or_read": 2 * 2 * valid * 2 * H,
    }


def _sized_sample(run, m, target_s):
    """Rows of a bounded oracle sample: a 64-row probe sizes the slice so
    that the timed run takes about target_s seconds (at most m rows)."""
    rows = min(64, m)
    dt = run(rows)
    if dt < target_s / 2 and rows < m:
        rows = int(min(m, max(rows, 64 * round(rows * target_s / dt / 64))))
        dt = run(rows)
    return rows, dt


def cpu_baseline_dense(O, np, a_cpu, w_cpu, synth, target_s=20.0):
    """The oracle on a bounded sample of the same step: the weight is
    quantized once, untimed (offline in the GPU step too); the timed part
    quantizes a slice of activation rows (dynamic gs over the slice) and
    computes the GEMM for those rows."""
    wq = O.quantize(synth.bits(w_cpu))          # untimed, like the GPU's weights
    m, k = a_cpu.shape
    n = w_cpu.shape[0]

    def run(rows):
        a = synth.bits(a_cpu[:rows])
        t0 = time.perf_counter()
        qa, sa, ga = O.quantize(a)
        alpha = np.float32(1.0) / (ga[0] * wq[2][0])
        O.gemm_rows(qa, wq[0], sa, wq[1], alpha, rows, n, k)
        return time.perf_counter() - t0

    rows, dt = _sized_sample(run, m, target_s)
    flops = 2.0 * rows * n * k
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": O.num_threads(),
        "kind": "oracle",
        "sample": f"{rows} of {m} activation rows: oracle dynamic quantize of those rows + "
                  f"oracle dequant-GEMM {rows}x{n}x{k} (fp64 accumulation), {dt:.2f} s wall",
    }


def cpu_baseline_moe(O, np, mo, synth, target_s=20.0):
    """The routed-expert step's oracle on a bounded sample: the first valid
    rows of the experts in order (expert 0's, then expert 1's, ...), their
    silu_and_mul quantization (dynamic gs per expert over its sampled rows)
    and their rows of the expert's GEMM; the experts' weights are quantized
    once, untimed.  Every valid row costs the same, so the rate stands for
    the step's."""
    valid = [int(v) for v in mo.mask.clamp(0, mo.m)]
    n, h = mo.n, mo.h
    wq = {}

    def take(rows):  # (expert, rows of it) covering `rows` valid rows
        out = []
        for e, v in enumerate(valid):
            if rows <= 0:
                break
            if v:
                out.append((e, min(v, rows)))
                rows -= min(v, rows)
        return out

    def run(rows):
        parts = take(rows)
        for e, _ in parts:
            if e not in wq:
                wq[e] = O.quantize(synth.bits(mo.w[e]))
        xs = [synth.bits(mo.x[e, :r]) for e, r in parts]
        t0 = time.perf_counter()
        for (e, r), x in zip(parts, xs):
            qa, sa, ga = O.quantize(x, prologue=O.PRO_SILU)
            alpha = np.float32(1.0) / (ga[0] * wq[e][2][0])
            O.gemm_rows(qa, wq[e][0], sa, wq[e][1], alpha, r, n, h)
        return time.perf_counter() - t0

    rows, dt = _sized_sample(run, sum(valid), target_s)
    used = take(rows)
    return {
        "value": 2.0 * rows * n * h / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": O.num_threads(),
        "kind": "oracle",
        "sample": f"{rows} of the {sum(valid)} valid rows (experts {[e for e, _ in used]}): oracle silu_and_mul "
                  f"NVFP4 quantize of those rows (dynamic gs per expert over them) + oracle dequant-GEMM {rows}"
                  f"x{n}x{h} (fp64 accumulation), {dt:.2f} s wall",
    }


def cpu_baseline_svdquant(O, np, s, synth, target_s=20.0):
    """The SVDQuant step's oracle on a bounded sample of activation rows:
    smooth quantize with a static gs (the oracle's global scale of the whole
    smoothed activation, untimed, as the step's is calibrated offline), the
    LoRA-down projection d (rounded to bf16 as the kernel stores it), and the
    GEMM rows with the LoRA-up term and bias; the weight is quantized once,
    untimed."""
    import torch
    wq = O.quantize(synth.bits(s.w))
    m, n, k = s.m, s.n, s.k
    pqs = synth.bits(s.pqs)
    amax = float((s.x.float() * s.pqs.float()).abs().max())   # bf16 x bf16: exact in fp32
    gs = np.float32(O.global_scale(amax))
    al = np.float32(1.0) / (gs * wq[2][0])
    l2 = synth.bits(s.l2.to(torch.bfloat16))
    l1 = synth.bits((s.l1_raw / float(al)).to(torch.bfloat16))
    bias = synth.bits(s.bias)

    def run(rows):
        x = synth.bits(s.x[:rows])
        t0 = time.perf_counter()
        qa, sa, _ = O.quantize(x, prologue=O.PRO_SMOOTH, pqs=pqs, gs=np.array([gs], np.float32),
                               gs_mode=O.STATIC)
        d = O.f64_to_bf16_via_f32(O.lora_down(x, pqs, l2))
        O.gemm_rows(qa, wq[0], sa, wq[1], al, rows, n, k, bias=bias, d=d, l1=l1)
        return time.perf_counter() - t0

    rows, dt = _sized_sample(run, m, target_s)
    return {
        "value": 2.0 * rows * n * (k + s.r) / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": O.num_threads(),
        "kind": "oracle",
        "sample": f"{rows} of {m} activation rows: oracle smooth quantize (static gs) + LoRA-down + "
                  f"dequant-GEMM {rows}x{n}x{k} with the rank-{s.r} LoRA-up and bias (fp64), {dt:.2f} s wall",
    }


# HBM traffic of the GEMM kernel per launch, from two rocprofv3 --pmc runs
# (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch) of this script, scaled by
# what the same counters read for a plain copy of known size
# (--copy-calibration: fetch x2.000, write x1.000).  A record is used only
# while the kernel sources hash to the value it was measured on.  The moe
# record is the split-tail schedule's two launches together (k_gemm and
# k_gemm_fixup), which the bench times as the GEMM.
MEASURED_TRAFFIC = {
    "prefill": {"sources_sha256": "23c0338bd9c1335a9e56f0ab048ab04c418de029918179069bdb4be93c069bc8"
                          "c7df1564c2660c5b6936c0d9acdfca2473753bd4dac2d6c405d89edece56c024"
                          "0b8ab37c346d4290d1fdb25793ffb74b674eb91941278aed19a6fa7e4e266b6a"
                          "54b19610b17c816426fc33a6ab2620605cb533220f8d2b2ba5de96d5cd0cf1df",
             "fetch_kib": 276682.1, "write_kib": 262144.0, "fetch_factor": 2.0, "write_factor": 1.0},
    "moe": {"sources_sha256": "23c0338bd9c1335a9e56f0ab048ab04c418de029918179069bdb4be93c069bc8"
                          "c7df1564c2660c5b6936c0d9acdfca2473753bd4dac2d6c405d89edece56c024"
                          "0b8ab37c346d4290d1fdb25793ffb74b674eb91941278aed19a6fa7e4e266b6a"
                          "54b19610b17c816426fc33a6ab2620605cb533220f8d2b2ba5de96d5cd0cf1df",
             "fetch_kib": 139075.5, "write_kib": 43510.0, "fetch_factor": 2.0, "write_factor": 1.0},
    "dense": {"sources_sha256": "23c0338bd9c1335a9e56f0ab048ab04c418de029918179069bdb4be93c069bc8"
                          "c7df1564c2660c5b6936c0d9acdfca2473753bd4dac2d6c405d89edece56c024"
                          "0b8ab37c346d4290d1fdb25793ffb74b674eb91941278aed19a6fa7e4e266b6a"
                          "54b19610b17c816426fc33a6ab2620605cb533220f8d2b2ba5de96d5cd0cf1df",
             "fetch_kib": 18604.5, "write_kib": 16384.0, "fetch_factor": 2.0, "write_factor": 1.0},
    "svdquant": {"sources_sha256": "23c0338bd9c1335a9e56f0ab048ab04c418de029918179069bdb4be93c069bc8"
                          "c7df1564c2660c5b6936c0d9acdfca2473753bd4dac2d6c405d89edece56c024"
                          "0b8ab37c346d4290d1fdb25793ffb74b674eb91941278aed19a6fa7e4e266b6a"
                          "54b19610b17c816426fc33a6ab2620605cb533220f8d2b2ba5de96d5cd0cf1df",
             "fetch_kib": 19884.5, "write_kib": 24577.9, "fetch_factor": 2.0, "write_factor": 1.0},
    "decode": {"sources_sha256": "23c0338bd9c1335a9e56f0ab048ab04c418de029918179069bdb4be93c069bc8"
                          "c7df1564c2660c5b6936c0d9acdfca2473753bd4dac2d6c405d89edece56c024"
                          "0b8ab37c346d4290d1fdb25793ffb74b674eb91941278aed19a6fa7e4e266b6a"
                          "54b19610b17c816426fc33a6ab2620605cb533220f8d2b2ba5de96d5cd0cf1df",
             "fetch_kib": 6383.1, "write_kib": 128.0, "fetch_factor": 2.0, "write_factor": 1.0},
}
GEMM_SOURCES = ("nvfp4_block_scaled_04_amd/csrc/gemm.hip", "nvfp4_block_scaled_04_amd/csrc/gemm_common.h",
                "nvfp4_block_scaled_04_amd/csrc/device_common.h", "nvfp4_block_scaled_04_amd/csrc/quant_block.h")


def library_comparison(ops, torch, w, a16, w_cpu, dev, rounds=3):
    """For comparison only: the vendor library's GEMMs (hipBLASLt through
    torch) on the same shape and the same data, timed beside this library's
    two GEMMs by the same method (reps launches back to back between HIP
    events on the current stream, best of `rounds` interleaved rounds):
      * bf16 x bf16 with the weight [n, k] (both operands K-contiguous, as in
        the NVFP4 GEMM) -- the unquantized linear, on the same fp16/bf16
        MFMA pipe the exact NVFP4 path runs on;
      * fp8 e4m3 with per-tensor scales;
      * MXFP4 (torch._scaled_mm with e2m1 operands and e8m0 block scales) on
        this library's MX-quantized operands; the scale bytes are handed over
        in this library's swizzled order, so this leg is timed only and its
        output is not checked."""
    m, k = a16.shape
    n = w_cpu.shape[0]
    flops = 2.0 * m * n * k
    w16 = w_cpu.to(dev)
    out16 = torch.empty(m, n, dtype=torch.bfloat16, device=dev)
    w.quant(a16)   # the shared output set the GEMM leg reads
    legs = {"k_gemm (NVFP4, this library)": (w.gemm0, MFMA_F16_PEAK_TFLOPS),
            "hipblaslt bf16": (lambda: torch.matmul(a16, w16.t(), out=out16), MFMA_F16_PEAK_TFLOPS)}
    fa, sfa = ops.mxfp4_quantize(a16)
    fw, sfw = ops.mxfp4_quantize(w16)
    out_mx = torch.empty(m, n, dtype=torch.bfloat16, device=dev)
    legs["k_gemm_mx (MXFP4, this library)"] = (lambda: ops.mxfp4_gemm(fa, fw, sfa, sfw, out=out_mx),
                                                MFMA_FP4_PEAK_TFLOPS)
    one = torch.ones((), dtype=torch.float32, device=dev)
    a8, w8 = a16.to(torch.float8_e4m3fn), w16.to(torch.float8_e4m3fn)
    legs["hipblaslt fp8 e4m3"] = (lambda: torch._scaled_mm(a8, w8.t(), one, one, out_dtype=torch.bfloat16),
                                  2 * MFMA_F16_PEAK_TFLOPS)
    fa4, fw4 = fa.view(torch.float4_e2m1fn_x2), fw.view(torch.float4_e2m1fn_x2)
    sa8, sw8 = sfa.view(torch.float8_e8m0fnu), sfw.view(torch.float8_e8m0fnu)
    legs["hipblaslt mxfp4"] = (lambda: torch._scaled_mm(fa4, fw4.t(), sa8, sw8, out_dtype=torch.bfloat16),
                               MFMA_FP4_PEAK_TFLOPS)
    res, ok = {}, {}
    for name, (fn, peak) in legs.items():
        try:
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            ok[name] = (fn, peak)
        except Exception as ex:  # a library leg this torch build does not support
            res[name] = {"error": repr(ex)[:200]}
    est_ms = flops / 1.0e12   # the launch time at 1 PFLOP/s
    reps = max(5, min(200, int(30.0 / est_ms)))
    best = {}
    for _ in range(rounds):
        for name, (fn, _) in ok.items():
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) / reps
            best[name] = min(best.get(name, t), t)
    for name, (_, peak) in ok.items():
        tf = flops / (best[name] * 1e-3) / 1e12
        res[name] = {"ms": round(best[name], 5), "tflops": round(tf, 1), "frac_of_dtype_peak": round(tf / peak, 4),
                     "dtype_peak_tflops": peak}
    return {"note": "comparison only: vendor GEMMs on the same shape and data, timed by the same method "
                    f"({reps} launches back to back, best of {rounds} interleaved rounds)", "legs": res}


def gemm_traffic(workload):
    import hashlib

    rec = MEASURED_TRAFFIC.get(workload)
    if rec is None:
        return None
    h = "".join(hashlib.sha256(open(os.path.join(ROOT, f), "rb").read()).hexdigest() for f in GEMM_SOURCES)
    if h != rec["sources_sha256"]:
        return None
    return round(1024 * (rec["fetch_kib"] * rec["fetch_factor"] + rec["write_kib"] * rec["write_factor"]))


def capture(torch, fn):
    """A HIP graph of fn()'s launches on the capture stream (no memset nodes:
    the library launches kernels only)."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def time_graph(torch, g, reps=3):
    """Average time of one replay of g (ms), best of `reps` replays, bracketed
    by HIP events on the replay stream."""
    best = None
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1)
        best = t if best is None else min(best, t)
    return best


def settle(torch, replay, ms=SETTLE_MS):
    """Untimed replays of the graphs about to be timed, back to back for at
    least `ms` of device time, so the timed region starts at the clock the
    chip holds under this load: after the host-side gap of a graph capture
    the clock has dropped, and a single replay of a short graph is still
    ramping (measured: the SVDQuant GEMM 72-85 us per step after one replay,
    72 us steady)."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    replay()
    e1.record()
    torch.cuda.synchronize()
    once = max(e0.elapsed_time(e1), 1e-3)
    for _ in range(min(int(ms / once), 200)):
        replay()
    torch.cuda.synchronize()


def flush_caches(torch):
    """Stream 1 GiB of writes through the caches (L2 and the 256 MB Infinity
    Cache), so the next kernel finds none of its inputs there."""
    buf = torch.empty(2 ** 28, dtype=torch.float32, device="cuda")
    buf.zero_()
    del buf


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import numpy as np
    import torch

    from nvfp4_block_scaled_04_amd import ops, synth

    torch.cuda.set_device(0)
    K = args.steps
    w = build_workload(args.workload, ops, synth, torch)
    n_copies = min(args.rotate or w.rotate_hint, 64)
    acts = w.make_acts(n_copies)
    steps = w.make_steps(acts, K)
    torch.cuda.synchronize()

    for i in range(args.warmup):
        pre, gemm = steps[i % K]
        pre()
        gemm()
    torch.cuda.synchronize()

    if args.copy_calibration:
        src = torch.ones(64 * 2 ** 20, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    # ---- the timed K steps: the K quantizations as one HIP graph, then the K
    # GEMMs (each reading its own step's quantized activation) as another,
    # replayed back to back between three HIP events on the stream the
    # kernels run on; the caches are flushed first, so the steps start cold.
    # ms_per_step, the quantize share and the GEMM's average duration (the
    # roofline's) all come from these events.
    g_q = capture(torch, lambda: [pre() for pre, _ in steps])
    g_g = capture(torch, lambda: [gemm() for _, gemm in steps])
    settle(torch, lambda: (g_q.replay(), g_g.replay()))
    flush_caches(torch)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record()
    g_q.replay()
    ev[1].record()
    g_g.replay()
    ev[2].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_ms = ev[0].elapsed_time(ev[2]) / K
    quant_ms = ev[0].elapsed_time(ev[1]) / K
    gemm_ms = ev[1].elapsed_time(ev[2]) / K
    wall_step_ms = (t1 - t0) * 1e3 / K
    del g_q, g_g

    # ---- for reference: the same steps interleaved (quantize, GEMM, quantize,
    # ...) in one graph, and launched eagerly
    g_i = capture(torch, lambda: [f() for pair in steps for f in pair])
    settle(torch, g_i.replay)
    flush_caches(torch)
    torch.cuda.synchronize()
    inter_ms = time_graph(torch, g_i, reps=1) / K
    del g_i
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for pre, gemm in steps:
        pre()
        gemm()
    torch.cuda.synchronize()
    eager_step_ms = (time.perf_counter() - t0) * 1e3 / K

    # ---- kernel passes back to back, over every activation copy (cold inputs),
    # as HIP graphs so the host's launch latency stays out of the kernel times
    g_pass = capture(torch, lambda: [w.quant(a, ops.GS_STATIC) for a in acts])
    qpass_ms = time_graph(torch, g_pass) / n_copies
    del g_pass
    qdyn_ms = qdyn3_ms = None
    if w.amax_bytes:
        g_dyn = capture(torch, lambda: [w.quant(a, ops.GS_DYNAMIC) for a in acts])
        qdyn_ms = time_graph(torch, g_dyn) / n_copies
        del g_dyn
        if w.quant_3launch is not None:
            g_dyn3 = capture(torch, lambda: [w.quant_3launch(a) for a in acts])
            qdyn3_ms = time_graph(torch, g_dyn3) / n_copies
            del g_dyn3
    w4 = None
    if w.w4a16 is not None:
        # step i reads weight copy i (cold after the flush)
        g_w4 = capture(torch, lambda: [w.w4a16(acts[i % n_copies], i) for i in range(K)])
        settle(torch, g_w4.replay)
        flush_caches(torch)
        torch.cuda.synchronize()
        w4_ms = time_graph(torch, g_w4, reps=1) / K
        del g_w4
        w4_gbs = w.w4a16_bytes / (w4_ms * 1e-3) / 1e9
        w4 = {"ms": round(w4_ms, 5), "gbs": round(w4_gbs, 1), "frac_hbm": round(w4_gbs / HBM_PEAK_GBS, 4),
              "bytes": w.w4a16_bytes, "weights": "cold (one weight copy per launch, caches flushed first)",
              "kernel": "k_gemm_w4a16 (bf16 activation x NVFP4 weight, no activation quantize)"}
    ls = None
    if w.linear_small is not None:
        # the same steps as one launch each, on the same cold weight copies
        g_ls = capture(torch, lambda: [w.linear_small(acts[i % n_copies], i) for i in range(K)])
        settle(torch, g_ls.replay)
        flush_caches(torch)
        torch.cuda.synchronize()
        ls_ms = time_graph(torch, g_ls, reps=1) / K
        del g_ls
        ls_gbs = w.w4a16_bytes / (ls_ms * 1e-3) / 1e9
        ls = {"ms": round(ls_ms, 5), "tflops": round(w.flops / (ls_ms * 1e-3) / 1e12, 2),
              "gbs": round(ls_gbs, 1), "frac_hbm": round(ls_gbs / HBM_PEAK_GBS, 4), "bytes": w.w4a16_bytes,
              "weights": "cold (one weight copy per launch, caches flushed first)",
              "kernel": ("k_linear_small (nvfp4_linear_small: the activation's dynamic quantization into LDS "
                         "in every workgroup, then the skinny GEMM; bit for bit the quantize + alpha + GEMM calls)")}
    ld = None
    if w.lora_down is not None:
        g_ld = capture(torch, lambda: [w.lora_down(a) for a in acts])
        ld_ms = time_graph(torch, g_ld) / n_copies
        del g_ld
        ld_gbs = w.lora_down_bytes / (ld_ms * 1e-3) / 1e9
        g_ldu = capture(torch, lambda: [w.lora_down_unprepared(a) for a in acts])
        ldu_ms = time_graph(torch, g_ldu) / n_copies
        del g_ldu
        ld = {"ms": round(ld_ms, 5), "gbs": round(ld_gbs, 1), "frac_hbm": round(ld_gbs / HBM_PEAK_GBS, 4),
              "bytes": w.lora_down_bytes,
              "kernel": ("k_quantize_lora (smooth quantize + LoRA-down projection, one read of x; the weight "
                         "prepared once as exact bf16 halves of pqs * L2 in operand order)"),
              "unprepared_ms": round(ldu_ms, 5),
              "unprepared_gbs": round(w.lora_down_unprepared_bytes / (ldu_ms * 1e-3) / 1e9, 1),
              "unprepared": "nvfp4_quantize_lora_down on the raw l2: x * pqs split into bf16 halves per element"}
    # ceilings of the memory system on this machine, timed the same way: a plain
    # elementwise copy (read + write) and a read-only reduction (torch)
    src = torch.ones(64 * 2 ** 20, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    g_copy = capture(torch, lambda: [torch.neg(src, out=dst) for _ in range(4)])
    copy_gbs = 2 * src.numel() * 4 / (time_graph(torch, g_copy) / 4 * 1e-3) / 1e9
    del g_copy
    # (launched eagerly: a reduction may record memset nodes, which stay out
    # of graphs here; each launch reads 256 MiB, so launch gaps are small)
    red = torch.empty((), dtype=torch.float32, device="cuda")
    torch.sum(src, dim=0, out=red)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(4):
        torch.sum(src, dim=0, out=red)
    e1.record()
    torch.cuda.synchronize()
    read_gbs = src.numel() * 4 / (e0.elapsed_time(e1) / 4 * 1e-3) / 1e9
    del src, dst

    gemm_tflops = w.flops / (gemm_ms * 1e-3) / 1e12
    value = w.flops / (step_ms * 1e-3) / 1e12
    q_gbs = w.q_bytes / (qpass_ms * 1e-3) / 1e9
    e2e_bytes = w.q_bytes + w.amax_bytes
    quant = {"pass_ms": round(qpass_ms, 5), "pass_gbs": round(q_gbs, 1),
             "pass_frac_hbm": round(q_gbs / HBM_PEAK_GBS, 4),
             "pass_frac_copy": round(q_gbs / copy_gbs, 4),
             "in_step_ms": round(quant_ms, 5),
             "pass_bytes": w.q_bytes, "amax_pass_bytes": w.amax_bytes,
             "copy_kernel_gbs": round(copy_gbs, 1), "read_only_reduction_gbs": round(read_gbs, 1)}
    if qdyn_ms is not None:
        quant["dynamic_call_ms"] = round(qdyn_ms, 5)
        quant["dynamic_call_gbs"] = round(e2e_bytes / (qdyn_ms * 1e-3) / 1e9, 1)
        quant["dynamic_call"] = getattr(w, "dynamic_call_desc", None) or (
            "the step's call: amax pass with partials in a workspace, then the quantize pass (which reduces "
            "them and writes gs and alpha); bytes = amax pass + quantize pass")
    if qdyn3_ms is not None:
        quant["dynamic_call_3launch_ms"] = round(qdyn3_ms, 5)
        quant["dynamic_call_3launch"] = w.quant_3launch_desc
        quant["dynamic_call_3launch_gbs"] = round(e2e_bytes / (qdyn3_ms * 1e-3) / 1e9, 1)
    res = {
        "metric": "NVFP4 GEMM TFLOP/s (+% peak) and quantize GB/s (+% HBM peak), 1xMI355X",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "wall_ms_per_step": round(wall_step_ms, 5),
        "interleaved_graph_ms_per_step": round(inter_ms, 5),
        "eager_ms_per_step": round(eager_step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic (seeded N(0,1) activations with outlier channels, N(0,0.02) weights)",
        "config": {"workload": w.desc, **w.cfg, "operands": "NVFP4 (e2m1 + ue4m3 per 16, 128x4 swizzled)",
                   "parallelism": "none (1 GPU)", "activation_copies_rotated": n_copies,
                   "weight_copies_rotated": w.n_wcopies},
        "gemm": {"ms": round(gemm_ms, 5), "tflops": round(gemm_tflops, 2),
                 "frac_f16_mfma_peak": round(gemm_tflops / MFMA_F16_PEAK_TFLOPS, 4)},
        "quantize": quant,
        "roofline": {"bound": "mfma", "achieved": round(gemm_tflops, 2), "peak": MFMA_F16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(gemm_tflops / MFMA_F16_PEAK_TFLOPS, 4),
                     "traffic": gemm_traffic(args.workload), "kernel": w.gemm_kernel,
                     "flops_per_launch": w.flops, "algorithmic_bytes_per_launch": w.gemm_bytes},
        "timing": ("one timed region: the K steps' quantizations as one HIP graph, then their K GEMMs as "
                   "another, between HIP events on the kernels' stream, after >= 30 ms of untimed replays of "
                   "both graphs and a cache flush; ms_per_step, "
                   "quantize.in_step_ms, gemm.ms and roofline.achieved all come from those events"),
    }
    if w.hbm_bound:
        # 16 activation rows: the GEMM streams the weight once; its roofline is
        # HBM, over the same event-timed GEMM duration, cold weights
        gbs = w.gemm_bytes / (gemm_ms * 1e-3) / 1e9
        res["roofline"] = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": gemm_traffic(args.workload),
                           "kernel": "k_gemm_skinny (block-scaled NVFP4 GEMM, 16 rows, cold weight copies)",
                           "algorithmic_bytes_per_launch": w.gemm_bytes}
    if w4 is not None:
        res["w4a16"] = w4
    if ls is not None:
        res["linear_small"] = ls
    if ld is not None:
        res["quantize_lora_down"] = ld
    if w.mx is not None:
        res["mx"] = w.mx(acts)
    if w.library is not None and not args.no_library:
        res["library"] = w.library(acts)
    if w.swiglu is not None:
        del acts, steps
        torch.cuda.empty_cache()
        res["swiglu_gate_up"] = w.swiglu()
    if not args.no_cpu_baseline and w.cpu_sample is not None:
        import oracle as O
        res["cpu_baseline"] = w.cpu_sample(O, np)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
