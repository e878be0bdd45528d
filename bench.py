"""Benchmark of the NVFP4 hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input that
is already resident in HBM: NVFP4 quantization of the bf16 activation with a
dynamic global scale (amax pass, finish, quantize pass; one launch for small
activations) whose last launch also writes alpha = 1/(gs_a*gs_w), and the
block-scaled GEMM to bf16.  Weights are
quantized once before timing (same kernels, untimed).  The K timed steps
are launched as one HIP graph (captured after the W warm-up steps, launched
once untimed to upload it); the same K steps launched eagerly, with HIP
events between the quantize part and the GEMM, give the two parts' times and
`eager_ms_per_step`.

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
    """Device-resident inputs plus the step closure and its algorithmic work."""


def build_workload(name, ops, synth, torch):
    w = Workload()
    w.hbm_bound = False
    w.w4a16 = None
    w.lora_down = None
    w.swiglu = None
    w.mx = None
    w.library = None
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
            w.desc = "decode linear 16x4096x4096: bf16 activation -> dynamic NVFP4 quantize -> block-scaled GEMM -> bf16"
        else:
            d = synth.tiny()
            a_cpu, w_cpu = d.a, d.w
            w.desc = "tiny 128x256x256: fp32 activation -> dynamic NVFP4 quantize -> block-scaled GEMM -> bf16"
        m, k = a_cpu.shape
        n = w_cpu.shape[0]
        fw, sfw, gsw = ops.nvfp4_quantize(w_cpu.to(dev))
        esz = a_cpu.element_size()
        act_bytes = m * k * esz
        copies = w.rotate_hint = max(1, -(-512 * 2 ** 20 // act_bytes))
        w.acts = None
        w.a_cpu, w.w_cpu = a_cpu, w_cpu
        w.m, w.n, w.k = m, n, k
        w.flops = 2.0 * m * n * k
        w.q_bytes = m * k * esz + m * k // 2 + sf_size(m, k)     # quantize pass
        w.amax_bytes = m * k * esz                                 # amax pass
        w.gemm_bytes = m * k // 2 + sf_size(m, k) + n * k // 2 + sf_size(n, k) + 2 * m * n
        fa = torch.empty(m, k // 2, dtype=torch.uint8, device=dev)
        sfa = torch.empty(sf_size(m, k), dtype=torch.uint8, device=dev)
        gsa = torch.zeros(1, dtype=torch.float32, device=dev)
        alpha = torch.empty(1, dtype=torch.float32, device=dev)
        out = torch.empty(m, n, dtype=torch.bfloat16, device=dev)

        def quant(a, mode=ops.GS_DYNAMIC):
            ops.nvfp4_quantize(a, gsa, mode, out_fp4=fa, out_sf=sfa)

        def gemm():
            ops.nvfp4_gemm(fa, fw, sfa, sfw, alpha, out=out)

        def pre(a):  # dynamic quantize; the same launch writes alpha = 1/(gs_a*gs_w)
            ops.nvfp4_quantize_alpha(a, gsw, gsa, ops.GS_DYNAMIC, out_fp4=fa, out_sf=sfa, alpha=alpha)

        w.make_acts = lambda n_copies: [a_cpu.to(dev) for _ in range(n_copies)]
        w.pre, w.quant, w.gemm = pre, quant, gemm
        w.outputs = (fa, sfa, gsa, alpha, out)
        w.cfg = {"m": m, "n": n, "k": k}
        w.hbm_bound = name == "decode"   # 16 rows: the weight read bounds the GEMM
        if name == "decode":
            # weight-only form: the bf16 activation against the NVFP4 weight,
            # no activation quantization (alpha = 1 / the weight's gs)
            alpha_w = ops.nvfp4_alpha(torch.ones(1, dtype=torch.float32, device=dev), gsw)
            out_w = torch.empty(m, n, dtype=torch.bfloat16, device=dev)
            w.w4a16 = lambda a: ops.nvfp4_gemm_w4a16(a, fw, sfw, alpha_w, out=out_w)
            w.w4a16_bytes = n * k // 2 + sf_size(n, k) + m * k * 2 + 2 * m * n
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
        mask = mo.mask.to(dev)
        valid = int(mo.mask.clamp(0, m).sum())
        fa = torch.empty(E, m, h // 2, dtype=torch.uint8, device=dev)
        sfa = torch.empty(E, sf_size(m, h), dtype=torch.uint8, device=dev)
        gsa = torch.zeros(E, dtype=torch.float32, device=dev)
        alpha = torch.empty(E, dtype=torch.float32, device=dev)
        out = torch.empty(E, m, n, dtype=torch.bfloat16, device=dev)

        def quant(x, mode=ops.GS_DYNAMIC):
            ops.silu_mul_nvfp4_quantize(x, mask, gsa, mode, out_fp4=fa, out_sf=sfa)

        def gemm():
            ops.nvfp4_gemm_grouped_masked(fa, fw, sfa, sfw, alpha, mask, out=out)

        def pre(x):
            quant(x)
            ops.nvfp4_alpha(gsa, gsw, out=alpha)

        w.desc = ("Llama4-style routed experts: E=8 gate|up [512,16384] bf16, valid rows "
                  f"{mo.mask.tolist()} -> fused silu_and_mul + NVFP4 quantize -> grouped masked GEMM vs [8,5120,8192]")
        act_bytes = mo.x.numel() * 2
        w.rotate_hint = max(1, -(-512 * 2 ** 20 // act_bytes))
        w.make_acts = lambda n_copies: [mo.x.to(dev) for _ in range(n_copies)]
        w.pre, w.quant, w.gemm = pre, quant, gemm
        w.outputs = (fa, sfa, gsa, alpha, out)
        w.flops = 2.0 * n * h * valid
        w.q_bytes = valid * 2 * h * 2 + E * m * h // 2 + E * sf_size(m, h)
        w.amax_bytes = valid * 2 * h * 2
        w.gemm_bytes = valid * h // 2 + E * sf_size(m, h) + E * n * h // 2 + E * sf_size(n, h) + 2 * valid * n
        w.m, w.n, w.k = valid, n, h
        w.cfg = {"experts": E, "m_max": m, "valid_rows": mo.mask.tolist(), "n": n, "k": h}
        w.cpu_sample = None
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
        d = torch.empty(m, r, dtype=torch.bfloat16, device=dev)   # formed inside the step
        l1 = synth.lora_up(s, al).to(dev)
        bias = s.bias.to(dev)
        fa = torch.empty(m, k // 2, dtype=torch.uint8, device=dev)
        sfa = torch.empty(sf_size(m, k), dtype=torch.uint8, device=dev)
        out = torch.empty(m, n, dtype=torch.bfloat16, device=dev)

        def quant(x, mode=ops.GS_STATIC):
            ops.nvfp4_quantize(x, gsa, mode, pre_quant_scale=pqs, out_fp4=fa, out_sf=sfa)

        def gemm():
            ops.nvfp4_gemm_svdquant(fa, fw, sfa, sfw, alpha, d, l1, bias=bias, out=out)

        def pre(x):
            # smooth quantize and the LoRA-down projection d, one read of x
            ops.nvfp4_quantize_lora_down(x, pqs, l2, gsa, ops.GS_STATIC, out_fp4=fa, out_sf=sfa, d=d)

        w.lora_down = pre
        w.lora_down_bytes = m * k * 2 + k * 2 + r * k * 2 + m * k // 2 + sf_size(m, k) + 2 * m * r
        w.desc = ("SVDQuant linear 4096x3072x3072, r=32: smooth NVFP4 quantize (static gs) with the LoRA-down "
                  "projection fused -> fused GEMM + LoRA-up + bias")
        w.rotate_hint = max(1, -(-512 * 2 ** 20 // (m * k * 2)))
        w.make_acts = lambda n_copies: [s.x.to(dev) for _ in range(n_copies)]
        w.pre, w.quant, w.gemm = pre, quant, gemm
        w.outputs = (fa, sfa, out)
        w.flops = 2.0 * m * n * k + 2.0 * m * n * r
        w.q_bytes = m * k * 2 + k * 2 + m * k // 2 + sf_size(m, k)
        w.amax_bytes = 0
        w.gemm_bytes = m * k // 2 + sf_size(m, k) + n * k // 2 + sf_size(n, k) + 2 * m * n + 2 * (m + n) * r + 2 * n
        w.m, w.n, w.k = m, n, k
        w.cfg = {"m": m, "n": n, "k": k, "r": r}
        w.cpu_sample = None
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


def cpu_baseline_dense(O, np, a_cpu, w_cpu, synth, target_s=12.0):
    """The oracle on a bounded sample of the same step: the weight is
    quantized once, untimed (offline in the GPU step too); the timed part
    quantizes a slice of activation rows (dynamic gs over the slice) and
    computes the GEMM for those rows.  A 64-row probe sizes the slice so the
    timed run takes about `target_s` seconds."""
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

    rows = 64
    dt = run(rows)
    if dt < target_s / 2:
        rows = int(min(m, max(rows, 64 * round(rows * target_s / dt / 64))))
        dt = run(rows)
    flops = 2.0 * rows * n * k
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": O.num_threads(),
        "kind": "oracle",
        "sample": f"{rows} of {m} activation rows: oracle dynamic quantize of those rows + "
                  f"oracle dequant-GEMM {rows}x{n}x{k} (fp64 accumulation), {dt:.2f} s wall",
    }


# HBM traffic of the GEMM kernel per launch, from two rocprofv3 --pmc runs
# (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch) of this script, scaled by
# what the same counters read for a plain copy of known size
# (--copy-calibration: fetch x2.000, write x1.000).  A record is used only
# while the kernel sources hash to the value it was measured on.
MEASURED_TRAFFIC = {
    "prefill": {"sources_sha256": "4c38f76689a21cab5a4420095a8271d49a34bdd6848c6b134907006c5cc32195"
                                  "faf55d4cd243fe2a127d65280e8b95f55a1c37a38f9c6433dcc115ee1fe0f350"
                                  "b78954052145e2babdd6f327935f70bab87bfb0bca4c38bc415b04c1fd7708b1"
                                  "1286af577a92b62864a1892dab16fdf95f9c00e73cc4786fcdc44f6510096e56",
                "fetch_kib": 276691.5, "write_kib": 262144.0, "fetch_factor": 2.0, "write_factor": 1.0},
    "moe": {"sources_sha256": "4c38f76689a21cab5a4420095a8271d49a34bdd6848c6b134907006c5cc32195"
                              "faf55d4cd243fe2a127d65280e8b95f55a1c37a38f9c6433dcc115ee1fe0f350"
                              "b78954052145e2babdd6f327935f70bab87bfb0bca4c38bc415b04c1fd7708b1"
                              "1286af577a92b62864a1892dab16fdf95f9c00e73cc4786fcdc44f6510096e56",
            "fetch_kib": 158206.1, "write_kib": 15350.0, "fetch_factor": 2.0, "write_factor": 1.0},
    "dense": {"sources_sha256": "4c38f76689a21cab5a4420095a8271d49a34bdd6848c6b134907006c5cc32195"
                                "faf55d4cd243fe2a127d65280e8b95f55a1c37a38f9c6433dcc115ee1fe0f350"
                                "b78954052145e2babdd6f327935f70bab87bfb0bca4c38bc415b04c1fd7708b1"
                                "1286af577a92b62864a1892dab16fdf95f9c00e73cc4786fcdc44f6510096e56",
              "fetch_kib": 18638.0, "write_kib": 16384.0, "fetch_factor": 2.0, "write_factor": 1.0},
    "svdquant": {"sources_sha256": "4c38f76689a21cab5a4420095a8271d49a34bdd6848c6b134907006c5cc32195"
                                   "faf55d4cd243fe2a127d65280e8b95f55a1c37a38f9c6433dcc115ee1fe0f350"
                                   "b78954052145e2babdd6f327935f70bab87bfb0bca4c38bc415b04c1fd7708b1"
                                   "1286af577a92b62864a1892dab16fdf95f9c00e73cc4786fcdc44f6510096e56",
                 "fetch_kib": 18474.0, "write_kib": 24576.0, "fetch_factor": 2.0, "write_factor": 1.0},
    "decode": {"sources_sha256": "4c38f76689a21cab5a4420095a8271d49a34bdd6848c6b134907006c5cc32195"
                                 "faf55d4cd243fe2a127d65280e8b95f55a1c37a38f9c6433dcc115ee1fe0f350"
                                 "b78954052145e2babdd6f327935f70bab87bfb0bca4c38bc415b04c1fd7708b1"
                                 "1286af577a92b62864a1892dab16fdf95f9c00e73cc4786fcdc44f6510096e56",
               "fetch_kib": 6404.0, "write_kib": 128.0, "fetch_factor": 2.0, "write_factor": 1.0},
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
    legs = {"k_gemm (NVFP4, this library)": (w.gemm, MFMA_F16_PEAK_TFLOPS),
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
    w = build_workload(args.workload, ops, synth, torch)
    n_copies = min(args.rotate or w.rotate_hint, 64)
    acts = w.make_acts(n_copies)
    torch.cuda.synchronize()

    for i in range(args.warmup):
        w.pre(acts[i % n_copies])
        w.gemm()
    torch.cuda.synchronize()

    if args.copy_calibration:
        src = torch.ones(64 * 2 ** 20, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    # ---- the K steps launched eagerly on the current stream, with HIP events
    # between the quantize part and the GEMM (the per-phase times)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        evs[i][0].record()
        w.pre(acts[i % n_copies])
        evs[i][1].record()
        w.gemm()
        evs[i][2].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    eager_step_ms = (t1 - t0) * 1e3 / args.steps
    quant_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    gemm_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))

    # ---- the timed K steps: the same launches captured as one HIP graph (a
    # launch-bound step such as decode spends most of its eager time in host
    # launches), launched once untimed so that the timed launch finds it
    # uploaded, then timed between two synchronizations
    g_steps = capture(torch, lambda: [(w.pre(acts[i % n_copies]), w.gemm()) for i in range(args.steps)])
    g_steps.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g_steps.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_ms = (t1 - t0) * 1e3 / args.steps
    del g_steps

    # ---- kernel passes back to back, over every activation copy (cold inputs),
    # as HIP graphs so the host's launch latency stays out of the kernel times
    g_pass = capture(torch, lambda: [w.quant(a, ops.GS_STATIC) for a in acts])
    qpass_ms = time_graph(torch, g_pass) / n_copies
    if w.amax_bytes:
        g_dyn = capture(torch, lambda: [w.quant(a, ops.GS_DYNAMIC) for a in acts])
        qdyn_ms = time_graph(torch, g_dyn) / n_copies
    else:
        qdyn_ms = qpass_ms
    # the GEMM alone, back to back (for the weight-bound decode shape, whose
    # eager launches cost more than the kernel)
    g_gemm = capture(torch, lambda: [w.gemm() for _ in range(n_copies)])
    gemm_graph_ms = time_graph(torch, g_gemm) / n_copies
    del g_gemm
    w4 = None
    if w.w4a16 is not None:
        g_w4 = capture(torch, lambda: [w.w4a16(a) for a in acts])
        w4_ms = time_graph(torch, g_w4) / n_copies
        del g_w4
        w4_gbs = w.w4a16_bytes / (w4_ms * 1e-3) / 1e9
        w4 = {"ms": round(w4_ms, 5), "gbs": round(w4_gbs, 1), "frac_hbm": round(w4_gbs / HBM_PEAK_GBS, 4),
              "bytes": w.w4a16_bytes, "kernel": "k_gemm_w4a16 (bf16 activation x NVFP4 weight, no activation quantize)"}
    ld = None
    if w.lora_down is not None:
        g_ld = capture(torch, lambda: [w.lora_down(a) for a in acts])
        ld_ms = time_graph(torch, g_ld) / n_copies
        del g_ld
        ld_gbs = w.lora_down_bytes / (ld_ms * 1e-3) / 1e9
        ld = {"ms": round(ld_ms, 5), "gbs": round(ld_gbs, 1), "frac_hbm": round(ld_gbs / HBM_PEAK_GBS, 4),
              "bytes": w.lora_down_bytes,
              "kernel": "k_quantize_lora (smooth quantize + LoRA-down projection, one read of x)"}
    src = torch.ones(64 * 2 ** 20, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    g_copy = capture(torch, lambda: [torch.neg(src, out=dst) for _ in range(4)])
    copy_gbs = 2 * src.numel() * 4 / (time_graph(torch, g_copy) / 4 * 1e-3) / 1e9
    del src, dst, g_copy

    gemm_tflops = w.flops / (gemm_ms * 1e-3) / 1e12
    value = w.flops / (step_ms * 1e-3) / 1e12
    q_gbs = w.q_bytes / (qpass_ms * 1e-3) / 1e9
    amax_ms = qdyn_ms - qpass_ms
    e2e_bytes = w.q_bytes + w.amax_bytes
    res = {
        "metric": "NVFP4 GEMM TFLOP/s (+% peak) and quantize GB/s (+% HBM peak), 1xMI355X",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "eager_ms_per_step": round(eager_step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic (seeded N(0,1) activations with outlier channels, N(0,0.02) weights)",
        "config": {"workload": w.desc, **w.cfg, "operands": "NVFP4 (e2m1 + ue4m3 per 16, 128x4 swizzled)",
                   "parallelism": "none (1 GPU)", "activation_copies_rotated": n_copies},
        "gemm": {"ms": round(gemm_ms, 4), "tflops": round(gemm_tflops, 2),
                 "frac_f16_mfma_peak": round(gemm_tflops / MFMA_F16_PEAK_TFLOPS, 4),
                 "back_to_back_ms": round(gemm_graph_ms, 5)},
        "quantize": {"pass_ms": round(qpass_ms, 4), "pass_gbs": round(q_gbs, 1),
                     "pass_frac_hbm": round(q_gbs / HBM_PEAK_GBS, 4),
                     "amax_and_finish_ms": round(amax_ms, 4),
                     "amax_gbs": round(w.amax_bytes / (amax_ms * 1e-3) / 1e9, 1) if w.amax_bytes else None,
                     "dynamic_call_ms": round(qdyn_ms, 4),
                     "dynamic_call_gbs": round(e2e_bytes / (qdyn_ms * 1e-3) / 1e9, 1),
                     "in_step_ms": round(quant_ms, 4),
                     "pass_bytes": w.q_bytes, "amax_pass_bytes": w.amax_bytes,
                     "copy_kernel_gbs": round(copy_gbs, 1)},
        "roofline": {"bound": "mfma", "achieved": round(gemm_tflops, 2), "peak": MFMA_F16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(gemm_tflops / MFMA_F16_PEAK_TFLOPS, 4),
                     "traffic": gemm_traffic(args.workload), "kernel": "k_gemm (block-scaled NVFP4 GEMM)",
                     "flops_per_launch": w.flops, "algorithmic_bytes_per_launch": w.gemm_bytes},
    }
    if w.hbm_bound:
        # 16 activation rows: the GEMM streams the weight once; its roofline is
        # HBM, over the back-to-back kernel time
        gbs = w.gemm_bytes / (gemm_graph_ms * 1e-3) / 1e9
        res["roofline"] = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": gemm_traffic(args.workload),
                           "kernel": "k_gemm_skinny (block-scaled NVFP4 GEMM, 16 rows)",
                           "algorithmic_bytes_per_launch": w.gemm_bytes}
    if w4 is not None:
        res["w4a16"] = w4
    if ld is not None:
        res["quantize_lora_down"] = ld
    if w.mx is not None:
        res["mx"] = w.mx(acts)
    if w.library is not None and not args.no_library:
        res["library"] = w.library(acts)
    if w.swiglu is not None:
        del acts
        torch.cuda.empty_cache()
        res["swiglu_gate_up"] = w.swiglu()
    if not args.no_cpu_baseline and w.cpu_sample is not None:
        import oracle as O
        res["cpu_baseline"] = w.cpu_sample(O, np)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
