"""Benchmark of the TTQ q_proj hot path on one MI355X.

Workload: the Qwen3-32B q_proj (d = 5120 -> d' = 8192, thelatestinai.com
listing, Table 15: 64 heads x 128), one prompt of T = 16384 fp16 tokens,
q = 4, g = 32, alpha = 0.5, lambda = 0.4, p = 2.  Synthetic seeded
activations and weights (workloads module); inputs are resident in HBM
before the timed region.

One step = the whole per-prompt hot path: ttq_prepare (column statistic +
quantise/pack) then ttq_linear (the low-bit projection of the prompt).
Reported: prefill k tokens/s at r = 0 (the value), the GEMM's own duration
inside the timed steps against the fp16 matrix-core peak (roofline), the same
step at r = 16, the decode projection for T in {1, 16, 64} reusing the
prefill quantisation, per-kernel times with their roofline fractions, q/k/v
sharing one prepare, the other code widths and group sizes, and the CPU
oracle on one step of the workload as a baseline.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--skip-cpu]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 matrix peak


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--settle-ms", type=float, default=250.0,
                    help="untimed steps run for this long before the warmup steps, so that the GPU's "
                         "clock and power state is the steady one of continuous work")
    ap.add_argument("--skip-cpu", action="store_true", help="leave out the CPU oracle baseline")
    ap.add_argument("--only", default="", help="comma list of parts to run: step,r16,decode,kernels,qkv,variants,configs; "
                    "'copy' (never by default) adds a plain device copy of 512 MiB, the reference "
                    "for scaling the profiler's FETCH_SIZE / WRITE_SIZE counters")
    return ap.parse_args()


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "traffic_qwen3_32b_qproj_q4g32r0.md")
CSRC = os.path.join(ROOT, "test_activation_aware_amd", "csrc")
DENSE_SOURCE = os.path.join(CSRC, "dense_gemm.hip")          # the dense form's GEMM (handles with W_hat)
LOWBIT_SOURCE = os.path.join(CSRC, "wlowbit_gemm_impl.h")    # the low-bit GEMM on the codes


def gemm_traffic(source):
    """HBM bytes per launch of the GEMM built from `source`, from the committed
    counter runs, or None when that source has changed since they were
    taken.  The profile records one line per kernel source:
        - <file name> sha256 <hex>, traffic bytes per launch <n>"""
    try:
        text = open(TRAFFIC_PROFILE).read()
        src = hashlib.sha256(open(source, "rb").read()).hexdigest()
    except OSError:
        return None
    m = re.search(re.escape(os.path.basename(source)) + r" sha256 ([0-9a-f]{64}), traffic bytes per launch (\d+)", text)
    if not m or m.group(1) != src:
        return None
    return int(m.group(2))


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def time_loop(fn, n, torch):
    """Average GPU time of fn() over n back-to-back calls on the current stream."""
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(n):
        fn()
    e1.record(s)
    e1.synchronize()
    return e0.elapsed_time(e1) / n * 1e-3  # seconds


def time_graph(fn, n, torch, replays=5):
    """Average GPU time of fn() with the host taken out: n calls captured in a
    HIP graph (fn must not allocate or synchronise), the graph replayed
    `replays` times between two events.  For kernels of a few tens of
    microseconds the Python side of a call takes about as long as the kernel,
    so back-to-back eager calls would time the host."""
    fn()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(n):
            fn()
    graph.replay()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(replays):
        graph.replay()
    e1.record(s)
    e1.synchronize()
    del graph
    return e0.elapsed_time(e1) / (n * replays) * 1e-3


def settle(fn, ms, torch):
    """Run fn() back to back for about ms milliseconds (untimed).  After an idle
    spell the first GEMMs run up to 30 % slower while the power controller
    settles; without this the timed steps would measure that transient."""
    t0 = time.perf_counter()
    n = 0
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(4):
            fn()
        torch.cuda.synchronize()
        n += 4
    return n


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this implementation runs on one GPU only; the multi-GPU sharding of the path "
              "is described, not implemented (use --gpus 1)", file=sys.stderr)
        sys.exit(2)
    only = set(filter(None, args.only.split(","))) or {"step", "r16", "decode", "kernels", "qkv", "variants",
                                                        "configs"}

    import numpy as np
    import torch

    import test_activation_aware_amd as ttq
    import workloads as wl

    torch.cuda.set_device(0)
    w = wl.by_name("qwen3_32b_qproj")
    T, d, d_out, q, g = w.T, w.d, w.d_out, 4, 32
    log(f"bench: generating inputs T={T} d={d} d'={d_out}")
    X_np, W_np = wl.config_inputs(w.cfg)
    X = torch.from_numpy(X_np).cuda()
    W = torch.from_numpy(W_np).cuda()
    Y = torch.empty((T, d_out), dtype=torch.float16, device="cuda")
    layer = ttq.TTQLinear(W, q=q, g=g, alpha=w.alpha, lam=w.lam, p=w.p, r=0, T_max=T)
    torch.cuda.synchronize()

    def step():
        layer.prepare(X)
        layer.linear(X, out=Y)

    result = {}
    # ---- the headline step: prepare + prefill projection, r = 0 ----
    n_settle = settle(step, args.settle_ms, torch)
    log(f"bench: {n_settle} settling steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"bench: timing {args.steps} steps")
    # HIP events on the launching stream around ttq_linear inside the timed
    # steps: for fp16 input, T > 64 and r = 0 it launches exactly one kernel,
    # the raw-input GEMM, so each pair brackets that kernel's run within the
    # step (the host enqueues far ahead of the GPU, so no idle time falls
    # between the events)
    s = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    evp = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for ep, (e0, e1) in zip(evp, evs):
        ep.record(s)
        layer.prepare(X)
        e0.record(s)
        layer.linear(X, out=Y)
        e1.record(s)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = elapsed / args.steps * 1e3
    value = T * args.steps / elapsed / 1e3
    # the prepare step (colstats + quantize_pack) inside the timed steps
    t_prep_step = sum(ep.elapsed_time(e0) for ep, (e0, _) in zip(evp, evs)) / args.steps * 1e-3
    result["prepare_k_tok_s"] = T / t_prep_step / 1e3
    result["prepare_us_in_step"] = t_prep_step * 1e6
    gm_launches = sorted(e0.elapsed_time(e1) * 1e-3 for e0, e1 in evs)
    t_gm_step = sum(gm_launches) / len(gm_launches)
    gm_pct = {f"us_p{k}": gm_launches[min(len(gm_launches) - 1, (len(gm_launches) * k) // 100)] * 1e6
              for k in (10, 50, 90)}

    gemm_flops = 2.0 * T * d * d_out
    dense = layer.wexp is not None and T >= ttq.ttq_dense_min_tokens(d_out)
    result["projection_k_tok_s"] = T / t_gm_step / 1e3
    result["roofline"] = {"bound": "mfma", "achieved": gemm_flops / t_gm_step / 1e12,
                          "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                          "frac": gemm_flops / t_gm_step / 1e12 / MFMA_F16_PEAK_TFLOPS,
                          "traffic": gemm_traffic(DENSE_SOURCE if dense else LOWBIT_SOURCE),
                          "kernel": ("dense_gemm_kernel: fp16 GEMM on the effective weight W_hat formed by "
                                     "the prepare step (ttq_linear, long prompts)" if dense else
                                     "wlowbit_gemm_kernel: low-bit GEMM on the packed codes, raw fp16 input with "
                                     "D^(-1/2) on the weight side (ttq_linear, long prompts)"),
                          "launch_us": t_gm_step * 1e6}

    # ---- per-kernel times, back to back (same inputs, same launch configuration) ----
    kernels = {}
    n_k = max(10, args.steps)
    if "kernels" in only:
        D, R = layer.D, layer.dinvsqrt
        ws = layer.workspace
        t_cs = time_graph(lambda: ttq.ttq_colstats(X, w.p, w.lam, w.alpha, D=D, dinvsqrt=R, workspace=ws), n_k, torch)
        t_qp = time_graph(lambda: ttq.ttq_quantize_pack(W, D, q, g, layer.codes, layer.scales, layer.zeros), n_k, torch)
        Xs = ttq.ttq_prescale(X, R)
        t_ps = time_graph(lambda: ttq.ttq_prescale(X, R, out=Xs), n_k, torch)
        t_gm = time_loop(lambda: ttq.ttq_wlowbit_gemm_raw(X, layer.dinvsqrt16, layer.codes, layer.scales,
                                                          layer.zeros, q, g, d_out, out=Y), n_k, torch)
        # the dense form (GEMM on the effective weight W_hat, an opt-in of the
        # handle API): its GEMM back to back and its whole step, on this machine
        layer_d = ttq.TTQLinear(W, q=q, g=g, alpha=w.alpha, lam=w.lam, p=w.p, r=0, T_max=T, expand=True)
        layer_d.prepare(X)
        t_dg = time_loop(lambda: ttq.ttq_wexp_gemm(X, layer_d.wexp, out=Y), n_k, torch)

        def step_d():
            layer_d.prepare(X)
            layer_d.linear(X, out=Y)
        for _ in range(args.warmup):
            step_d()
        t_step_d = time_loop(step_d, args.steps, torch)
        layer_d.close()
        del layer_d
        t_prep = time_graph(lambda: layer.prepare(X), n_k, torch)
        t_gm_pre = time_loop(lambda: ttq.ttq_wlowbit_gemm(Xs, layer.codes, layer.scales, layer.zeros, q, g, d_out,
                                                          out=Y), n_k, torch)
        cs_bytes = T * d * 2 + 8 * d
        qp_bytes = 2 * d_out * d + 4 * d + q * d_out * d // 8 + 4 * d_out * d // g
        # cold: every call reads a different copy of X (3 x 168 MB) or of W with
        # its own outputs (6 x 110 MB), more than the 256 MB Infinity Cache and
        # the 8 x 4 MB L2 hold, so each call streams its inputs from HBM
        n_xc, n_wc = 3, 6
        Xc = [X.clone() for _ in range(n_xc)]
        Dc = [torch.empty_like(D) for _ in range(n_xc)]
        Rc = [torch.empty_like(R) for _ in range(n_xc)]
        wsc = [torch.empty_like(ws) for _ in range(n_xc)]
        Wc = [W.clone() for _ in range(n_wc)]
        outc = [(torch.empty_like(layer.codes), torch.empty_like(layer.scales), torch.empty_like(layer.zeros))
                for _ in range(n_wc)]

        def cs_cold():
            for i in range(n_xc):
                ttq.ttq_colstats(Xc[i], w.p, w.lam, w.alpha, D=Dc[i], dinvsqrt=Rc[i], workspace=wsc[i])

        def qp_cold():
            for i in range(n_wc):
                ttq.ttq_quantize_pack(Wc[i], D, q, g, *outc[i])
        t_cs_cold = time_graph(cs_cold, 4, torch) / n_xc
        t_qp_cold = time_graph(qp_cold, 4, torch) / n_wc
        del Xc, Dc, Rc, wsc, Wc, outc
        ps_bytes = 4 * T * d + 4 * d
        gm_flops = gemm_flops
        kernels = {
            "colstats": {"us": t_cs * 1e6, "GBs": cs_bytes / t_cs / 1e9,
                         "frac_hbm": cs_bytes / t_cs / 1e9 / HBM_PEAK_GBS,
                         "us_cold": t_cs_cold * 1e6, "frac_hbm_cold": cs_bytes / t_cs_cold / 1e9 / HBM_PEAK_GBS},
            "quantize_pack": {"us": t_qp * 1e6, "GBs": qp_bytes / t_qp / 1e9,
                              "frac_hbm": qp_bytes / t_qp / 1e9 / HBM_PEAK_GBS,
                              "us_cold": t_qp_cold * 1e6,
                              "frac_hbm_cold": qp_bytes / t_qp_cold / 1e9 / HBM_PEAK_GBS},
            # the raw-input GEMM of the step (back to back), and the pre-scaled
            # pair it replaces for fp16 input (ttq_prescale + ttq_wlowbit_gemm,
            # still the path for fp32 input)
            "wlowbit_gemm_raw": {"us": t_gm * 1e6, "TFLOPs": gm_flops / t_gm / 1e12,
                                 "frac_mfma": gm_flops / t_gm / 1e12 / MFMA_F16_PEAK_TFLOPS},
            # the whole prepare step (colstats, quantize_pack and, for a
            # handle with room for it, the effective weight), graph replay
            "prepare": {"us": t_prep * 1e6, "k_tok_s": T / t_prep / 1e3},
            "prescale": {"us": t_ps * 1e6, "GBs": ps_bytes / t_ps / 1e9,
                         "frac_hbm": ps_bytes / t_ps / 1e9 / HBM_PEAK_GBS},
            "wlowbit_gemm_prescaled": {"us": t_gm_pre * 1e6, "TFLOPs": gm_flops / t_gm_pre / 1e12,
                                       "frac_mfma": gm_flops / t_gm_pre / 1e12 / MFMA_F16_PEAK_TFLOPS},
            "gemm_in_step": {"us": t_gm_step * 1e6, **gm_pct, "TFLOPs": gm_flops / t_gm_step / 1e12,
                             "frac_mfma": gm_flops / t_gm_step / 1e12 / MFMA_F16_PEAK_TFLOPS,
                             "kernel": "dense_gemm_kernel" if dense else "wlowbit_gemm_kernel"},
        }
        # the dense form of the step (a handle given room for W_hat)
        kernels["dense_gemm"] = {"us": t_dg * 1e6, "TFLOPs": gm_flops / t_dg / 1e12,
                                 "frac_mfma": gm_flops / t_dg / 1e12 / MFMA_F16_PEAK_TFLOPS,
                                 "step_ms": t_step_d * 1e3, "step_k_tok_s": T / t_step_d / 1e3}
        # context: torch's dense fp16 GEMM (hipBLASLt) of the same shape on the
        # same activations, i.e. what an unquantised q_proj costs on this GPU
        Wd = torch.randn((d_out, d), dtype=torch.float16, device="cuda") * 0.01
        for _ in range(3):
            torch.nn.functional.linear(X, Wd)
        t_dense = time_loop(lambda: torch.nn.functional.linear(X, Wd), n_k, torch)
        kernels["dense_fp16_gemm_context"] = {"us": t_dense * 1e6, "TFLOPs": gm_flops / t_dense / 1e12}
        del Wd
        log(f"bench: kernels {json.dumps(kernels)}")

    # ---- a plain copy of known size: calibrates the byte counters ----
    if "copy" in only:
        nbytes = 512 << 20
        src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"bench: copied {nbytes} bytes 3 times")
        del src, dst

    # ---- r = 16: the same step with the rank-16 factors ----
    r16 = None
    if "r16" in only:
        rng = np.random.default_rng(5)
        log("bench: host SVD for r=16")
        B, A = ttq.svd_factors(W_np, 16)
        layer16 = ttq.TTQLinear(W, q=q, g=g, alpha=w.alpha, lam=w.lam, p=w.p, r=16, T_max=T, B=B, A=A)

        def step16():
            # ttq_prefill: with r = 16 the column statistic and Z = X A^T come
            # from one read of X
            layer16.prefill(X, out=Y)
        settle(step16, args.settle_ms, torch)
        for _ in range(args.warmup):
            step16()
        t16 = time_loop(step16, args.steps, torch)
        Zbuf = torch.empty((T, 16), dtype=torch.float32, device="cuda")
        # graph replays: an eager call's host side takes about as long as
        # these kernels
        t_z = time_graph(lambda: ttq.ttq_lowrank_z(X, layer16.A, out=Zbuf), n_k, torch)
        t_p16 = time_graph(lambda: layer16.prepare(X), n_k, torch)
        r16 = {"value": T / t16 / 1e3, "ms_per_step": t16 * 1e3, "lowrank_z_us": t_z * 1e6,
               "prepare_us": t_p16 * 1e6}
        layer16.close()
        # the same step with the online refresh of the rank-16 factors: per
        # prompt one subspace-iteration step from the previous right basis,
        # then W_res and its quantisation, then the projection
        log("bench: r=16 with the online refresh")
        layerR = ttq.TTQLinear(W, q=q, g=g, alpha=w.alpha, lam=w.lam, p=w.p, r=16, T_max=T, refresh=True)

        def stepR():
            layerR.prefill(X, out=Y)
        settle(stepR, args.settle_ms, torch)
        for _ in range(args.warmup):
            stepR()
        tR = time_loop(stepR, args.steps, torch)
        t_pR = time_graph(lambda: layerR.prepare(X), n_k, torch)
        r16["refresh"] = {"value": T / tR / 1e3, "ms_per_step": tR * 1e3, "prepare_us": t_pR * 1e6}
        layerR.close()
        del rng

    # ---- other code widths and group sizes on the same prompt and weight ----
    # (the same step, r = 0: prepare + projection, settled and timed like the
    # headline; the quantize_pack and GEMM kernels alone by their own events)
    variants = None
    if "variants" in only:
        variants = {}
        for qv, gv in ((2, 32), (3, 32), (5, 32), (4, 16), (4, 64), (4, 128)):
            lv = ttq.TTQLinear(W, q=qv, g=gv, alpha=w.alpha, lam=w.lam, p=w.p, r=0, T_max=T)

            def step_v():
                lv.prepare(X)
                lv.linear(X, out=Y)
            settle(step_v, args.settle_ms / 4, torch)
            t_v = time_loop(step_v, args.steps, torch)
            t_q = time_graph(lambda: ttq.ttq_quantize_pack(W, lv.D, qv, gv, lv.codes, lv.scales, lv.zeros),
                             10, torch)
            t_g = time_loop(lambda: ttq.ttq_wlowbit_gemm_raw(X, lv.dinvsqrt16, lv.codes, lv.scales, lv.zeros, qv,
                                                             gv, d_out, out=Y), 10, torch)
            # one decode token reusing this quantisation (graph replay)
            X1 = torch.from_numpy(wl.decode_inputs(w.cfg, 1, step=1)).cuda()
            Y1 = torch.empty((1, d_out), dtype=torch.float16, device="cuda")
            t_d1 = time_graph(lambda: lv.linear(X1, out=Y1), 20, torch)
            d1_b = qv * d_out * d // 8 + 4 * d_out * d // gv + 2 * (d + d_out) + 4 * d
            qp_b = 2 * d_out * d + 4 * d + qv * d_out * d // 8 + 4 * d_out * d // gv
            variants[f"q{qv}_g{gv}"] = {
                "k_tok_s": T / t_v / 1e3, "ms_per_step": t_v * 1e3,
                "quantize_pack_us": t_q * 1e6, "quantize_pack_frac_hbm": qp_b / t_q / 1e9 / HBM_PEAK_GBS,
                "gemm_us_back_to_back": t_g * 1e6,
                "gemm_frac_mfma_back_to_back": gemm_flops / t_g / 1e12 / MFMA_F16_PEAK_TFLOPS,
                "decode_1_us": t_d1 * 1e6, "decode_1_frac_hbm": d1_b / t_d1 / 1e9 / HBM_PEAK_GBS}
            lv.close()
        log(f"bench: variants {json.dumps(variants)}")

    # ---- the other layer shapes of the pages' models (OPT-125M, OPT-350M,
    # Qwen3-1.7B, Qwen3-8B q_proj) with their own q, g, alpha and r: the same
    # step, its kernels alone, and the projection's duration inside the
    # steps (events around ttq_linear; for r = 16 and fp16 input it also
    # launches the Z pass, reported on its own) ----
    configs = None
    if "configs" in only:
        configs = {}
        for cfg, r_c in ((1, 0), (2, 16), (3, 0), (4, 0), (4, 16)):
            wc = wl.CONFIGS[cfg]
            qc, gc = wc.q[0], wc.g[0]
            Xc_np, Wc_np = wl.config_inputs(cfg)
            Xc = torch.from_numpy(Xc_np).cuda()
            Wc = torch.from_numpy(Wc_np).cuda()
            Bc = Ac = None
            if r_c:
                Bc, Ac = ttq.svd_factors(Wc_np, r_c)
            lc = ttq.TTQLinear(Wc, q=qc, g=gc, alpha=wc.alpha, lam=wc.lam, p=wc.p, r=r_c, T_max=wc.T, B=Bc, A=Ac)
            Yc = torch.empty((wc.T, wc.d_out), dtype=Xc.dtype, device="cuda")

            def step_c():
                lc.prepare(Xc)
                lc.linear(Xc, out=Yc)
            settle(step_c, args.settle_ms / 4, torch)
            evc = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(args.steps)]
            torch.cuda.synchronize()
            t0c = time.perf_counter()
            for e0, e1 in evc:
                lc.prepare(Xc)
                e0.record(s)
                lc.linear(Xc, out=Yc)
                e1.record(s)
            torch.cuda.synchronize()
            t_c = (time.perf_counter() - t0c) / args.steps
            t_lin = sum(e0.elapsed_time(e1) for e0, e1 in evc) / len(evc) * 1e-3
            t_cs_c = time_graph(lambda: ttq.ttq_colstats(Xc, wc.p, wc.lam, wc.alpha, D=lc.D, dinvsqrt=lc.dinvsqrt,
                                                         workspace=lc.workspace), 10, torch)
            Wq = lc.wres if r_c else Wc
            t_qp_c = time_graph(lambda: ttq.ttq_quantize_pack(Wq, lc.D, qc, gc, lc.codes, lc.scales, lc.zeros),
                                10, torch)
            fl = 2.0 * wc.T * wc.d * wc.d_out
            xb = Xc.element_size()
            cs_b = wc.T * wc.d * xb + 8 * wc.d
            qp_b = 2 * wc.d_out * wc.d + 4 * wc.d + qc * wc.d_out * wc.d // 8 + 4 * wc.d_out * wc.d // gc
            configs[f"{wc.name}_q{qc}g{gc}r{r_c}"] = {
                "d": wc.d, "d_out": wc.d_out, "T": wc.T, "x_dtype": wc.x_dtype,
                "k_tok_s": wc.T / t_c / 1e3, "ms_per_step": t_c * 1e3,
                "colstats_us": t_cs_c * 1e6, "colstats_frac_hbm": cs_b / t_cs_c / 1e9 / HBM_PEAK_GBS,
                "quantize_pack_us": t_qp_c * 1e6, "quantize_pack_frac_hbm": qp_b / t_qp_c / 1e9 / HBM_PEAK_GBS,
                "linear_us_in_step": t_lin * 1e6,
                "linear_frac_mfma_in_step": fl / t_lin / 1e12 / MFMA_F16_PEAK_TFLOPS}
            lc.close()
            del Xc, Wc, Yc
        log(f"bench: configs {json.dumps(configs)}")

    # ---- q, k, v of one layer sharing one prepare (GQA: k, v have 1024 rows) ----
    qkv = None
    if "qkv" in only:
        Wk = torch.from_numpy(wl.weight(w.cfg, 1024, d, w.w_sigma, part=1)).cuda()
        Wv = torch.from_numpy(wl.weight(w.cfg, 1024, d, w.w_sigma, part=2)).cuda()
        Wqkv = torch.cat([W, Wk, Wv]).contiguous()
        kw = dict(q=q, g=g, alpha=w.alpha, lam=w.lam, p=w.p, r=0, T_max=T)
        fused = ttq.TTQLinear(Wqkv, **kw)
        sep = [ttq.TTQLinear(Wi, **kw) for Wi in (W, Wk, Wv)]
        Yqkv = torch.empty((T, Wqkv.shape[0]), dtype=torch.float16, device="cuda")
        Ys = [torch.empty((T, Wi.shape[0]), dtype=torch.float16, device="cuda") for Wi in (W, Wk, Wv)]

        def step_fused():
            fused.prepare(X)
            fused.linear(X, out=Yqkv)

        def step_sep():
            for layer_i, Yi in zip(sep, Ys):
                layer_i.prepare(X)
                layer_i.linear(X, out=Yi)
        settle(step_fused, args.settle_ms / 2, torch)
        t_f = time_loop(step_fused, args.steps, torch)
        settle(step_sep, args.settle_ms / 2, torch)
        t_s = time_loop(step_sep, args.steps, torch)
        qkv = {"d_out": [d_out, 1024, 1024], "fused_k_tok_s": T / t_f / 1e3, "fused_ms": t_f * 1e3,
               "separate_k_tok_s": T / t_s / 1e3, "separate_ms": t_s * 1e3}
        fused.close()
        for layer_i in sep:
            layer_i.close()
        del Wqkv, Yqkv, Ys, Wk, Wv

    # ---- decode: reuse the prefill quantisation for T = 1, 16, 64 ----
    decode = {}
    if "decode" in only:
        layer.prepare(X)
        for Td in w.decode_T:
            Xn = torch.from_numpy(wl.decode_inputs(w.cfg, Td, step=Td)).cuda()
            Yn = torch.empty((Td, d_out), dtype=torch.float16, device="cuda")
            for _ in range(3):
                layer.linear(Xn, out=Yn)
            # one decode call = ttq_linear (prescale + split-K kernel); graph
            # replay times the GPU side, eager calls include the host's call cost
            td = time_graph(lambda: layer.linear(Xn, out=Yn), 50, torch)
            td_eager = time_loop(lambda: layer.linear(Xn, out=Yn), 50, torch)
            wbytes = q * d_out * d / 8 + 4 * d_out * d / g + 2 * Td * (d + d_out) + 4 * d
            decode[str(Td)] = {"k_tok_s": Td / td / 1e3, "us": td * 1e6, "us_eager": td_eager * 1e6,
                               "GBs": wbytes / td / 1e9, "frac_hbm": wbytes / td / 1e9 / HBM_PEAK_GBS}
        # cold: 12 layers with their own packed weights (12 x 26 MB = 315 MB, more
        # than the 256 MB Infinity Cache and the 8 x 4 MB L2) called in turn, so
        # every call streams its weight from HBM; the calls above reuse one
        # layer's 26 MB, which the Infinity Cache can hold
        n_cold = 12
        cold_layers = []
        Xp = X[:64].contiguous()
        for _ in range(n_cold):
            lc = ttq.TTQLinear(W, q=q, g=g, alpha=w.alpha, lam=w.lam, p=w.p, r=0, T_max=64)
            lc.prepare(Xp)
            cold_layers.append(lc)
        for Td in w.decode_T:
            Xn = torch.from_numpy(wl.decode_inputs(w.cfg, Td, step=Td)).cuda()
            Yn = torch.empty((Td, d_out), dtype=torch.float16, device="cuda")

            def calls():
                for lc in cold_layers:
                    lc.linear(Xn, out=Yn)
            tc = time_graph(calls, 4, torch) / n_cold
            wbytes = q * d_out * d / 8 + 4 * d_out * d / g + 2 * Td * (d + d_out) + 4 * d
            decode[str(Td)].update({"us_cold": tc * 1e6, "frac_hbm_cold": wbytes / tc / 1e9 / HBM_PEAK_GBS})
        for lc in cold_layers:
            lc.close()
        del cold_layers

    # ---- CPU oracle baseline on a bounded sample ----
    cpu = None
    if not args.skip_cpu:
        import oracle
        cores = len(os.sched_getaffinity(0))
        try:
            from threadpoolctl import threadpool_info
            pools = threadpool_info()
            blas_threads = max([i.get("num_threads", 1) for i in pools] or [1])
            blas_name = ",".join(sorted({str(i.get("internal_api", "?")) for i in pools})) or "?"
        except Exception:
            blas_threads, blas_name = cores, "?"
        log("bench: timing the CPU oracle")
        t0 = time.perf_counter()
        D0 = oracle.colstats(X_np, w.p, w.lam, w.alpha)
        c0, s0, z0 = oracle.quantize(W_np, D0, q, g)
        oracle.device_codes(c0, q)
        t_prep = time.perf_counter() - t0
        n_tok = T
        t0 = time.perf_counter()
        oracle.linear(X_np[:n_tok], c0, s0, z0, D0, g)
        t_lin = time.perf_counter() - t0
        t_cpu = t_prep + t_lin * T / n_tok
        cpu = {"value": T / t_cpu / 1e3, "unit": "k tokens/s", "cores": int(max(1, blas_threads)),
               "kind": "oracle",
               "sample": (f"one full step of the workload: prepare (colstats + quantize + pack) on the "
                          f"{T}-token prompt ({t_prep:.2f} s) and the fp64 projection of all {n_tok} tokens "
                          f"({t_lin:.2f} s); numpy with {blas_name} ({blas_threads} threads), {cores} cores visible")}

    out = {
        "metric": "q_proj prefill k tokens/s (prepare+GEMM) at 4-bit r=0/16; % HBM/MFMA peak",
        "value": value,
        "unit": "k tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms": args.settle_ms,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "Qwen3-32B q_proj prefill, one prompt", "d": d, "d_out": d_out, "T": T,
                   "q": q, "g": g, "r": 0, "alpha": w.alpha, "lambda": w.lam, "p": w.p,
                   "x_dtype": "f16"},
    }
    if "roofline" in result:
        out["roofline"] = result["roofline"]
        out["projection_k_tok_s"] = result["projection_k_tok_s"]
        out["prepare_k_tok_s"] = result["prepare_k_tok_s"]
        out["prepare_us_in_step"] = result["prepare_us_in_step"]
    if cpu is not None:
        out["cpu_baseline"] = cpu
    if r16 is not None:
        out["r16"] = r16
    if kernels:
        out["kernels"] = kernels
    if decode:
        out["decode"] = decode
    if qkv is not None:
        out["qkv_shared_prepare"] = qkv
    if variants is not None:
        out["variants"] = variants
    if configs is not None:
        out["configs"] = configs
    print(json.dumps(out), flush=True)
    layer.close()


if __name__ == "__main__":
    main()
