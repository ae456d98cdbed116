"""Benchmark of the MoE-layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload main_bf16] [--no-cpu-baseline]
                    [--cpu-sample-tokens 4096] [--no-backward] [--no-cold-cache]

One step = one moe_forward call (router, dispatch, both grouped GEMMs, combine, aux loss) over
the workload's seeded synthetic batch, with inputs already resident in HBM. W untimed steps,
then exactly K timed steps between two device synchronisations, each after a 1 GiB write that
evicts the L2s and the Infinity Cache, timed by HIP events around the step alone (the
throughput: cold cache); K more after a read of that buffer instead are reported apart
(cold_cache_read_flush: then no write-back of the flush's dirty lines falls inside the step).
Then K warm steps back to back between two synchronisations (reported as warm_cache), then K
more with HIP events recorded by the library between its kernels on the launch stream (the
per-kernel durations and the roofline; the events themselves add a few microseconds per step).
Then the backward leg (unless --no-backward): moe_backward timed over W + K calls, in the
layer's own configuration and with keep_preact (the training setting, whose forward is timed
too).

Prints one JSON line: tokens/s of the whole layer, the roofline of the dominant kernel (the
slower grouped GEMM: MFMA bound on the large workloads, HBM bound when a few tokens per expert
make it a pass over the expert weights), the CPU oracle timed single-threaded on a bounded
sample of the same workload on the host, and the parity of this run's output against the oracle
on the whole workload (with the near-tie count).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer fwd tokens/sec + grouped-GEMM TFLOP/s (% bf16 MFMA peak), E=8 top-2"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3        # MI355X dense fp32 MFMA
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=4096,
                    help="tokens of the single-threaded CPU-oracle sample (0 = the whole workload)")
    ap.add_argument("--no-cold-cache", action="store_true",
                    help="time warm steps only (the hardware-counter runs use this: their per-dispatch bytes are "
                         "those of warm steps, like the roofline's durations)")
    ap.add_argument("--backward", action="store_true",
                    help="kept for older command lines: the backward leg runs by default")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the backward leg (moe_backward timed the same way, in a 'backward' object)")
    ap.add_argument("--no-vendor-gemm", action="store_true",
                    help="skip the vendor dense-GEMM reference (torch.matmul on the two layers' shapes)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after the timed steps, run one elementwise copy of this many MiB (a known-size "
                         "kernel to scale hardware byte counters against)")
    return ap.parse_args()


def recorded_traffic(workload: str, kernel: str):
    """HBM-side bytes per dispatch (FETCH_SIZE + WRITE_SIZE, calibrated) recorded in
    profiles/traffic_<workload>.txt for `kernel`, or None when no record exists or the grouped
    GEMM sources have changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        if line.startswith("# ") and ":" in line:
            k, v = line[2:].split(":", 1)
            rec[k.strip()] = v.strip()
    from sparse_mixture_experts_02_amd.rocprof_summary import gemm_sources_digest
    if rec.get("grouped GEMM sources sha256") != gemm_sources_digest():
        return None
    try:
        return int(rec[f"{kernel} fetch_bytes"]) + int(rec[f"{kernel} write_bytes"])
    except KeyError:
        return None


def host_cpu() -> dict:
    """The host the oracle runs on: CPU model, the cores this process may use, the machine's count."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count()
    return {"cpu_model": model, "nproc": usable, "cpu_count": os.cpu_count()}


def oracle_layer(w, inp, ntok: int, logits=None):
    """The oracle's steps one by one on the first `ntok` tokens of the workload (all weights):
    returns (out, aux, routing, per-step seconds). With `logits`, routing runs on those fp32
    logits (the parity protocol's routing "given the fp32 router logits")."""
    import oracle
    x = inp["x"][:ntok]
    g = inp["gumbel"][:ntok] if inp["gumbel"] is not None else None
    m = inp["token_mask"][:ntok].numpy() if inp["token_mask"] is not None else None
    C = oracle.capacity_from_factor(ntok, w.top_k, w.num_experts, w.capacity_factor)
    w1, w2 = inp["w1"], inp["w2"]
    if w.weight_dtype == "int4":   # the 4-bit layer: its dequantised weights (quantising is not timed)
        w1 = oracle.dequantize_int4(*oracle.quantize_int4(w1))
        w2 = oracle.dequantize_int4(*oracle.quantize_int4(w2))
    secs = {}
    t = time.perf_counter()
    r = oracle.route(x, inp["w_router"], inp["bias"], g, w.temperature, w.top_k, w.renormalize, logits,
                     noise_in_logits=w.router_noise > 0.0, token_mask=m, straight_through=w.straight_through)
    secs["route"] = time.perf_counter() - t
    t = time.perf_counter()
    dp = oracle.dispatch(r.ids, w.num_experts, C, x)
    secs["dispatch"] = time.perf_counter() - t
    t = time.perf_counter()
    _, y = oracle.expert_ffn(dp.xp, dp.offsets, w1, w2, w.dtype)
    ys = None
    if inp["w1_shared"] is not None:
        _, ys = oracle.shared_ffn(x, inp["w1_shared"], inp["w2_shared"], w.dtype)
    secs["expert_ffn"] = time.perf_counter() - t
    t = time.perf_counter()
    out = oracle.combine(y, dp.row_of, r.weights, w.dtype, d=w.d_model, y_shared=ys)
    secs["combine"] = time.perf_counter() - t
    t = time.perf_counter()
    aux = oracle.aux_loss(r.probs, dp.counts_pre, w.top_k, w.aux_coef, r.real, r.entropy)
    secs["aux"] = time.perf_counter() - t
    return out, aux, r, secs


def cpu_leg(w, inp, gpu: dict, sample_tokens: int):
    """The CPU oracle beside the GPU: (cpu_baseline, parity).

    cpu_baseline: the oracle as it stands, single-threaded (one BLAS thread), on the first
    `sample_tokens` tokens of the workload, step by step; tokens/s of the sample.
    parity: the oracle on the whole workload (all host threads), routed from its own fp32 logits;
    the near-tie count (tokens whose k-th and (k+1)-th keys differ by less than 1e-4), the expert
    ids against the GPU's, and the GPU output and aux values against the oracle's (normwise
    output error against 2e-2 for bf16 and 1e-5 for fp32; aux relative error against 1e-5). When
    any token's ids differ (a near tie resolved the other way), the oracle is run again routed
    from the GPU's logits, so that the outputs compare the same routing."""
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_info, threadpool_limits
    host = host_cpu()
    ntok = w.T if sample_tokens <= 0 else min(sample_tokens, w.T)
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        _, _, _, secs = oracle_layer(w, inp, ntok)
        dt = time.perf_counter() - t0
    baseline = {"value": ntok / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
                "sample": f"first {ntok} of {w.T} tokens of {w.name} with all expert weights, capacity for "
                          f"{ntok} tokens (oracle steps in float64, numpy/OpenBLAS on 1 thread); {dt:.2f} s",
                "step_seconds": secs, **host}
    threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    t0 = time.perf_counter()
    out, aux, r, secs_full = oracle_layer(w, inp, w.T)
    dt_full = time.perf_counter() - t0
    baseline["whole_workload"] = {"seconds": dt_full, "threads": threads, "tokens_per_s": w.T / dt_full,
                                  "step_seconds": secs_full}
    real = r.real
    gap = oracle.topk_gap(r.keys, w.top_k)
    near = (gap < 1e-4) & real
    gids = gpu["ids"].numpy()
    differ = np.any(gids != r.ids, axis=1)
    par = {"near_tie_tokens": int(near.sum()), "ids_differ_clear_gap": int(np.sum(differ & ~near)),
           "ids_differ_near_tie": int(np.sum(differ & near)), "routing": "oracle's own logits"}
    if differ.any():
        out, aux, _, _ = oracle_layer(w, inp, w.T, logits=gpu["logits"].numpy())
        par["routing"] = "the GPU's fp32 logits (ids differ on near ties)"
    go = gpu["out"].float().numpy().astype(np.float64)
    m = float(np.max(np.abs(out)))
    err = float(np.max(np.abs(go - out)) / m) if m > 0 else float(np.max(np.abs(go)))
    tol = 2e-2 if w.dtype == "bf16" else 1e-5
    ga = gpu["aux"].numpy().astype(np.float64)
    rel = [abs(a - b) / max(abs(b), 1e-30) if abs(a - b) > 1e-12 else 0.0 for a, b in zip(ga, aux)]
    par.update(out_normwise_error=err, out_tol=tol, aux_rel_error=rel, aux_tol=1e-5, tokens_checked=w.T,
               passed=bool(err <= tol and max(rel) <= 1e-5 and par["ids_differ_clear_gap"] == 0))
    return baseline, par


def bench_backward(args, w, cfg, dev, ws, N: int) -> dict:
    """moe_backward over a forward pass's workspace: W untimed then K timed calls between two
    device synchronisations, each producing dx and every weight gradient (router, bias, W1, W2,
    the shared expert's). Two configurations: the layer's own (the backward recomputes the
    pre-activation Xp W1^T) and keep_preact (the training setting: the forward keeps it, so the
    backward skips that grouped GEMM); for the latter the forward is timed too."""
    import dataclasses

    import torch

    import sparse_mixture_experts_02_amd as moe
    if cfg.int4:
        return {"skipped": "4-bit expert weights have no backward"}
    T, d, f, E = w.T, w.d_model, w.d_ffn, w.num_experts
    fs = w.d_ffn_shared
    dt = cfg.torch_dtype
    gen = torch.Generator().manual_seed(5)
    d_out = torch.randn(T, d, generator=gen).to(dt).cuda()
    z = lambda *shape: torch.empty(*shape, dtype=torch.float32, device="cuda")
    grads = {"dw_router": z(E, d), "dbias": z(E), "dw1": z(E, f, d), "dw2": z(E, d, f)}
    if fs:
        grads.update(dw1_shared=z(fs, d), dw2_shared=z(d, fs))
    dx = torch.empty(T, d, dtype=dt, device="cuda")
    out = torch.empty(T, d, dtype=dt, device="cuda")
    aux = torch.empty(3, dtype=torch.float32, device="cuda")

    def fwd(c, wsp):
        moe.moe_forward(c, dev["x"], dev["w_router"], dev["w1"], dev["w2"], out, aux, wsp, bias=dev["bias"],
                        gumbel=dev["gumbel"], token_mask=dev["token_mask"], w1_shared=dev["w1_shared"],
                        w2_shared=dev["w2_shared"])

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / args.steps

    def bwd(c, wsp, bws):
        moe.moe_backward(c, dev["x"], dev["w_router"], dev["w1"], dev["w2"], d_out, wsp, dx, bws,
                         token_mask=dev["token_mask"], w1_shared=dev["w1_shared"], w2_shared=dev["w2_shared"],
                         d_aux=1.0, **grads)

    # the layer's own configuration: a forward without debug outputs leaves every intermediate
    fwd(cfg, ws)
    bws = moe.new_backward_workspace(cfg)
    ms = timed(lambda: bwd(cfg, ws, bws))
    # the training configuration
    cfg_t = dataclasses.replace(cfg, keep_preact=True)
    ws_t = moe.new_workspace(cfg_t)
    fwd_t_ms = timed(lambda: fwd(cfg_t, ws_t))
    fwd(cfg_t, ws_t)
    bwd_t_ms = timed(lambda: bwd(cfg_t, ws_t, bws))
    # the backward's matrix products: the pre-activation Xp W1^T (recomputed unless kept), dH, dXp,
    # dW2 and dW1 of the routed experts (2 N d f flop each), and the shared expert's five of 2 T d fs
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    flop = 5 * 2.0 * N * d * f + 5 * 2.0 * T * d * fs
    flop_t = 4 * 2.0 * N * d * f + 5 * 2.0 * T * d * fs
    return {"ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3), "matmul_flop": flop,
            "matmul_tflops": flop / (ms * 1e-3) / 1e12, "frac_of_peak": flop / (ms * 1e-3) / 1e12 / peak,
            "keep_preact": {"forward_ms": fwd_t_ms, "backward_ms": bwd_t_ms, "training_step_ms": fwd_t_ms + bwd_t_ms,
                            "training_tokens_per_s": T / ((fwd_t_ms + bwd_t_ms) * 1e-3),
                            "backward_matmul_tflops": flop_t / (bwd_t_ms * 1e-3) / 1e12},
            "steps": args.steps, "warmup": args.warmup}


def vendor_gemm(N: int, d: int, f: int, steps: int) -> dict:
    """The vendor library's dense GEMM (torch.matmul, which runs hipBLASLt) on the two layers'
    shapes, for context beside the grouped kernels: [N, d] x [d, f] and [N, f] x [f, d] in bf16 with
    fp32 accumulation, the operands drawn like the layer's (activations N(0, 1), weights
    N(0, 0.02^2), the second product's left operand the SiLU of the first's output), one weight
    matrix for all N rows (the grouped kernels use one per expert segment). Warm cache, K
    launches back to back between two HIP events. Not part of the layer."""
    import torch
    gen = torch.Generator(device="cuda").manual_seed(5)
    a = torch.randn(N, d, device="cuda", generator=gen).to(torch.bfloat16)
    w1 = (torch.randn(d, f, device="cuda", generator=gen) * 0.02).to(torch.bfloat16)
    w2 = (torch.randn(f, d, device="cuda", generator=gen) * 0.02).to(torch.bfloat16)
    h = torch.nn.functional.silu(torch.matmul(a, w1).float()).to(torch.bfloat16)
    res = {"library": "torch.matmul (hipBLASLt), dense, one weight matrix",
           "protocol": "warm cache: K launches back to back between two HIP events"}
    for name, x, wt in (("gemm1_shape", a, w1), ("gemm2_shape", h, w2)):
        for _ in range(3):
            torch.matmul(x, wt)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            torch.matmul(x, wt)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        tflops = 2.0 * N * x.shape[1] * wt.shape[1] / (ms * 1e-3) / 1e12
        res[name] = {"m_n_k": [N, int(wt.shape[1]), int(x.shape[1])], "ms": ms, "tflops": tflops,
                     "frac_of_bf16_peak": tflops / PEAK_BF16_TFLOPS}
    del a, w1, w2, h
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the layer has no multi-GPU path here.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import sparse_mixture_experts_02_amd as moe
    from sparse_mixture_experts_02_amd.binding import FORWARD_KERNEL_NAMES, MOE_FORWARD_NUM_KERNELS
    from sparse_mixture_experts_02_amd.inputs import MAIN, WORKLOADS, inputs_digest, make_inputs

    name = args.workload or MAIN
    w = WORKLOADS[name]
    torch.cuda.set_device(0)
    inp = make_inputs(w)
    digest = inputs_digest(inp)
    dev = {k: (v.cuda() if v is not None else None) for k, v in inp.items()}
    cfg = moe.config_for(w)
    if cfg.int4:   # 4-bit expert weights: packed once on the GPU, before anything is timed
        dev["w1"] = moe.quantize_int4(dev["w1"])
        dev["w2"] = moe.quantize_int4(dev["w2"])
    ws = moe.new_workspace(cfg)
    out = torch.empty(w.T, w.d_model, dtype=cfg.torch_dtype, device="cuda")
    aux = torch.empty(3, dtype=torch.float32, device="cuda")
    offsets = torch.empty(w.num_experts + 1, dtype=torch.int32, device="cuda")
    nd = torch.empty(1, dtype=torch.int32, device="cuda")
    nev = MOE_FORWARD_NUM_KERNELS + 1
    events = [moe.HipEvents(nev) for _ in range(args.steps)]

    def step(ev=None):
        moe.moe_forward(cfg, dev["x"], dev["w_router"], dev["w1"], dev["w2"], out, aux, ws, bias=dev["bias"],
                        gumbel=dev["gumbel"], token_mask=dev["token_mask"], w1_shared=dev["w1_shared"],
                        w2_shared=dev["w2_shared"], debug={"offsets": offsets, "n_dropped": nd}, events=ev)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    cold_ms = cold_read_ms = None
    if not args.no_cold_cache:
        # the timed steps, cold cache: before each step a 1 GiB write evicts the L2s and the
        # 256 MB Infinity Cache, and HIP events on the launch stream bracket the step alone (the
        # flush is outside them); exactly K steps between two device synchronisations. Then K
        # more the same way after a read of the buffer instead (reported apart): after the write
        # the step also writes back the flush's dirty lines, ~35-40 us of the main layer's step
        flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")

        def cold_steps(write: bool):
            ev0 = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
            ev1 = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
            torch.cuda.synchronize()
            for i in range(args.steps):
                if write:
                    flush.fill_(float(i))
                else:
                    flush.amax()   # read for its cache effect only
                ev0[i].record()
                step()
                ev1[i].record()
            torch.cuda.synchronize()
            return np.array([a.elapsed_time(b) for a, b in zip(ev0, ev1)])

        cold_ms = cold_steps(True)
        cold_read_ms = cold_steps(False)
        del flush
    # warm cache: K steps back to back between two device synchronisations (forward passes only:
    # recording the per-kernel events costs a few microseconds per event on the GPU timeline)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    warm_ms_per_step = (t1 - t0) * 1e3 / args.steps
    # the same number of steps again with HIP events between the kernels: per-kernel durations
    t2 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    t3 = time.perf_counter()
    ms_per_step_events = (t3 - t2) * 1e3 / args.steps
    ms_per_step = float(cold_ms.mean()) if cold_ms is not None else warm_ms_per_step

    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.mul(src, 1.0, out=dst)   # reads n*4 bytes, writes n*4 bytes
        torch.cuda.synchronize()
        del src, dst

    # the cost of an event interval with no kernel in it (two records back to back on the launch
    # stream): every per-kernel interval carries it, which matters for the short kernels
    gap_ev = moe.HipEvents(2 * args.steps)
    for i in range(args.steps):
        gap_ev.record(2 * i)
        gap_ev.record(2 * i + 1)
    torch.cuda.synchronize()
    event_gap_ms = float(np.median([gap_ev.elapsed_ms(2 * i, 2 * i + 1) for i in range(args.steps)]))
    gap_ev.close()

    per_kernel = np.zeros((args.steps, MOE_FORWARD_NUM_KERNELS))
    warm_ms = np.zeros(args.steps)
    for i, ev in enumerate(events):
        for j in range(MOE_FORWARD_NUM_KERNELS):
            per_kernel[i, j] = ev.elapsed_ms(j, j + 1)
        warm_ms[i] = ev.elapsed_ms(0, MOE_FORWARD_NUM_KERNELS)
        ev.close()
    kms_raw = per_kernel.mean(axis=0)
    kms = np.maximum(kms_raw - event_gap_ms, 0.0)   # net of the event interval's own cost
    N = int(offsets[-1].item())
    n_dropped = int(nd.item())

    T, d, f = w.T, w.d_model, w.d_ffn
    a = 2 if w.dtype == "bf16" else 4
    flop_gemm = 2.0 * N * d * f                     # per grouped GEMM launch
    names = list(FORWARD_KERNEL_NAMES)
    t_g1 = kms[names.index("gemm1_silu")] * 1e-3
    t_g2 = kms[names.index("gemm2")] * 1e-3
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    dom = "gemm1_silu" if t_g1 >= t_g2 else "gemm2"          # the dominant kernel
    t_dom = max(t_g1, t_g2)
    dom_tflops = flop_gemm / t_dom / 1e12
    # algorithmic bytes of one grouped GEMM launch: its activations in and out once, every expert's
    # weight matrix once
    wbytes = (0.5 + 2.0 / 64) if cfg.int4 else a   # bytes per expert weight (4-bit: codes + bf16 scales)
    gemm_bytes = N * d * a + w.num_experts * d * f * wbytes + N * f * a
    # a launch whose flop per byte is below the machine's ridge point is bound by HBM
    hbm_bound = flop_gemm / gemm_bytes < peak * 1e12 / (PEAK_HBM_GBS * 1e9)
    if hbm_bound:
        roof = {"bound": "hbm", "achieved": gemm_bytes / t_dom / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": dom_tflops, "peak": peak, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    gemm_tflops = 2 * flop_gemm / (t_g1 + t_g2) / 1e12
    t_sh = kms[names.index("shared_ffn")] * 1e-3
    shared_tflops = (4.0 * T * d * w.d_ffn_shared / t_sh / 1e12) if w.d_ffn_shared and t_sh > 0 else None
    dispatch_bytes = T * d * a + N * d * a + 12 * T * w.top_k
    combine_bytes = N * d * a + T * d * a + 8 * T * w.top_k
    t_disp = sum(kms[names.index(n)] for n in ("dispatch_hist", "dispatch_scan_aux", "dispatch_gather")) * 1e-3
    t_comb = kms[names.index("combine")] * 1e-3

    line = {
        "metric": METRIC,
        "value": T / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "timing": ("cold cache: mean of K steps, each after a 1 GiB write that evicts the L2s and the Infinity "
                   "Cache, timed by HIP events on the launch stream around the step alone"
                   if cold_ms is not None else "warm cache: K steps back to back between two synchronisations"),
        "ms_per_step_with_kernel_events": ms_per_step_events,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded Gaussian inputs and random-init weights of the workload's shapes)",
        "config": {"workload": w.name, "T": T, "d_model": d, "d_ffn": f, "num_experts": w.num_experts,
                   "top_k": w.top_k, "capacity": cfg.capacity, "temperature": w.temperature,
                   "gumbel": w.gumbel, "router_bias": w.router_bias, "router_noise": w.router_noise,
                   "padding": w.padding, "d_ffn_shared": w.d_ffn_shared,
                   "expert_weights": "int4" if cfg.int4 else w.dtype, "parallelism": "single GPU"},
        "roofline": {"kernel": dom, **roof, "traffic": recorded_traffic(w.name, dom),
                     "traffic_unit": "bytes per dispatch beyond L2 (FETCH_SIZE+WRITE_SIZE, calibrated)",
                     "algorithmic_bytes": gemm_bytes, "algorithmic_flop": flop_gemm},
        "gemm_tflops": gemm_tflops,
        "gemm_frac_of_peak": gemm_tflops / peak,
        "shared_ffn_tflops": shared_tflops,
        "kernel_ms": {n: float(v) for n, v in zip(names, kms)},
        "kernel_ms_event_intervals": {n: float(v) for n, v in zip(names, kms_raw)},
        "event_gap_ms": event_gap_ms,
        "kernel_ms_note": ("kernel_ms = mean HIP-event interval around each kernel step on the launch stream, less "
                           "event_gap_ms (the median interval between two events recorded back to back); the GB/s "
                           "and the roofline use these net times"),
        "route_gbs": (T * d * a + w.num_experts * d * 4 + T * w.num_experts * 4 * (2 if w.gumbel else 1)
                      + 8 * T * w.top_k) / (kms[names.index("route")] * 1e-3) / 1e9,
        "dispatch_gbs": dispatch_bytes / t_disp / 1e9,
        "combine_gbs": combine_bytes / t_comb / 1e9,
        "cold_cache": None if cold_ms is None else {
            "ms_mean": float(cold_ms.mean()), "ms_median": float(np.median(cold_ms)),
            "ms_p10": float(np.percentile(cold_ms, 10)), "ms_p90": float(np.percentile(cold_ms, 90)),
            "tokens_per_s_median": T / (float(np.median(cold_ms)) * 1e-3),
            "protocol": "1 GiB buffer written before each step (outside the timed events)"},
        "cold_cache_read_flush": None if cold_read_ms is None else {
            "ms_mean": float(cold_read_ms.mean()), "ms_median": float(np.median(cold_read_ms)),
            "tokens_per_s": T / (float(cold_read_ms.mean()) * 1e-3),
            "protocol": "the same, after a read of the 1 GiB buffer instead of a write (the caches then "
                        "hold no dirty lines of the flush, whose write-back otherwise falls inside the step)"},
        "warm_cache": {"ms_per_step": warm_ms_per_step, "tokens_per_s": T / (warm_ms_per_step * 1e-3),
                       "protocol": "K steps back to back between two device synchronisations"},
        "warm_cache_events": {"ms_median": float(np.median(warm_ms)), "ms_p10": float(np.percentile(warm_ms, 10)),
                              "ms_p90": float(np.percentile(warm_ms, 90)),
                              "note": "steps with the per-kernel events, caches warm from the previous step"},
        "kept_rows": N,
        "n_dropped": n_dropped,
        "inputs_sha256": digest,
    }
    if not args.no_backward:
        line["backward"] = bench_backward(args, w, cfg, dev, ws, N)
    # (only where the grouped kernels are matrix-core bound: with a few rows per expert the layer
    # streams E weight matrices where the dense product reads one)
    if (not args.no_vendor_gemm and w.dtype == "bf16" and w.weight_dtype is None and N > 0
            and line["roofline"]["bound"] == "mfma"):
        line["vendor_gemm"] = vendor_gemm(N, w.d_model, w.d_ffn, args.steps)
    if not args.no_cpu_baseline:
        # one more forward with the routing captured (not timed), for the oracle's parity check
        gids = torch.empty(w.T, w.top_k, dtype=torch.int32, device="cuda")
        glog = torch.empty(w.T, w.num_experts, dtype=torch.float32, device="cuda")
        moe.moe_forward(cfg, dev["x"], dev["w_router"], dev["w1"], dev["w2"], out, aux, ws, bias=dev["bias"],
                        gumbel=dev["gumbel"], token_mask=dev["token_mask"], w1_shared=dev["w1_shared"],
                        w2_shared=dev["w2_shared"], debug={"ids": gids, "logits": glog})
        torch.cuda.synchronize()
        gpu = {"ids": gids.cpu(), "logits": glog.cpu(), "out": out.cpu(), "aux": aux.cpu()}
        line["cpu_baseline"], line["parity"] = cpu_leg(w, inp, gpu, args.cpu_sample_tokens)
        line["near_tie_tokens"] = line["parity"]["near_tie_tokens"]
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
