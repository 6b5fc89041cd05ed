#!/usr/bin/env python3
"""Benchmark of the retention hot path on one MI355X.

A step is one ret_chunkwise_fwd call over the 7b-class retention layer (B=1, N=8192, H=16, d_k=256, d_v=512,
chunk 128, bf16 inputs/outputs, xPos rotation, fp32 state out): tokens/s = B*N / step time, with inputs
resident in HBM, from a replayed HIP graph of `steps` calls. Its roofline is the MFMA one: causal-count FLOPs
per call over the dominant kernel's average launch duration (HIP events the library records on the launch
stream, through a caller-owned timer, over the timed region), against the dense bf16 peak; the HBM fraction
of the same kernel is reported beside it.

The same JSON line carries, each with its own roofline:
  * long-sequence (B=1, N=65536, H=8, d=128, chunk 128) and retention-layer-d512 (B=8, N=2048, H=8, d=64,
    chunk 64) chunkwise calls, warm and MALL-cold (each call after a 512 MiB scratch write);
  * the long-sequence workload's 256 decode steps from its final state (steps/s; launch-latency-bound);
  * batched decode (B=128, H=8, d=64, fp32 state, 1024 single-token ret_recurrent_step calls replayed from a
    HIP graph), warm (one 16 MiB state, which the 256 MB Infinity Cache holds between steps) and MALL-cold
    (the graph's steps cycle through 32 distinct states, 512 MiB, so every state read comes from HBM);
  * the multi-scale retention epilogue on the d512 layer's output, and the gradients of each chunkwise
    workload;
  * the fp64 CPU oracle timed on this host on a bounded sample of the 7b-class workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-decode] [--no-epilogue]
                       [--no-backward] [--no-cpu-baseline] [--no-extra] [--no-cold] [--decode-mode MODE]
                       [--decode-steps S] [--copy-calibration]
       python bench.py --record-traffic KEY KERNEL FETCH_DIR WRITE_DIR COPY_FETCH_DIR COPY_WRITE_DIR
The second form (no GPU) records HBM traffic per launch of the kernels whose name contains KERNEL from two
`rocprofv3 --pmc FETCH_SIZE` / `--pmc WRITE_SIZE` runs, scaled by the same counters of `--copy-calibration` runs,
under KEY ("timer name@workload") in profiles/traffic.json.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
METRIC = "retention fwd tokens/sec (chunkwise) + decode steps/sec; % MFMA / HBM peak"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# Chunkwise workloads by name -> key (and seed) in workloads.WORKLOADS
CHUNK_WORKLOADS = {"retention-layer-d512": 2, "7b-class-layer": 4, "long-sequence": 5}
CHUNK_KERNELS = ("ret_rotate_qk", "ret_chunk_seg", "ret_chunk_fused", "ret_chunk_wide", "ret_chunk_dma",
                 "ret_chunk_dma_local", "ret_chunk_dma_scan", "ret_chunk_fused_local", "ret_chunk_fused_scan",
                 "ret_chunk_local", "ret_segment_scan", "ret_chunk_full")


def source_digest() -> str:
    """Digest of the library's sources; counter-based traffic figures are only valid for the sources they came
    from."""
    from linear_recurrent_sequence_amd import build
    return build.source_digest()


def chunk_algorithmic(w, in_bytes=2, out_bytes=2):
    """Bytes and FLOPs the chunkwise op must move / perform for one call over workload w.
    Bytes: read q, k, v once, write o once, write the fp32 final state.
    FLOPs per (token, head): causal minimum (C+1)(dk+dv) + 4 dk dv, and the pages' full-block
    count 2C(dk+dv) + 4 dk dv (chunkwise cost analysis)."""
    toks = w.B * w.N * w.H
    nbytes = toks * ((2 * w.dk + w.dv) * in_bytes + w.dv * out_bytes) + w.B * w.H * w.dk * w.dv * 4
    C = w.chunk
    f_causal = toks * ((C + 1) * (w.dk + w.dv) + 4 * w.dk * w.dv)
    f_pages = toks * (2 * C * (w.dk + w.dv) + 4 * w.dk * w.dv)
    return nbytes, f_causal, f_pages


def decode_algorithmic(B, H, dk, dv, in_bytes=2, out_bytes=2):
    """Per decode step: read + write the fp32 state, read q, k, v, write o; 5 flops per state element."""
    nbytes = B * H * (2 * dk * dv * 4 + (2 * dk + dv) * in_bytes + dv * out_bytes)
    return nbytes, B * H * 5 * dk * dv


def load_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` on `workload` from the recorded FETCH_SIZE / WRITE_SIZE counters, scaled
    by a plain copy's counters; None unless recorded for the current sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            recs = json.load(f)
    except (OSError, ValueError):
        return None
    rec = recs.get("%s@%s" % (kernel, workload)) or recs.get(kernel)
    if not rec or rec.get("workload") != workload or rec.get("source_digest") != source_digest():
        return None
    fetch = rec["fetch_kib_per_launch"] * 1024.0 / rec["copy_factor_fetch"]
    write = rec["write_kib_per_launch"] * 1024.0 / rec["copy_factor_write"]
    return fetch + write


def graph_ms(torch, fn, steps, reps=1):
    """Milliseconds per call of `steps` calls of fn captured into one HIP graph and replayed (HIP events on the
    replay stream; the fastest of `reps` replays)."""
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for _ in range(steps):
                fn()
    torch.cuda.current_stream().wait_stream(s)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = None
    for _ in range(reps):
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        best = ms if best is None else min(best, ms)
    return best


def kernel_times(timer, names, calls):
    out = {}
    for name in names:
        tot, n = timer.query(name)
        if n:
            out[name] = {"avg_us": 1e3 * tot / n, "launches_per_call": n / calls}
    return out


def bench_chunkwise(R, W, torch, wid, steps, warmup, cold_reps=20):
    """One chunkwise workload: warm graph replay, eager calls with per-kernel events, MALL-cold calls."""
    w = W.WORKLOADS[wid]
    q, k, v, _ = W.make_qkv(w)
    dev = lambda x: torch.from_numpy(x).to(torch.bfloat16).cuda()
    qd, kd, vd = dev(q), dev(k), dev(v)
    del q, k, v
    o = torch.empty((w.B, w.N, w.H, w.dv), dtype=torch.bfloat16, device="cuda")
    state = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device="cuda")
    ws = R.chunkwise_workspace(qd, vd, w.chunk)

    def step(options=None):
        R.ret_chunkwise_fwd(qd, kd, vd, o, w.gamma, w.chunk, theta=w.theta, state_out=state, workspace=ws,
                            options=options)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # the timed region: `steps` calls replayed from a captured HIP graph (no host launch cost between them)
    ms_graph = graph_ms(torch, step, steps, reps=3)
    # per-kernel durations: the same calls eager, each launch bracketed by HIP events on its stream
    timer = R.Timer()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        step({"timer": timer})
    e1.record()
    torch.cuda.synchronize()
    ms_eager = e0.elapsed_time(e1) / steps
    kernels = kernel_times(timer, CHUNK_KERNELS, steps)
    timer.close()
    # each call after a 512 MiB scratch write, which evicts q, k, v from the 256 MB Infinity Cache (the warm
    # replays reuse the same inputs, which then partly come from it); events around the call alone
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    cold = []
    for _ in range(cold_reps):
        scratch.fill_(1)
        e0.record()
        step()
        e1.record()
        torch.cuda.synchronize()
        cold.append(e0.elapsed_time(e1))
    del scratch
    R.ret_chunkwise_check(ws)  # no call of the timed regions abandoned a segment-chain wait
    cold.sort()
    nbytes, f_causal, f_pages = chunk_algorithmic(w)
    ms_cold = cold[len(cold) // 2] if cold else None
    tokens = w.B * w.N
    dom = max(kernels, key=lambda n: kernels[n]["avg_us"] * kernels[n]["launches_per_call"])
    # When a call is one kernel its duration is also the replayed graph's per-call time; otherwise its share
    # from the per-launch events.
    dom_us = kernels[dom]["avg_us"]
    res = {
        "workload": "%s: B=%d N=%d H=%d d_k=%d d_v=%d chunk=%d, bf16 in/out, fp32 state, xPos rotation"
                    % (w.name, w.B, w.N, w.H, w.dk, w.dv, w.chunk),
        "ms_per_call": ms_graph,
        "tokens_per_s": tokens / (ms_graph * 1e-3),
        "ms_per_call_eager": ms_eager,
        "ms_per_call_mall_cold_median": ms_cold,
        "tokens_per_s_mall_cold": tokens / (ms_cold * 1e-3) if cold else None,
        "kernels": kernels,
        "dominant_kernel": dom,
        "dominant_kernel_avg_us": dom_us,
        "alg_bytes_per_call": nbytes,
        "alg_flops_causal_per_call": f_causal,
        "alg_flops_pages_count_per_call": f_pages,
        "hbm_frac_whole_call": nbytes / (ms_graph * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "hbm_frac_dominant_kernel": nbytes / (dom_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
        "mfma_frac_causal_whole_call": f_causal / (ms_graph * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
        "mfma_frac_causal_dominant_kernel": f_causal / (dom_us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS,
        "mfma_frac_pages_count_whole_call": f_pages / (ms_graph * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
        "traffic_bytes_dominant_kernel": load_traffic(dom, w.name),
        "workspace_bytes": 0 if ws is None else ws.numel(),
    }
    return w, res


def roofline_of(res, bound):
    """The contract's roofline object for a chunkwise result: MFMA (causal-count TFLOP/s) or HBM (GB/s)."""
    dom_us = res["dominant_kernel_avg_us"]
    if bound == "mfma":
        ach = res["alg_flops_causal_per_call"] / (dom_us * 1e-6) / 1e12
        peak, unit = BF16_PEAK_TFLOPS, "TFLOP/s"
    else:
        ach = res["alg_bytes_per_call"] / (dom_us * 1e-6) / 1e9
        peak, unit = HBM_PEAK_GBS, "GB/s"
    # The dominant kernel is credited with the call's algorithmic work (it writes every output); where the call
    # has other launches (rotation, local passes, a scan), the whole call's fraction is given beside it.
    ms = res["ms_per_call"]
    whole = (res["alg_flops_causal_per_call"] / (ms * 1e-3) / 1e12 if bound == "mfma"
             else res["alg_bytes_per_call"] / (ms * 1e-3) / 1e9)
    return {"bound": bound, "achieved": ach, "peak": peak, "unit": unit, "frac": ach / peak,
            "traffic": res["traffic_bytes_dominant_kernel"], "kernel": res["dominant_kernel"],
            "kernel_avg_us": dom_us, "alg_bytes_per_launch": res["alg_bytes_per_call"],
            "alg_flops_causal_per_launch": res["alg_flops_causal_per_call"],
            "whole_call": {"achieved": whole, "frac": whole / peak, "ms_per_call": ms,
                           "launches": {k: v["launches_per_call"] for k, v in res["kernels"].items()}}}


def bench_epilogue(R, W, torch, wid, steps):
    """The multi-scale retention epilogue y = swish(gate) (.) GroupNorm_h(o) (per-channel affine; bf16 o, gate
    and y) on the chunkwise workload's output: alone, and as the layer without its projections, both as
    ret_chunkwise_msr_fwd (fused into the output stores where the kernel allows) and as two calls."""
    import numpy as np
    w = W.WORKLOADS[wid]
    q, k, v, rng = W.make_qkv(w)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).cuda()
    qd, kd, vd = dev(q), dev(k), dev(v)
    gate = dev(W.normal(rng, (w.B, w.N, w.H, w.dv), 1.0, "bf16"))
    del q, k, v
    gw = torch.from_numpy(rng.uniform(0.5, 1.5, w.H * w.dv).astype(np.float32)).cuda()
    gb = torch.from_numpy((0.1 * rng.standard_normal(w.H * w.dv)).astype(np.float32)).cuda()
    o = torch.empty((w.B, w.N, w.H, w.dv), dtype=torch.bfloat16, device="cuda")
    y = torch.empty_like(o)
    ws = R.chunkwise_workspace(qd, vd, w.chunk)
    chunk = lambda: R.ret_chunkwise_fwd(qd, kd, vd, o, w.gamma, w.chunk, theta=w.theta, workspace=ws)
    epi = lambda: R.ret_msr_epilogue(o, y, gate=gate, gn_weight=gw, gn_bias=gb, eps=1e-5)
    layer = lambda: R.ret_chunkwise_msr_fwd(qd, kd, vd, y, w.gamma, w.chunk, gate=gate, gn_weight=gw, gn_bias=gb,
                                            eps=1e-5, theta=w.theta, workspace=ws)
    chunk()
    ms_epi = graph_ms(torch, epi, steps)
    ms_layer2 = graph_ms(torch, lambda: (chunk(), epi()), steps)
    ms_layer = graph_ms(torch, layer, steps)
    R.ret_chunkwise_check(ws)
    nbytes = 3 * o.numel() * 2 + 2 * w.H * w.dv * 4  # o and gate read, y written (bf16); weight and bias
    ach = nbytes / (ms_epi * 1e-3) / 1e9
    return {
        "workload": "%s output: [%d, %d, %d, %d] bf16 o, gate and y, fp32 per-channel affine"
                    % (w.name, w.B, w.N, w.H, w.dv),
        "us_per_call": 1e3 * ms_epi,
        "roofline": {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBS,
                     "traffic": load_traffic("ret_msr_epilogue", w.name), "kernel": "ret_msr_epilogue",
                     "kernel_avg_us": 1e3 * ms_epi, "alg_bytes_per_launch": nbytes},
        "layer_us_per_call": 1e3 * ms_layer,
        "layer_tokens_per_s": w.B * w.N / (ms_layer * 1e-3),
        "layer_two_calls_us_per_call": 1e3 * ms_layer2,
    }


def bench_backward(R, W, torch, wid, steps):
    """Gradients dq, dk, dv of the chunkwise workload (bf16 q, k, v, dO in; bf16 gradients out), replayed from a
    HIP graph (the fastest of three replays), with the per-kernel split from the launch events of eager calls; on
    their own, and after the forward call whose workspace they reuse."""
    import numpy as np
    w = W.WORKLOADS[wid]
    q, k, v, rng = W.make_qkv(w)
    do = W.make_dout(w, rng)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).cuda()
    qd, kd, vd, dod = dev(q), dev(k), dev(v), dev(do)
    del q, k, v, do
    dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
    ws = R.chunkwise_bwd_workspace(qd, vd, w.chunk)
    call = lambda options=None: R.ret_chunkwise_bwd(qd, kd, vd, dod, dq, dk, dv, w.gamma, w.chunk, theta=w.theta,
                                                    workspace=ws, options=options)
    ms = graph_ms(torch, call, steps, 3)
    torch.cuda.synchronize()
    timer = R.Timer()
    for _ in range(3):
        call({"timer": timer})
    torch.cuda.synchronize()
    kernels = kernel_times(timer, ("ret_rotate_qk", "ret_permute_rotate") + CHUNK_KERNELS[1:], 3)
    timer.close()
    R.ret_chunkwise_check(ws)
    # after the forward call of a training step: its workspace (rotated q, k and segment states, where its kernels
    # leave them) passed to the gradients, which then reuse them (ret_chunkwise_bwd_saved_ex); the forward runs
    # once, outside the timed replays
    o = torch.empty_like(vd)
    fws = R.chunkwise_workspace(qd, vd, w.chunk)
    R.ret_chunkwise_fwd(qd, kd, vd, o, w.gamma, w.chunk, theta=w.theta, workspace=fws)
    call_saved = lambda options=None: R.ret_chunkwise_bwd(qd, kd, vd, dod, dq, dk, dv, w.gamma, w.chunk,
                                                          theta=w.theta, workspace=ws, fwd_workspace=fws,
                                                          options=options)
    ms_saved = graph_ms(torch, call_saved, steps, 3)
    torch.cuda.synchronize()
    timer = R.Timer()
    for _ in range(3):
        call_saved({"timer": timer})
    torch.cuda.synchronize()
    kernels_saved = kernel_times(timer, ("ret_rotate_qk", "ret_permute_rotate") + CHUNK_KERNELS[1:], 3)
    timer.close()
    del o, fws
    toks = w.B * w.N * w.H
    nbytes = toks * (2 * w.dk + 2 * w.dv) * 2 + toks * (2 * w.dk + w.dv) * 2  # q, k, v, dO in; dq, dk, dv out
    C = w.chunk
    # three retentions, each the forward's causal count (C+1)(d_k+d_v) + 4 d_k d_v per (token, head)
    flops = 3 * toks * ((C + 1) * (w.dk + w.dv) + 4 * w.dk * w.dv)
    ach = nbytes / (ms * 1e-3) / 1e9
    return {
        "workload": "%s: B=%d N=%d H=%d d_k=%d d_v=%d chunk=%d, bf16 q/k/v/dO in, bf16 dq/dk/dv out, xPos rotation"
                    % (w.name, w.B, w.N, w.H, w.dk, w.dv, w.chunk),
        "us_per_call": 1e3 * ms,
        "us_per_call_after_forward": 1e3 * ms_saved,
        "tokens_per_s": w.B * w.N / (ms * 1e-3),
        "hbm_frac_whole_call": ach / HBM_PEAK_GBS,
        "alg_bytes_per_call": nbytes,
        "tflops_causal": flops / (ms * 1e-3) / 1e12,
        "mfma_frac_causal": flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
        "kernels": kernels,
        "kernels_after_forward": kernels_saved,
        "workspace_bytes": ws.numel(),
    }


def bench_decode(R, W, torch, steps_graph=1024, reps=3, cold_states=32, mode="both"):
    """Batched decode: 1024 steps of the workload's q, k, v (drawn step by step) from its prefilled state,
    replayed from a HIP graph. MALL-cold: step t updates state t % cold_states, a working set of cold_states x
    16 MiB, so no state is still cached when its turn comes again; the library's default, the streamed state.
    Warm: one state, with the option that lets its accesses stay cached (step_cache 1). mode "warm" / "cold"
    runs one of the two (None for the other)."""
    import numpy as np
    w = W.WORKLOADS[3]
    rng = np.random.default_rng(w.seed)
    q, k, v, rng = W.make_qkv(w, rng)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).cuda()
    qd, kd, vd = dev(q), dev(k), dev(v)
    o = torch.empty((w.B, w.N, w.H, w.dv), dtype=torch.bfloat16, device="cuda")
    state = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device="cuda")
    R.ret_chunkwise_fwd(qd, kd, vd, o, w.gamma, w.chunk, theta=w.theta, state_out=state,
                        workspace=R.chunkwise_workspace(qd, vd, w.chunk))
    del qd, kd, vd, o
    # per-step inputs drawn step by step (q, k, v), as the workload defines them
    sq = np.empty((steps_graph, w.B, w.H, w.dk), np.float32)
    sk = np.empty_like(sq)
    sv = np.empty((steps_graph, w.B, w.H, w.dv), np.float32)
    for t in range(steps_graph):
        sq[t], sk[t], sv[t] = W.make_step(w, rng)
    sqd, skd, svd = dev(sq), dev(sk), dev(sv)
    outs = torch.empty((steps_graph, w.B, w.H, w.dv), dtype=torch.bfloat16, device="cuda")
    theta = w.theta
    states = state.unsqueeze(0).repeat(cold_states, 1, 1, 1, 1).contiguous()

    def run_steps(cold=False, options=None):
        for t in range(steps_graph):
            st = states[t % cold_states] if cold else state
            R.ret_recurrent_step(sqd[t], skd[t], svd[t], outs[t], st, w.gamma, pos=w.prefill + t, theta=theta,
                                 options=options)

    def measure(cold):
        opts = None if cold else {"step_cache": 1}
        us = 1e3 * graph_ms(torch, lambda: run_steps(cold, opts), 1, reps) / steps_graph
        # kernel duration from per-launch events (eager launches)
        timer = R.Timer()
        run_steps(cold, dict(opts or {}, timer=timer))
        torch.cuda.synchronize()
        tot, n = timer.query("ret_recurrent_step")
        timer.close()
        return us, 1e3 * tot / n

    us_warm, k_warm = measure(False) if mode != "cold" else (None, None)
    us_cold, k_cold = measure(True) if mode != "warm" else (None, None)
    return w, us_warm, us_cold, k_warm, k_cold


def bench_decode_long(R, W, torch, reps=3):
    """The long-sequence workload's 256 decode steps (B=1, H=8, d=128: a 512 KiB fp32 state, 1.06 MB per step)
    from its chunkwise final state, replayed from a HIP graph; positions 65536 onward. Each step is one small
    launch, so the figure is steps per second (launch latency bounds it, not HBM)."""
    import numpy as np
    w = W.WORKLOADS[5]
    q, k, v, rng = W.make_qkv(w)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).cuda()
    qd, kd, vd = dev(q), dev(k), dev(v)
    o = torch.empty((w.B, w.N, w.H, w.dv), dtype=torch.bfloat16, device="cuda")
    state = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device="cuda")
    R.ret_chunkwise_fwd(qd, kd, vd, o, w.gamma, w.chunk, theta=w.theta, state_out=state,
                        workspace=R.chunkwise_workspace(qd, vd, w.chunk))
    del qd, kd, vd, o
    steps = [W.make_step(w, rng) for _ in range(w.steps)]
    sqd = dev(np.stack([x[0] for x in steps]))
    skd = dev(np.stack([x[1] for x in steps]))
    svd = dev(np.stack([x[2] for x in steps]))
    outs = torch.empty((w.steps, w.B, w.H, w.dv), dtype=torch.bfloat16, device="cuda")

    def run_steps():
        for t in range(w.steps):
            R.ret_recurrent_step(sqd[t], skd[t], svd[t], outs[t], state, w.gamma, pos=w.N + t, theta=w.theta)

    us = 1e3 * graph_ms(torch, run_steps, 1, reps) / w.steps
    db, _ = decode_algorithmic(w.B, w.H, w.dk, w.dv)
    return {"workload": "%s decode: B=%d H=%d d_k=%d d_v=%d, fp32 state from the %d-token chunkwise call, %d steps, "
                        "HIP graph" % (w.name, w.B, w.H, w.dk, w.dv, w.N, w.steps),
            "us_per_step": us, "steps_per_s": 1e6 / us, "alg_bytes_per_step": db,
            "hbm_frac": db / (us * 1e-6) / 8e12, "bound": "launch latency (1.06 MB per step)"}


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(W, wid, seconds=8.0, single_seconds=3.0, sample_tokens=1024):
    """The fp64 oracle's chunkwise form on this host over a bounded sample of the workload: the first
    `sample_tokens` tokens of every sequence and head, one thread per (b, h) up to the oracle's default thread
    count, repeated for about `seconds`; then one (b, h) of the same sample on one thread for about
    `single_seconds`. Scaled to tokens/s of the whole layer (all heads)."""
    import oracle
    w = W.WORKLOADS[wid]
    q, k, v, _ = W.make_qkv(w)
    n = min(w.N, sample_tokens)
    q, k, v = q[:, :n], k[:, :n], v[:, :n]
    threads = min(oracle.default_threads(), w.B * w.H)

    def timed(qq, kk, vv, gamma, nthreads, budget):
        runs, total = 0, 0.0
        while runs == 0 or total < budget:
            t0 = time.perf_counter()
            oracle.chunkwise(qq, kk, vv, gamma, w.chunk, theta=w.theta, threads=nthreads)
            total += time.perf_counter() - t0
            runs += 1
        return runs, total

    runs, total = timed(q, k, v, w.gamma, threads, seconds)
    runs1, total1 = timed(q[:1, :, :1], k[:1, :, :1], v[:1, :, :1], w.gamma[:1], 1, single_seconds)
    return {"value": runs * w.B * n / total, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "%d runs of the first %d tokens of the %s workload (B=%d H=%d d_k=%d d_v=%d chunk=%d), fp64 "
                      "chunkwise form, one thread per (b, h), %.1f s in total"
                      % (runs, n, w.name, w.B, w.H, w.dk, w.dv, w.chunk, total),
            "single_thread_value": runs1 * n / total1 / (w.B * w.H),
            "single_thread_sample": "%d runs of one head over the same %d tokens on one thread, %.1f s in total; "
                                    "scaled to tokens/s of all %d heads" % (runs1, n, total1, w.B * w.H),
            "cpu_model": _cpu_model(), "host_cpus": len(os.sched_getaffinity(0))}


COPY_BYTES = 256 << 20


def copy_calibration(torch):
    """A plain device copy of known size, for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    n = COPY_BYTES
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    # and its rate (bytes read + written per second) over 20 more copies, for context beside the HBM peak
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(20):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    gbps = 2 * n * 20 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    print(json.dumps({"copy_calibration_bytes": n, "launches": 3, "copy_GBps": round(gbps, 1)}), flush=True)


def _counter_rows(directory, counter, kernel_substr):
    """Per-dispatch values of `counter` for kernels whose name contains kernel_substr, from the
    *_counter_collection.csv files rocprofv3 wrote under directory. "NAME@grid=N" also requires a grid of N
    threads (one kernel launched in several roles, as the split launches of the streaming kernel)."""
    import csv
    grid = None
    if "@grid=" in kernel_substr:
        kernel_substr, g = kernel_substr.split("@grid=", 1)
        grid = int(g)
    vals = {}
    for root, _, files in os.walk(directory):
        for fn in files:
            if not fn.endswith("counter_collection.csv"):
                continue
            with open(os.path.join(root, fn), newline="") as f:
                for row in csv.DictReader(f):
                    if grid is not None and int(row["Grid_Size"]) != grid:
                        continue
                    if row["Counter_Name"] == counter and kernel_substr in row["Kernel_Name"]:
                        key = (fn, row["Dispatch_Id"])
                        vals[key] = vals.get(key, 0.0) + float(row["Counter_Value"])
    return list(vals.values())


def record_traffic(key, kernel_substr, fetch_dir, write_dir, copy_fetch_dir, copy_write_dir):
    workload = key.split("@", 1)[1] if "@" in key else ""
    cf = _counter_rows(copy_fetch_dir, "FETCH_SIZE", "copyBuffer")
    cw = _counter_rows(copy_write_dir, "WRITE_SIZE", "copyBuffer")
    fe = _counter_rows(fetch_dir, "FETCH_SIZE", kernel_substr)
    wr = _counter_rows(write_dir, "WRITE_SIZE", kernel_substr)
    if not (cf and cw and fe and wr):
        sys.exit("record-traffic: no counter rows (copy %d/%d, kernel %d/%d)" % (len(cf), len(cw), len(fe), len(wr)))
    avg = lambda xs: sum(xs) / len(xs)
    rec = {"workload": workload, "kernel_match": kernel_substr,
           "fetch_kib_per_launch": avg(fe), "write_kib_per_launch": avg(wr), "dispatches": [len(fe), len(wr)],
           # counter KiB per byte of a plain copy of COPY_BYTES (both directions)
           "copy_factor_fetch": avg(cf) * 1024.0 / COPY_BYTES, "copy_factor_write": avg(cw) * 1024.0 / COPY_BYTES,
           "source_digest": source_digest()}
    try:
        with open(TRAFFIC_FILE) as f:
            recs = json.load(f)
    except (OSError, ValueError):
        recs = {}
    recs[key] = rec
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(recs, f, indent=1, sort_keys=True)
        f.write("\n")
    mb = lambda kib, fac: kib * 1024.0 / fac / 1e6
    print("%s: fetch %.2f MB, write %.2f MB per launch (%d / %d dispatches)"
          % (key, mb(rec["fetch_kib_per_launch"], rec["copy_factor_fetch"]),
             mb(rec["write_kib_per_launch"], rec["copy_factor_write"]), len(fe), len(wr)))


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--record-traffic":
        if len(sys.argv) != 8:
            sys.exit("usage: bench.py --record-traffic KEY KERNEL FETCH_DIR WRITE_DIR COPY_FETCH_DIR COPY_WRITE_DIR")
        record_traffic(*sys.argv[2:8])
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="7b-class-layer", choices=sorted(CHUNK_WORKLOADS),
                    help="chunkwise workload timed for `value`")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-epilogue", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="only the `value` workload's chunkwise call")
    ap.add_argument("--no-cold", action="store_true", help="skip the MALL-cold chunkwise calls (warm-only traces)")
    ap.add_argument("--decode-mode", default="both", choices=("both", "warm", "cold"))
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--decode-steps", type=int, default=1024, help="decode steps per graph (1024 in the workload)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path, and nothing here launches work "
              "on a second GPU (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    from linear_recurrent_sequence_amd import retention as R
    from linear_recurrent_sequence_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    R.load(build_if_missing=True)
    if args.copy_calibration:
        copy_calibration(torch)
        return

    def progress(msg):
        print("[bench] %s" % msg, file=sys.stderr, flush=True)

    wid = CHUNK_WORKLOADS[args.workload]
    progress("chunkwise %s" % args.workload)
    cold_reps = 0 if args.no_cold else 20
    w, main_res = bench_chunkwise(R, W, torch, wid, args.steps, args.warmup, cold_reps)
    bound = "mfma" if w.dk >= 256 else "hbm"  # the d_k 256 layer sits at the ridge; the others are HBM-bound
    tokens = w.B * w.N
    result = {
        "metric": METRIC,
        "value": main_res["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res["ms_per_call"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": main_res["workload"], "global_batch": w.B, "seq_len": w.N},
        "roofline": roofline_of(main_res, bound),
        "chunkwise": main_res,
    }
    result["roofline"]["hbm_frac"] = main_res["hbm_frac_dominant_kernel"]
    if not args.no_extra:
        for name, key in sorted(CHUNK_WORKLOADS.items(), key=lambda kv: kv[1]):
            if key == wid:
                continue
            progress("chunkwise %s" % name)
            wx, res = bench_chunkwise(R, W, torch, key, args.steps, args.warmup, cold_reps)
            res["roofline"] = roofline_of(res, "mfma" if wx.dk >= 256 else "hbm")
            result[name] = res
    if not args.no_decode:
        progress("decode")
        dw, us_warm, us_cold, k_warm, k_cold = bench_decode(R, W, torch, steps_graph=args.decode_steps,
                                                            mode=args.decode_mode)
        db, dflops = decode_algorithmic(dw.B, dw.H, dw.dk, dw.dv)

        def decode_roofline(us, key, state):
            ach = db / (us * 1e-6) / 1e9
            # one kernel per step: the graph's per-step time (events on the replay stream)
            return {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBS,
                    "traffic": load_traffic("ret_recurrent_step", key), "kernel": "ret_recurrent_step",
                    "kernel_avg_us": us, "alg_bytes_per_launch": db, "state": state}

        cold_state = ("MALL-cold: the steps cycle through 32 distinct 16 MiB states (512 MiB); the default "
                      "streamed state (non-temporal loads and stores)")
        warm_state = "warm: one 16 MiB state, held by the Infinity Cache between steps (option step_cache 1)"
        us_main = us_cold if us_cold is not None else us_warm
        result["decode"] = {
            "workload": "%s: B=%d H=%d d_k=%d d_v=%d, fp32 state, bf16 q/k/v/o, %d steps from a %d-token prefill, "
                        "HIP graph" % (dw.name, dw.B, dw.H, dw.dk, dw.dv, args.decode_steps, dw.prefill),
            "steps_per_s": 1e6 / us_main, "tokens_per_s": dw.B * 1e6 / us_main, "us_per_step": us_main,
            "roofline": decode_roofline(us_cold, dw.name + " mall-cold", cold_state) if us_cold is not None
            else decode_roofline(us_warm, dw.name, warm_state),
            "kernel_avg_us_eager": {"warm": k_warm, "mall_cold": k_cold},
        }
        if us_cold is not None and us_warm is not None:
            result["decode"]["warm"] = {"us_per_step": us_warm, "steps_per_s": 1e6 / us_warm,
                                        "roofline": decode_roofline(us_warm, dw.name, warm_state)}
        if not args.no_extra:
            progress("decode long-sequence")
            result["long-sequence-decode"] = bench_decode_long(R, W, torch)
    if not args.no_epilogue:
        progress("epilogue")
        result["epilogue"] = bench_epilogue(R, W, torch, CHUNK_WORKLOADS["retention-layer-d512"], args.steps)
    if not args.no_backward:
        result["backward"] = {}
        for name, key in sorted(CHUNK_WORKLOADS.items(), key=lambda kv: kv[1]):
            if args.no_extra and key != wid:
                continue
            bw = W.WORKLOADS[key]
            if R.load().ret_chunkwise_bwd_workspace_bytes(bw.B, bw.N, bw.H, bw.dk, bw.dv, bw.chunk, R.RET_BF16):
                progress("backward %s" % name)
                bres = bench_backward(R, W, torch, key, max(3, args.steps // 4))
                fwd = result["chunkwise"] if key == wid else result.get(name)
                if fwd:
                    bres["x_forward"] = bres["us_per_call"] / (1e3 * fwd["ms_per_call"])
                    bres["x_forward_after_forward"] = bres["us_per_call_after_forward"] / (1e3 * fwd["ms_per_call"])
                result["backward"][name] = bres
    if not args.no_cpu_baseline:
        progress("cpu baseline")
        result["cpu_baseline"] = cpu_baseline(W, wid)
    result["context"] = ("pages' figures (whole 6.7B model, A100-80GB, vanilla PyTorch): 8.4x faster decoding and "
                         "70% less memory than a KV-cached Transformer at 8k; not comparable to this kernel metric")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
