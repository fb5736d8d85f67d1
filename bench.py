#!/usr/bin/env python3
"""Benchmark of the KDA chunked forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 3]

One step is one kda_fwd over the whole batch of the throughput workload
(B=4 rows x T=16384 tokens, H=32 heads, dk=dv=128, bf16 inputs, fp32 state,
chunk 64, one document per row, no lower bound), with every input already
resident in HBM.  W untimed steps, then exactly K timed steps between two
device synchronisations; rank 0 prints one JSON line.

Besides the throughput it reports
  * "short_conv": the same step after the layer's short convolution + SiLU of
    q, k, v (kda_fwd_short_conv), and that convolution kernel's own HBM rate;
  * "output_norm": the gated output norm after the forward (its kernel's HBM rate);
  * "backward": the gradients of the same forward (kda_bwd);
  * "workloads": the forward on the other four workloads (tiny fp32, packed
    varlen, long slice with carried state, short documents with a lower
    bound), each on its own seeded inputs, timed the same way;
  * "state_summary": the long row cut into 8 contiguous slices, the affine
    summary of every slice (kda_state_summary, one call) and their composition
    from the initial state (kda_apply_state_summary, slice by slice), compared
    with the forward's final state;
  * "roofline": the whole forward's algorithmic bytes (1,282 B per token-head
    at dk=dv=128 bf16: q, k, gate, v, beta read and o written once, plus the
    fp32 states) divided by the dominant kernel's duration, timed live with HIP
    events recorded by the library around each stage on the kernel's own
    stream (kda_fwd_profiled); "traffic" is the counter-measured HBM bytes of
    that kernel and "design_bytes_per_launch" the bytes it must move given
    this design's intermediates;
  * timing: per-step events with 1 GiB of scratch written between steps (the
    256 MB last-level cache evicted) for the headline and every workload,
    and the same steps back to back as warm_*;
  * "cpu_baseline": the CPU oracle, as it stands, timed on this host on a
    bounded sample of the same workload (a few heads of one row).
Only one GPU is used: --gpus above 1 exits with a message.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from gated_delta_rule_43_amd import kda, synthetic  # noqa: E402
from gated_delta_rule_43_amd.timing import StageEvents, evict_caches  # noqa: E402

METRIC = "KDA chunked fwd Mtokens/s at H=32,dk=dv=128 bf16; MFMA util % of peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
FP32_VECTOR_PEAK_TFLOPS = 157.3  # MI355X fp32 vector ALU, TFLOP/s


def algorithmic(w):
    """Algorithmic bytes and FLOPs of the whole forward, per token-head (bf16
    inputs/outputs, triangular savings counted; see the measurement notes)."""
    K, V, C = w.K, w.V, w.chunk_size
    elt = 2 if w.dtype == "bf16" else 4
    bytes_th = elt * (3 * K + V) + elt + elt * V
    flops_th = 2 * (3 * K * V + (C / 2) * (3 * K + 2 * V)) + C * C / 3
    return bytes_th, flops_th


def _current_profile(name):
    """A committed rocprofv3 summary (json under profiles/), or None when the
    kernel source it was taken from has changed since."""
    import hashlib
    try:
        info = json.load(open(os.path.join(ROOT, "profiles", name)))
        src = open(os.path.join(ROOT, info["source"]), "rb").read()
    except (OSError, ValueError, KeyError):
        return None
    return info if hashlib.sha256(src).hexdigest() == info.get("source_sha256") else None


def measured_traffic(stage_name):
    """HBM bytes per launch of a stage from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary, or None when the kernel source changed since then."""
    info = _current_profile("traffic_throughput_bf16_B4_T16384_H32_d128.json")
    k = None if info is None else info.get("kernels", {}).get(stage_name)
    return None if k is None else int(k["traffic_bytes"])


def measured_path_traffic():
    """HBM bytes of one whole forward (every kernel of the throughput workload's
    call) from the same committed summary, or None when stale/absent."""
    info = _current_profile("traffic_throughput_bf16_B4_T16384_H32_d128.json")
    return None if info is None else int(sum(k["traffic_bytes"] for k in info.get("kernels", {}).values()))


def measured_mfma_util(workload):
    """Per-kernel MFMA busy % (SQ_VALU_MFMA_BUSY_CYCLES over the SIMDs' active
    cycles) from the committed counter summary, or None when stale/absent."""
    info = _current_profile("mfma_util_throughput_and_varlen_bf16_d128.json")
    k = None if info is None else info.get("workloads", {}).get(str(workload))
    return None if not k else {n: v["mfma_util_pct"] for n, v in k.items()}


def measured_conv_traffic():
    """HBM bytes per launch of the short-convolution kernel on q alone, from the
    committed FETCH_SIZE / WRITE_SIZE summary, or None when stale/absent."""
    info = _current_profile("short_conv_throughput_bf16_B4_T16384_H32_d128.json")
    k = None if info is None else info.get("q_only")
    return None if k is None else int(k["traffic_bytes"])


def path_algorithmic_bytes(w, N):
    """Algorithmic HBM bytes of one whole forward (the measurement notes'
    figure): per token-head q, k, gate, v and beta read once and o written
    once, plus per (sequence, head) the fp32 state read (initial_state) and
    written (final_state) when present."""
    bytes_th, _ = algorithmic(w)
    states = N * w.H * w.K * w.V * 4 * ((1 if w.init_std is not None else 0)
                                        + (1 if w.output_final_state else 0))
    return int(w.B * w.T * w.H * bytes_th + states)


def record_bytes(K, V):
    """Bytes of one chunk record of the MFMA path (per chunk-head): Qt, W and
    Kbar^T fragments (C*K bf16 each), Aqk fragments (C*C bf16), gL (K fp32) and
    U tiles (C*V bf16)."""
    C = 64
    return 3 * C * K * 2 + C * C * 2 + K * 4 + C * V * 2


def stage_bytes(w, stage, NT, N):
    """Design bytes of one launch of a stage: the unique bytes it must move
    given this design's chunk records (every input element read once, every
    record and output element written once).  Not the path's algorithmic
    bytes: the records are the design's own intermediate."""
    B, T, H, K, V = w.B, w.T, w.H, w.K, w.V
    ein = 2 if w.dtype == "bf16" else 4
    tokh = B * T * H
    rec = record_bytes(K, V)
    states = N * H * K * V * 4 * ((1 if w.init_std is not None else 0) + (1 if w.output_final_state else 0))
    if stage == 2:   # chunk factors: q, k, gate, v, beta in -> one record per chunk-head out
        return tokh * (3 * K + V + 1) * ein + NT * H * rec
    if stage == 3:   # state pass: records in, o out, initial/final states
        return NT * H * rec + tokh * V * ein + states
    return 0


def fwd_runner(w, inp, dev):
    """A closure running kda_fwd once on resident inputs (its own output and
    workspace), with optional per-stage events; and the sequence count N."""
    cu = inp["cu_seqlens"]
    cu_host = None if cu is None else cu.cpu()
    N = w.B if cu is None else cu.numel() - 1
    o = torch.empty(w.B, w.T, w.H, w.V, dtype=w.torch_dtype, device=dev)
    need = kda.fwd_workspace_size((w.B, w.T, w.H, w.K), w.V, w.torch_dtype, w.chunk_size,
                                  w.lower_bound, N=N, cu_seqlens_host=cu_host)
    ws = torch.empty(need + 256, dtype=torch.uint8, device=dev)
    ws = ws[(-ws.data_ptr()) % 256:][:need]
    res = {"o": o, "fin": None}

    def step(events=None):
        _, res["fin"] = kda.kda_fwd(inp["q"], inp["k"], inp["v"], inp["gate"], inp["beta"],
                                    inp["a_log"], inp["dt_bias"], scale=w.scale,
                                    lower_bound=w.lower_bound, chunk_size=w.chunk_size,
                                    cu_seqlens=cu, cu_seqlens_host=cu_host,
                                    initial_state=inp["initial_state"],
                                    output_final_state=w.output_final_state, out=o, workspace=ws,
                                    stage_events=events)
    return step, res, N, cu_host


def time_fwd(step, steps, warmup):
    """W untimed runs, then two timed passes of `steps` runs each:

    * evicted (the headline, as the measurement notes prescribe): before each
      run 1 GiB of scratch is written (outside the run's events), so every
      run reads its inputs from HBM; the step time is the median over runs of
      the library's own events (first stage start to last stage end);
    * warm: the runs back to back between two synchronisations (wall clock),
      so small workloads may find their inputs in the 256 MB last-level cache.

    Returns {"ms": evicted median, "stage_ms": evicted median per stage,
    "warm_ms": ..., "warm_stage_ms": ...}."""
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev = StageEvents(steps)
    for i in range(steps):
        evict_caches()
        step(ev.arrays[i])
    torch.cuda.synchronize()
    per_step = ev.per_step_ms()
    per_stage = ev.per_step_stage_ms()
    ev.close()
    ev = StageEvents(steps)
    t0 = time.perf_counter()
    for i in range(steps):
        step(ev.arrays[i])
    torch.cuda.synchronize()
    warm = (time.perf_counter() - t0) * 1e3 / steps
    warm_stage = ev.stage_ms()
    ev.close()
    return {"ms": float(np.median(per_step)), "stage_ms": np.median(per_stage, axis=0),
            "warm_ms": warm, "warm_stage_ms": warm_stage}


def _stage_dict(x):
    return dict(zip(kda.STAGE_NAMES, [round(float(v), 4) for v in x]))


def bench_state_summary(w, inp, fin_fwd, steps, warmup, slices=8):
    """The long row as `slices` contiguous slices: the affine summary of every
    slice in one kda_state_summary call (the slices are rows of one batch, a
    view of the same memory), then the summaries composed from the initial
    state with kda_apply_state_summary, one slice after another.  Events on the
    launch stream around both parts; the composed state is compared with the
    forward's final state of the same row."""
    dev = inp["q"].device
    S = w.T // slices
    cut = lambda t: t.reshape(slices, S, *t.shape[2:])
    args = [cut(inp[x]) for x in ("q", "k", "v", "gate", "beta")]
    bufs = [torch.empty_like(inp["initial_state"]) for _ in range(2)]

    def summary():
        return kda.kda_state_summary(*args, inp["a_log"], inp["dt_bias"],
                                     lower_bound=w.lower_bound, chunk_size=w.chunk_size)

    def compose(E, P):
        st = inp["initial_state"]
        for r in range(slices):
            st = kda.kda_apply_state_summary(E[r:r + 1], P[r:r + 1], st, out=bufs[r % 2])
        return st

    for _ in range(max(1, warmup)):
        compose(*summary())
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for e0, e1, e2 in evs:
        e0.record(stream)
        E, P = summary()
        e1.record(stream)
        st = compose(E, P)
        e2.record(stream)
    torch.cuda.synchronize()
    sum_ms = float(np.mean([a.elapsed_time(b) for a, b, _ in evs]))
    app_ms = float(np.mean([b.elapsed_time(c) for _, b, c in evs]))
    err = float((st - fin_fwd).abs().max())
    ref = float(fin_fwd.abs().max())
    elt = 2 if w.dtype == "bf16" else 4
    # algorithmic bytes of the summary call: every input read once, the slice
    # summaries (E [slices,H,K,V], P [slices,H,K,K], fp32) written once
    nbytes = w.T * w.H * (3 * w.K + w.V + 1) * elt + slices * w.H * (w.K * w.V + w.K * w.K) * 4
    achieved = nbytes / (sum_ms / 1e3) / 1e9
    return {"workload": "%s as %d contiguous slices of %d tokens" % (w.name, slices, S),
            "value": round(w.T / ((sum_ms + app_ms) / 1e3) / 1e6, 4), "unit": "Mtokens/s",
            "summary_ms": round(sum_ms, 4), "compose_ms": round(app_ms, 4),
            "summary_path_algorithmic_GBps": round(achieved, 2),
            "summary_path_hbm_frac": round(achieved / HBM_PEAK_GBS, 5),
            "composed_vs_forward_final_state_max_abs": err,
            "forward_final_state_max_abs": ref}


def bench_other_workloads(skip, steps, warmup, dev):
    """The forward on each other workload, on its own seeded inputs, timed like
    the headline; the long-slice workload also times its slice summaries."""
    out = {}
    for wid in sorted(synthetic.WORKLOADS):
        if wid == skip:
            continue
        w = synthetic.WORKLOADS[wid]
        print("[bench] workload %s" % w.name, file=sys.stderr, flush=True)
        inp = synthetic.make_inputs(w, dev)
        step, res, N, cu_host = fwd_runner(w, inp, dev)
        t = time_fwd(step, steps, warmup)
        ms = t["ms"]
        path_bytes = path_algorithmic_bytes(w, N)
        out[w.name] = {"value": round(w.B * w.T / (ms / 1e3) / 1e6, 4), "unit": "Mtokens/s",
                       "ms_per_step": round(ms, 4), "dtype": w.dtype, "sequences": N,
                       "stage_ms": _stage_dict(t["stage_ms"]),
                       "warm_value": round(w.B * w.T / (t["warm_ms"] / 1e3) / 1e6, 4),
                       "warm_ms_per_step": round(t["warm_ms"], 4),
                       "warm_stage_ms": _stage_dict(t["warm_stage_ms"]),
                       "path_algorithmic_bytes": path_bytes,
                       "path_hbm_frac": round(path_bytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 5)}
        if w.init_std is not None and N == 1:
            print("[bench] slice summaries of %s" % w.name, file=sys.stderr, flush=True)
            out["state_summary"] = bench_state_summary(w, inp, res["fin"], steps, warmup)
        del inp, step, res
        torch.cuda.empty_cache()
    return out


def cpu_baseline(inp, w, budget_s=12.0):
    """The oracle as it stands on a bounded sample of the workload: whole rows
    (all tokens) of a growing number of (row, head) pairs, sized from a short
    probe to take about budget_s; scaled to Mtokens/s of the full H-head rows."""
    import oracle
    threads = oracle.default_threads()
    pairs_all = [(b, h) for b in range(w.B) for h in range(w.H)]

    def run(npairs, T):
        rows = sorted(set(b for b, _ in pairs_all[:npairs]))
        secs = 0.0
        done = 0
        for b in rows:
            heads = [h for bb, h in pairs_all[:npairs] if bb == b]
            cut = lambda t: t[b:b + 1, :T][:, :, heads].float().cpu().numpy()
            args = [cut(inp[x]) for x in ("q", "k", "v", "gate", "beta")]
            t0 = time.perf_counter()
            oracle.kda_fwd(*args, inp["a_log"][heads].cpu().numpy(),
                           inp["dt_bias"][heads].cpu().numpy(), scale=w.scale,
                           lower_bound=w.lower_bound, threads=threads, output_final_state=False)
            secs += time.perf_counter() - t0
            done += T * len(heads)
        return secs, done

    probe_pairs = min(len(pairs_all), threads)
    dt, _ = run(probe_pairs, 512)
    per_th = dt / (probe_pairs * 512)              # seconds per token-head at this parallelism
    npairs = probe_pairs
    while npairs < len(pairs_all) and per_th * npairs * w.T < budget_s * 0.5:
        npairs = min(len(pairs_all), npairs + threads)
    T = int(min(w.T, max(512, budget_s / max(per_th * npairs, 1e-12))))
    secs, token_heads = run(npairs, T)
    passes = 1
    # the whole workload finished early: repeat it so the timing spans the budget
    while npairs == len(pairs_all) and T == w.T and secs < budget_s * 0.8 and passes < 8:
        s2, th2 = run(npairs, T)
        secs, token_heads, passes = secs + s2, token_heads + th2, passes + 1
    mtok = token_heads / w.H / secs / 1e6
    model = next((ln.split(":", 1)[1].strip() for ln in open("/proc/cpuinfo")
                  if ln.startswith("model name")), "unknown")
    return {"value": round(mtok, 6), "unit": "Mtokens/s", "cores": threads, "kind": "oracle",
            "host_cpu": model,
            "sample": "%d (row, head) pairs x first %d tokens, %d pass(es) = %d token-heads in "
                      "%.1f s; fp64 token recurrence, rate scaled to %d heads per token"
                      % (npairs, T, passes, token_heads, secs, w.H)}


def bench_short_conv(inp, w, o, steps, warmup, width=4):
    """The forward after the layer's short convolution + SiLU (kda_fwd_short_conv,
    width-4 convolutions with bias on q, k, v) on the same resident inputs, and
    the convolution kernel alone (kda_short_conv_silu on q), timed with events
    on the stream both are launched on."""
    dev = inp["q"].device
    chans = (w.H * w.K, w.H * w.K, w.H * w.V)
    ws_, bs_ = synthetic.short_conv_params(123, chans, width, True, device=dev)
    cu = inp["cu_seqlens"]
    cu_host = None if cu is None else cu.cpu()

    def fwd():
        kda.kda_fwd_short_conv(inp["q"], inp["k"], inp["v"], inp["gate"], inp["beta"],
                               inp["a_log"], inp["dt_bias"], ws_, bs_, scale=w.scale,
                               lower_bound=w.lower_bound, chunk_size=w.chunk_size,
                               cu_seqlens=cu, cu_seqlens_host=cu_host,
                               initial_state=inp["initial_state"],
                               output_final_state=w.output_final_state, out=o)

    for _ in range(warmup):
        fwd()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fwd()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    # the convolution kernel alone, on q (events on the current stream, which
    # is the stream the binding launches on)
    y = torch.empty_like(inp["q"])
    for _ in range(2):
        kda.short_conv_silu(inp["q"], ws_[0], bs_[0], cu_seqlens=cu, cu_seqlens_host=cu_host, out=y)
    stream = torch.cuda.current_stream(dev)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for a, b in evs:
        a.record(stream)
        kda.short_conv_silu(inp["q"], ws_[0], bs_[0], cu_seqlens=cu, cu_seqlens_host=cu_host, out=y)
        b.record(stream)
    torch.cuda.synchronize()
    conv_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    elt = 2 if w.dtype == "bf16" else 4
    conv_bytes = 2 * w.B * w.T * chans[0] * elt      # x read once, y written once
    achieved = conv_bytes / (conv_ms / 1e3) / 1e9
    tokens = w.B * w.T
    return {"workload": w.name + " after a width-%d short convolution + SiLU (with bias) on q, k, v"
                        % width,
            "value": round(tokens / (ms / 1e3) / 1e6, 4), "unit": "Mtokens/s",
            "ms_per_step": round(ms, 4),
            "conv_kernel": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 5),
                            "kernel_ms": round(conv_ms, 4), "bytes_per_launch": conv_bytes,
                            "traffic": measured_conv_traffic() if w.name.startswith("throughput")
                            else None,
                            "tensor": "q [B,T,H*K]"}}


def bench_output_norm(o, w, steps):
    """The gated output norm after the forward (kda_gated_rms_norm, sigmoid gate)
    on the forward's output shape, with a seeded gate; events on its stream."""
    dev = o.device
    gen = torch.Generator(device=dev)
    gen.manual_seed(11)
    gate = torch.randn(o.shape, generator=gen, device=dev).to(o.dtype)
    weight = torch.rand(o.shape[-1], generator=gen, device=dev) + 0.5
    y = torch.empty_like(o)
    for _ in range(2):
        kda.gated_rms_norm(o, gate, weight, out=y)
    stream = torch.cuda.current_stream(dev)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for a, b in evs:
        a.record(stream)
        kda.gated_rms_norm(o, gate, weight, out=y)
        b.record(stream)
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    nbytes = 3 * o.numel() * o.element_size() + weight.numel() * 4   # o, gate in; y out
    achieved = nbytes / (ms / 1e3) / 1e9
    return {"kernel": "k_gated_rms_norm", "shape": list(o.shape), "kernel_ms": round(ms, 4),
            "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 5), "bytes_per_launch": nbytes}


def bwd_chunk_flops(C, K, V):
    """FLOPs one chunk-head of the chunk-gradient kernel must do (full chunk,
    2 per multiply-add, triangles counted once, exponentials not counted):
    dW, dQ~ and dKbar (C x K over V each), the S0 . dS_L row sums, P and the V
    half of Y (lower triangles over V), dV (triangular Tm^T over V), the K half
    of Y (lower triangle over K), the two triangular products of Tm (C^3/3),
    and the pairwise q^, k^, gamma terms (4 multiply-adds per pair and channel)."""
    tri = C * (C + 1) // 2
    macs = 3 * C * K * V + K * V + 3 * tri * V + tri * K + C ** 3 // 3 + 4 * tri * K
    return 2 * macs


def bench_backward(inp, w, steps, warmup):
    """The backward (kda_bwd) of the same forward on the same resident inputs,
    with a seeded output gradient; events on the launch stream around each call."""
    dev = inp["q"].device
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    d_o = torch.randn(w.B, w.T, w.H, w.V, generator=gen, device=dev).to(w.torch_dtype)
    cu = inp["cu_seqlens"]
    cu_host = None if cu is None else cu.cpu()

    def bwd():
        return kda.kda_bwd(inp["q"], inp["k"], inp["v"], inp["gate"], inp["beta"], inp["a_log"],
                           inp["dt_bias"], d_o, None, scale=w.scale, lower_bound=w.lower_bound,
                           chunk_size=w.chunk_size, cu_seqlens=cu, cu_seqlens_host=cu_host,
                           initial_state=inp["initial_state"])

    for _ in range(max(1, warmup)):
        bwd()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in evs:
        a.record(stream)
        bwd()
        b.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    # the same call with the library's per-stage events (kda_bwd_profiled)
    sev = StageEvents(steps, kda.BWD_NUM_STAGES)
    for i in range(steps):
        kda.kda_bwd(inp["q"], inp["k"], inp["v"], inp["gate"], inp["beta"], inp["a_log"],
                    inp["dt_bias"], d_o, None, scale=w.scale, lower_bound=w.lower_bound,
                    chunk_size=w.chunk_size, cu_seqlens=cu, cu_seqlens_host=cu_host,
                    initial_state=inp["initial_state"], stage_events=sev.arrays[i])
    torch.cuda.synchronize()
    stage_ms = sev.stage_ms()
    sev.close()
    tokens = w.B * w.T
    NT = w.B * math.ceil(w.T / w.chunk_size) if cu is None else int(
        sum(math.ceil(int(b - a) / w.chunk_size) for a, b in zip(cu_host[:-1], cu_host[1:])))
    kidx = kda.BWD_STAGE_NAMES.index("chunk_gradients")
    kms = float(stage_ms[kidx])
    flops = NT * w.H * bwd_chunk_flops(w.chunk_size, w.K, w.V)
    tflops = flops / (kms / 1e3) / 1e12 if kms > 0 else 0.0
    return {"workload": w.name + " backward (gradients of q, k, v, gate, beta, a_log, dt_bias)",
            "value": round(tokens / (ms / 1e3) / 1e6, 4), "unit": "Mtokens/s",
            "ms_per_step": round(ms, 3), "wall_ms_per_step": round(wall, 3),
            "arith": ("bf16 matrix-core recomputation of the chunk factors (fp32 accumulation); "
                      "state passes and the chunk kernel's value-dimension products on bf16 "
                      "matrix cores with fp32 states split into bf16 hi + lo pairs; the other "
                      "dense products on fp32 matrix cores, the per-element work fp32 VALU"
                      if w.torch_dtype == torch.bfloat16
                      else "fp32 (VALU, and fp32 matrix cores for the state passes and the chunk "
                      "kernel's dense products at chunk 64)"),
            "stage_ms": dict(zip(kda.BWD_STAGE_NAMES, [round(float(x), 4) for x in stage_ms])),
            "roofline": {"bound": "alu", "achieved": round(tflops, 3),
                         "peak": FP32_VECTOR_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tflops / FP32_VECTOR_PEAK_TFLOPS, 5), "traffic": None,
                         "kernel": "chunk_gradients (k_bwd_chunk)", "kernel_ms": round(kms, 4),
                         "flops_per_launch": flops}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-short-conv", action="store_true",
                    help="skip the forward-after-short-convolution measurement")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward measurement")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the forward on the other workloads and the slice summaries")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB a few times (to scale the "
                         "FETCH_SIZE/WRITE_SIZE counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the forward shards by head or by sequence slice; see DESIGN.md).", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n * 4, "launches": 5}))
        return
    kda.load_library()
    w = synthetic.WORKLOADS[args.workload]
    dev = torch.device("cuda", 0)
    print("[bench] drawing %s on %s" % (w.name, dev), file=sys.stderr, flush=True)
    inp = synthetic.make_inputs(w, dev)
    cu = inp["cu_seqlens"]
    step, res, N, cu_host = fwd_runner(w, inp, dev)
    o = res["o"]
    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        print("[bench] warmup %d/%d done" % (i + 1, args.warmup), file=sys.stderr, flush=True)
    t = time_fwd(step, args.steps, 0)
    ms_per_step, stage_ms = t["ms"], t["stage_ms"]
    print("[bench] timed %d steps: %.3f ms/step (caches evicted), %.3f ms/step (back to back); "
          "stages (ms) %s" % (args.steps, ms_per_step, t["warm_ms"], _stage_dict(stage_ms)),
          file=sys.stderr, flush=True)

    tokens = w.B * w.T
    value = tokens / (ms_per_step / 1e3) / 1e6
    bytes_th, flops_th = algorithmic(w)
    tokh = tokens * w.H
    NT = w.B * math.ceil(w.T / w.chunk_size) if cu is None else int(
        sum(math.ceil(int(b - a) / w.chunk_size) for a, b in zip(cu_host[:-1], cu_host[1:])))
    path_bytes = path_algorithmic_bytes(w, N)
    dom = int(np.argmax(stage_ms))
    dom_ms = float(stage_ms[dom])
    achieved = path_bytes / (dom_ms / 1e3) / 1e9 if dom_ms > 0 else 0.0
    traffic = measured_traffic(kda.STAGE_NAMES[dom]) if args.workload == 3 else None
    path_traffic = measured_path_traffic() if args.workload == 3 else None
    roofline = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 5), "traffic": traffic,
                "kernel": kda.STAGE_NAMES[dom], "kernel_ms": round(dom_ms, 4),
                "bytes_per_launch": path_bytes,
                "bytes_note": "the whole forward's algorithmic bytes (1282 B per token-head at "
                              "dk=dv=128 bf16, plus fp32 states) over the dominant kernel's time",
                "traffic_over_algorithmic": None if traffic is None else round(traffic / path_bytes, 3),
                "path_traffic": path_traffic,
                "path_traffic_over_algorithmic": None if path_traffic is None else round(path_traffic / path_bytes, 3),
                "design_bytes_per_launch": stage_bytes(w, dom, NT, N)}
    path_gbs = path_bytes / (ms_per_step / 1e3) / 1e9
    mfma_util = tokh * flops_th / (ms_per_step / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS * 100
    out = {
        "metric": METRIC, "value": round(value, 4), "unit": "Mtokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "T": w.T, "H": w.H, "dk": w.K, "dv": w.V,
                   "chunk_size": w.chunk_size, "lower_bound": w.lower_bound,
                   "documents": N, "initial_state": w.init_std is not None},
        "timing": "median of per-step HIP events with 1 GiB written between steps "
                  "(last-level cache evicted); warm_* = the same steps back to back",
        "stage_ms": _stage_dict(stage_ms),
        "warm_value": round(tokens / (t["warm_ms"] / 1e3) / 1e6, 4),
        "warm_ms_per_step": round(t["warm_ms"], 4),
        "warm_stage_ms": _stage_dict(t["warm_stage_ms"]),
        "path_algorithmic_bytes": path_bytes,
        "path_algorithmic_GBps": round(path_gbs, 2),
        "path_hbm_frac": round(path_gbs / HBM_PEAK_GBS, 5),
        "mfma_util_pct_useful_flops": round(mfma_util, 3),
        "mfma_util_pct_counters": measured_mfma_util(args.workload),
        "roofline": roofline,
    }
    if not args.no_short_conv:
        print("[bench] timing the forward after the short convolution", file=sys.stderr, flush=True)
        out["short_conv"] = bench_short_conv(inp, w, o, args.steps, args.warmup)
    if not args.no_short_conv:
        out["output_norm"] = bench_output_norm(o, w, args.steps)
    if not args.no_backward:
        print("[bench] timing the backward", file=sys.stderr, flush=True)
        out["backward"] = bench_backward(inp, w, min(args.steps, 5), 1)
    if not args.no_other_workloads:
        out["workloads"] = bench_other_workloads(args.workload, min(args.steps, 10),
                                                 max(1, args.warmup), dev)
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(inp, w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
