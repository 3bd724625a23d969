"""Benchmark: hybrid temporal-attention forward tokens/s on one MI355X.

One step = one hta_hybrid_fwd call over one batch of the workload B=2, H=16,
d=128, T=21 frames x P=1560 tokens (L=32760), bf16 q/k/v, fp32 accumulation
and output, inputs resident in HBM. The call gets a side stream from the
caller (hta_params): the GLA prep runs first, then the GLA chunk scan on the
call's stream beside one attention pass over both windows on the side stream,
then one elementwise pass adds the two partials. The dominant kernel's roofline
is timed on that attention pass run alone (hta_swa_dswa_fwd_ex); the GLA branch
is timed alone as well. Then: the 64-frame streaming continuation of the same
workload ("stream"), the training pair on the same batch ("train"), the
336-frame long-horizon workload, the 61-frame workloads at DSWA dilations 6 and
12 ("dilated"), the attention pass at unscaled logits ("attn_unscaled"), the
input-side projection, and the chip's measured MFMA and HBM ceilings ("peaks").

Prints ONE JSON line. With --gpus above 1 it exits: this build runs on a single
GPU (sharding is described in the design notes, not measured).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "hybrid temporal-attn fwd tokens/s at L=32760,H=16,d=128; % MFMA peak"
PEAK_MFMA_BF16_TFLOPS = 2500.0      # MI355X dense bf16/fp16 MFMA
PEAK_HBM_GBPS = 8000.0              # MI355X HBM3E
NUM_CUS = 256                       # MI355X compute units
CLOCK_GHZ = 2.4                     # MI355X peak engine clock (per-CU byte rates are quoted at it)
ATTN_KERNEL = "win_attn_bf16_kernel<3>"   # both windows in one pass (own frame shared)
PMC_FILE = os.path.join(ROOT, "profiles", "win_attn_bf16_onepass_hybrid_fwd_B2H16L32760_traffic.json")
ATTN_SRC = os.path.join(ROOT, "hybrid_linear_temporal_hta_amd", "csrc", "win_attn.hip")
ATTN_LAUNCHES = 1                   # one SWA+DSWA pass per step
GLA_SRC = os.path.join(ROOT, "hybrid_linear_temporal_hta_amd", "csrc", "gla_fwd.hip")
GLA_PREP_PMC = os.path.join(ROOT, "profiles", "gla_prep2_gla_fwd_B2H16L32760_traffic.json")
GLA_SCAN_PMC = os.path.join(ROOT, "profiles", "gla_scan3_gla_fwd_B2H16L32760_traffic.json")
ATTN_MFMA = os.path.join(ROOT, "profiles", "win_attn_bf16_onepass_hybrid_fwd_B2H16L32760_mfma.json")
GLA_PREP_MFMA = os.path.join(ROOT, "profiles", "gla_prep2_gla_fwd_B2H16L32760_mfma.json")
GLA_SCAN_MFMA = os.path.join(ROOT, "profiles", "gla_scan3_gla_fwd_B2H16L32760_mfma.json")


def attn_pairs(w) -> int:
    """Distinct (query frame, key frame) pairs of SWA and DSWA together: the key
    frames of frame f are the union of the two windows, the own frame once."""
    n = 0
    for f in range(w.T):
        keys = {f - j for j in range(w.window) if f - j >= 0}
        keys |= {f - j * w.dilation for j in range(w.taps) if f - j * w.dilation >= 0}
        n += len(keys)
    return n


def attn_flops(w) -> float:
    """Algorithmic FLOPs of SWA + DSWA: 4 d P^2 (QK^T and PV) per distinct (query
    frame, key frame) pair. A frame in both windows (the own frame; with W > dil
    others too) has one set of logits and weights, so it is counted once."""
    return 4.0 * w.dk * w.P * w.P * attn_pairs(w) * w.B * w.H


def attn_flops_double_counted(w) -> float:
    """SWA and DSWA each counted in full (a frame in both windows twice): what two
    separate branch passes would execute."""
    n_swa = sum(min(w.window, f + 1) for f in range(w.T))
    n_dswa = sum(sum(1 for j in range(w.taps) if f - j * w.dilation >= 0) for f in range(w.T))
    return 4.0 * w.dk * w.P * w.P * (n_swa + n_dswa) * w.B * w.H


def gla_flops(w) -> float:
    """Chunked GLA FLOPs per token (triangles at half): 5 C d + 6 d^2 + C^2 / 3."""
    C, d = w.chunk, w.dk
    return (5 * C * d + 6 * d * d + C * C / 3.0) * w.B * w.H * w.L


def cpu_info():
    """Host CPU model and logical CPU count (what the CPU baseline ran on)."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return model, os.cpu_count()


def gla_bytes(w, out_bytes=4) -> float:
    """Algorithmic HBM bytes of the GLA branch: q, k, v (bf16), alpha, beta, o."""
    return (3 * w.dk * 2 + 8 + w.dv * out_bytes) * w.B * w.H * w.L


def pmc_traffic(path: str, src: str):
    """HBM bytes per launch of one kernel from committed rocprofv3 counter runs
    (FETCH_SIZE + WRITE_SIZE, scaled by a copy-kernel calibration), valid only
    while the kernel source is the one they were taken on (else None)."""
    try:
        from hybrid_linear_temporal_hta_amd.profiling import source_digest
        rec = json.load(open(path))
        if rec.get("source_digest") != source_digest(src):
            return None
        return float(rec["hbm_bytes_per_launch"])
    except (OSError, ValueError, KeyError):
        return None


def profiled_mfma_busy(path: str, src: str):
    """MFMA busy fraction of a kernel from a committed rocprofv3 counter summary
    (busy cycles per SIMD over the kernel's active cycles), valid only while the
    kernel source is the one it was taken on (else None)."""
    try:
        from hybrid_linear_temporal_hta_amd.profiling import source_digest
        rec = json.load(open(path))
        if rec.get("source_digest") != source_digest(src):
            return None
        return round(float(rec["mfma_busy_frac"]), 4)
    except (OSError, ValueError, KeyError, TypeError):
        return None


COPY_BYTES = 1 << 30        # the calibration and measured-peak copy: 1 GiB read, 1 GiB written


def copy_calibration(steps: int):
    """A plain copy of known size for counter calibration: hbm_copy_kernel
    (libhta_peaks) copying COPY_BYTES, `steps` launches."""
    import torch
    from hybrid_linear_temporal_hta_amd import peaks
    dev = torch.device("cuda:0")
    src = torch.ones(COPY_BYTES // 4, device=dev)
    dst = torch.empty_like(src)
    for _ in range(steps):
        peaks.copy(src, dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_kernel": "hbm_copy_kernel", "launches": steps,
                      "bytes_read_per_launch": COPY_BYTES, "bytes_written_per_launch": COPY_BYTES}))


def measured_peaks(dev, stream):
    """The chip's ceilings as plain kernels reach them (libhta_peaks): an MFMA
    issue loop (bf16 32x32x16, register operands, 4 workgroups of 4 waves per
    CU) and a 1 GiB HBM copy, both timed with HIP events on `stream`."""
    import torch
    from hybrid_linear_temporal_hta_amd import peaks
    blocks, iters = 1024, 8000
    sink = torch.empty(blocks * 256, device=dev)
    mfma_ms = timed_events(lambda: peaks.mfma(blocks, iters, sink, stream), 5, 2, stream)
    fl = peaks.mfma_flop(blocks, iters)
    src = torch.ones(COPY_BYTES // 4, device=dev)
    dst = torch.empty_like(src)
    copy_ms = timed_events(lambda: peaks.copy(src, dst, stream), 10, 2, stream)
    del src, dst
    torch.cuda.empty_cache()
    # the on-chip paths of the kernels' tiles: direct global->LDS loads from an
    # L2-resident 2 MiB window (contiguous 1 KiB, and 32 rows x 32 bytes), and LDS
    # reads (ds_read_b128, ds_read_b64_tr_b16); two workgroups per CU
    win = 1 << 21
    lsrc = torch.ones(win // 4, device=dev)
    onchip = {}
    for name, pattern in (("l2_to_lds_contiguous", 0), ("l2_to_lds_32B_rows", 1)):
        ms = timed_events(lambda: peaks.lds_dma(lsrc, win, 512, 400, pattern, stream), 5, 1, stream)
        onchip[name] = peaks.lds_dma_bytes(512, 400) / (ms / 1e3)
    lsink = torch.empty(512 * 256, device=dev)
    for name, tr in (("lds_read_b128", False), ("lds_read_b64_tr_b16", True)):
        ms = timed_events(lambda: peaks.lds_read(512, 4000, tr, lsink, stream), 5, 1, stream)
        onchip[name] = peaks.lds_read_bytes(512, 4000, tr) / (ms / 1e3)
    del lsrc, lsink
    onchip_rates = {k: {"TBps": round(v / 1e12, 2),
                        "B_per_clk_per_CU": round(v / (NUM_CUS * CLOCK_GHZ * 1e9), 1)}
                    for k, v in onchip.items()}
    return {"mfma_kernel": "mfma_loop_kernel (v_mfma_f32_32x32x16_bf16)",
            "mfma_TFLOPs": round(fl / (mfma_ms / 1e3) / 1e12, 1),
            "mfma_frac_of_spec": round(fl / (mfma_ms / 1e3) / 1e12 / PEAK_MFMA_BF16_TFLOPS, 4),
            "copy_kernel": "hbm_copy_kernel", "copy_bytes_moved": 2 * COPY_BYTES,
            "hbm_copy_GBps": round(2 * COPY_BYTES / (copy_ms / 1e3) / 1e9, 1),
            "hbm_frac_of_spec": round(2 * COPY_BYTES / (copy_ms / 1e3) / 1e9 / PEAK_HBM_GBPS, 4),
            "onchip": onchip_rates,
            "onchip_clock_GHz": CLOCK_GHZ}


def cpu_baseline(w, x, heads: int):
    """The fp64 oracle, untuned, on a bounded sample: `heads` heads of batch 0
    -- SWA + DSWA for all their L query rows and the GLA recurrence over their
    L tokens. A token of the metric carries H heads, so the sample is worth
    L * heads / H tokens."""
    import numpy as np
    import oracle
    sl = (slice(0, 1), slice(0, heads))
    q = x["q"][sl].double().cpu().numpy()
    k = x["k"][sl].double().cpu().numpy()
    v = x["v"][sl].double().cpu().numpy()
    a = x["alpha"][sl].double().cpu().numpy()
    b = x["beta"][sl].double().cpu().numpy()
    t0 = time.perf_counter()
    oracle.swa(q, k, v, w.T, w.P, w.window)
    oracle.dswa(q, k, v, w.T, w.P, w.taps, w.dilation)
    oracle.gla(q, k, v, a, b)
    dt = time.perf_counter() - t0
    tokens = w.L * heads / w.H
    model, nproc = cpu_info()
    return {"value": round(tokens / dt, 1), "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle", "cpu_model": model, "nproc": nproc,
            "sample": f"{heads} of {w.H} heads of batch 0: SWA + DSWA for all {w.L} query rows "
                      f"and the GLA recurrence over all {w.L} tokens of each head "
                      f"(= {tokens:.0f} tokens of {w.H} heads), {dt:.1f} s wall"}


def setup(hta, w, x, dev, side=None):
    import torch
    prm = hta.make_params(w.window, w.taps, w.dilation, w.chunk, side=side)
    state = torch.zeros(w.B, w.H, w.dk, w.dv, device=dev)
    o = torch.empty(w.B, w.H, w.L, w.dv, dtype=torch.float32, device=dev)
    nws = hta.hta_workspace_bytes(hta.HTA_OP_HYBRID, hta.make_shape(x["q"], x["v"], w.P, o), prm)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    return prm, state, o, ws


def concurrent_side(hta, dev, make_call, tries=4):
    """A side stream that runs beside the caller's stream. HIP deals its streams
    out over a few hardware queues in turn, and two streams that share a queue run
    one after the other (the results are the same, the overlap is lost), so of
    `tries` new side streams this takes the one with which `make_call(side)()` is
    fastest: one warm-up call and two timed calls each."""
    import time
    import torch
    best = None
    for _ in range(tries):
        side = hta.SideStream(dev)
        fn = make_call(side)
        fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        fn()
        fn()
        torch.cuda.synchronize()
        t = time.perf_counter() - t0
        if best is None or t < best[0]:
            best = (t, side)
    return best[1]


def attn_ws(hta, w, x, o, prm, dev):
    import torch
    n = hta.hta_workspace_bytes(hta.HTA_OP_SWA_DSWA, hta.make_shape(x["q"], x["v"], w.P, o), prm)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=dev)


def timed_wall(fn, steps, warmup):
    """Wall time (ms) per call of `steps` calls after `warmup`, bracketed by
    device synchronisation."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def timed_events(fn, steps, warmup, stream):
    """Mean HIP-event time (ms) of `fn` on `stream` over `steps` calls."""
    import torch
    for _ in range(warmup):
        fn()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    torch.cuda.synchronize()
    for e0, e1 in evs:
        e0.record(stream)
        fn()
        e1.record(stream)
    torch.cuda.synchronize()
    return sum(e0.elapsed_time(e1) for e0, e1 in evs) / steps


def hybrid_call(hta, w, x, state, o, ws, prm, stream):
    """One hybrid forward through the library's entry point."""
    return lambda: hta.hta_hybrid_fwd(x["q"], x["k"], x["v"], x["alpha"], x["beta"], state, o,
                                      w.P, prm, workspace=ws, stream=stream)


def long_horizon(hta, dev, steps, side):
    """The 336-frame workload (B1 H16, L=524160): tokens/s and attention FLOP/s,
    to set beside the 21-frame figures (flatness in L)."""
    import torch
    from hybrid_linear_temporal_hta_amd.inputs import WORKLOADS, make_inputs
    w = WORKLOADS["long_horizon"]
    x = make_inputs(w, device=dev)
    prm, state, o, ws = setup(hta, w, x, dev, side=side)
    stream = torch.cuda.current_stream()
    ms = timed_wall(hybrid_call(hta, w, x, state, o, ws, prm, stream), steps, 1)
    wsa = attn_ws(hta, w, x, o, prm, dev)
    attn_ms = timed_events(lambda: hta.hta_swa_dswa_fwd_ex(x["q"], x["k"], x["v"], o, w.P, prm,
                                                           workspace=wsa, stream=stream),
                           steps, 0, stream)
    gla_ms = timed_events(lambda: hta.hta_gla_fwd(x["q"], x["k"], x["v"], x["alpha"], x["beta"],
                                                  state, o, w.P, w.chunk, 0.0, ws, stream),
                          steps, 0, stream)
    fl = attn_flops(w)
    res = {"workload": "B1 H16 T336 P1560 d128 (L=524160)", "steps": steps,
           "ms_per_step": round(ms, 3), "tokens_per_s": round(w.B * w.L / (ms / 1e3), 1),
           "attn_ms": round(attn_ms, 3), "gla_ms": round(gla_ms, 3),
           "attn_tflops": round(fl / (attn_ms / 1e3) / 1e12, 1),
           "attn_tap_frames_per_token": round(fl / (4.0 * w.dk * w.P * w.B * w.H * w.L), 3)}
    del x, o, ws
    torch.cuda.empty_cache()
    return res


def dilated(hta, dev, steps, side):
    """The 61-frame workloads at the pages' DSWA dilations 6 and 12 (B1 H16,
    P=1560, L=95160, W=3, 4 taps): the hybrid forward (side stream) and the
    attention pass alone, with its MFMA fraction."""
    import torch
    from hybrid_linear_temporal_hta_amd.inputs import WORKLOADS, make_inputs
    out = []
    stream = torch.cuda.current_stream()
    for name in ("dilated_d6", "dilated_d12"):
        w = WORKLOADS[name]
        x = make_inputs(w, device=dev)
        prm, state, o, ws = setup(hta, w, x, dev, side=side)
        ms = timed_wall(hybrid_call(hta, w, x, state, o, ws, prm, stream), steps, 1)
        wsa = attn_ws(hta, w, x, o, prm, dev)
        attn_ms = timed_events(lambda: hta.hta_swa_dswa_fwd_ex(x["q"], x["k"], x["v"], o, w.P,
                                                               prm, workspace=wsa, stream=stream),
                               steps, 1, stream)
        fl = attn_flops(w)
        out.append({"workload": f"B{w.B} H{w.H} T{w.T} P{w.P} d{w.dk} (L={w.L}), W={w.window}, "
                                f"{w.taps} taps dil {w.dilation}",
                    "steps": steps, "ms_per_step": round(ms, 3),
                    "tokens_per_s": round(w.B * w.L / (ms / 1e3), 1),
                    "attn_ms": round(attn_ms, 3), "attn_flop": fl,
                    "attn_frac_mfma": round(fl / (attn_ms / 1e3) / 1e12 / PEAK_MFMA_BF16_TFLOPS, 4),
                    "hybrid_frac_mfma": round((fl + gla_flops(w)) / (ms / 1e3) / 1e12
                                              / PEAK_MFMA_BF16_TFLOPS, 4)})
        del x, o, ws, wsa
        torch.cuda.empty_cache()
    return out


def attn_unscaled(hta, dev, steps):
    """The attention pass of the metric workload with q, k ~ N(0, 1) (no data
    scaling; logits of std 1 after the 1/sqrt(d) softmax scale), so the online
    softmax's running maximum moves and its rescale runs; beside the same pass
    on the metric's inputs (logits of std 1/sqrt(d))."""
    import torch
    from hybrid_linear_temporal_hta_amd.inputs import WORKLOADS, make_inputs
    w = WORKLOADS["hybrid_stream"].replace(qv_std=1.0, k_std=1.0, k_unit=False,
                                           stream_frames=0, seed=7)
    x = make_inputs(w, device=dev)
    stream = torch.cuda.current_stream()
    prm = hta.make_params(w.window, w.taps, w.dilation, w.chunk)
    o = torch.empty(w.B, w.H, w.L, w.dv, dtype=torch.float32, device=dev)
    wsa = attn_ws(hta, w, x, o, prm, dev)
    ms = timed_events(lambda: hta.hta_swa_dswa_fwd_ex(x["q"], x["k"], x["v"], o, w.P, prm,
                                                      workspace=wsa, stream=stream),
                      steps, 1, stream)
    fl = attn_flops(w)
    qk = (x["q"][0, 0, :4096].float() @ x["k"][0, 0, :4096].float().T) / w.dk ** 0.5
    res = {"workload": "B2 H16 T21 P1560 d128, q, k, v ~ N(0, 1)", "avg_launch_ms": round(ms, 4),
           "achieved_TFLOPs": round(fl / (ms / 1e3) / 1e12, 1),
           "frac": round(fl / (ms / 1e3) / 1e12 / PEAK_MFMA_BF16_TFLOPS, 4),
           "logit_std_sample": round(float(qk.std()), 3)}
    del x, o, wsa
    torch.cuda.empty_cache()
    return res


def projection(hta, dev, steps):
    """The input side (NEXT to the hot path): per-token q, k, v, alpha, beta for the
    workload's tokens (B2, L = 32760) from model width 2048 (= H x d), one GEMM
    of 2 * M * Dm * N FLOP with the fused epilogue; its MFMA roofline."""
    import torch
    B, L, H, Dm = 2, 32760, 16, 2048
    N = 3 * H * 128 + 2 * H
    g = torch.Generator(device=dev)
    g.manual_seed(21)
    x = torch.randn(B, L, Dm, generator=g, device=dev).to(torch.bfloat16)
    w = (torch.randn(Dm, N, generator=g, device=dev) / Dm ** 0.5).to(torch.bfloat16)
    q, k, v = (torch.empty(B, H, L, 128, dtype=torch.bfloat16, device=dev) for _ in range(3))
    al, be = (torch.empty(B, H, L, device=dev) for _ in range(2))
    stream = torch.cuda.current_stream()
    ms = timed_events(lambda: hta.hta_project_fwd(x, w, q, k, v, al, be, 1560, stream=stream),
                      steps, 2, stream)
    fl = 2.0 * B * L * Dm * N
    tf = fl / (ms / 1e3) / 1e12
    return {"kernel": "project_kernel", "workload": "B2 L32760 H16 d128, model width 2048",
            "avg_launch_ms": round(ms, 4), "flop_per_launch": fl, "achieved_TFLOPs": round(tf, 1),
            "frac_mfma": round(tf / PEAK_MFMA_BF16_TFLOPS, 4)}


def train(hta, w, x, dev, steps, warmup, cpu_heads, side):
    """The training pair on the same batch (NEXT to the forward hot path), with a
    side stream: one step = hta_hybrid_fwd_train + hta_hybrid_bwd (dL/do ~ N(0, 1), fp32), wall
    time; the backward alone and each attention branch's backward alone
    (HIP events), with the attention backward's MFMA roofline: its algorithmic
    work is 2.5x the branch's forward (recompute S, then dP, dV, dK, dQ: five
    products of 2 d P^2 per (query frame, tap frame) pair against two)."""
    import torch
    from hybrid_linear_temporal_hta_amd.inputs import make_output_grad
    # with a side stream, as the forward metric: the GLA backward runs beside the
    # SWA backward
    prm = hta.make_params(w.window, w.taps, w.dilation, w.chunk, side=side)
    q, k, v, a, b = x["q"], x["k"], x["v"], x["alpha"], x["beta"]
    o = torch.empty(w.B, w.H, w.L, w.dv, dtype=torch.float32, device=dev)
    st = torch.zeros(w.B, w.H, w.dk, w.dv, device=dev)
    shape = hta.make_shape(q, v, w.P, o)
    saved = torch.empty(hta.hta_hybrid_saved_bytes(shape), dtype=torch.uint8, device=dev)
    wsf = torch.empty(hta.hta_workspace_bytes(hta.HTA_OP_HYBRID, shape, prm), dtype=torch.uint8,
                      device=dev)
    wsb = torch.empty(hta.hta_workspace_bytes(hta.HTA_OP_HYBRID_BWD, shape, prm),
                      dtype=torch.uint8, device=dev)
    wsa = torch.empty(hta.hta_workspace_bytes(hta.HTA_OP_ATTN_BWD, shape, None),
                      dtype=torch.uint8, device=dev)
    dout = make_output_grad(w.replace(stream_frames=0), device=dev).to(torch.float32)
    dq, dk, dv = (torch.empty_like(t) for t in (q, k, v))
    da, db = torch.empty_like(a), torch.empty_like(b)
    dst = torch.zeros_like(st)
    stream = torch.cuda.current_stream()

    def step():
        hta.hta_hybrid_fwd_train(q, k, v, a, b, st, o, saved, w.P, prm, workspace=wsf,
                                 stream=stream)
        hta.hta_hybrid_bwd(q, k, v, a, b, saved, dout, dst, dq, dk, dv, da, db, w.P, prm,
                           workspace=wsb, stream=stream)
    step_ms = timed_wall(step, steps, warmup)
    bwd_ms = timed_events(lambda: hta.hta_hybrid_bwd(q, k, v, a, b, saved, dout, dst, dq, dk, dv,
                                                     da, db, w.P, prm, workspace=wsb,
                                                     stream=stream), steps, 1, stream)
    lse = torch.empty(w.B, w.H, w.L, device=dev)
    ob = torch.empty_like(o)
    hta.hta_swa_fwd_lse(q, k, v, ob, lse, w.P, w.window, stream=stream)
    swa_ms = timed_events(lambda: hta.hta_swa_bwd(q, k, v, ob, lse, dout, dq, dk, dv, w.P,
                                                  w.window, workspace=wsa, stream=stream),
                          steps, 1, stream)
    hta.hta_dswa_fwd_lse(q, k, v, ob, lse, w.P, w.taps, w.dilation, stream=stream)
    dswa_ms = timed_events(lambda: hta.hta_dswa_bwd(q, k, v, ob, lse, dout, dq, dk, dv, w.P,
                                                    w.taps, w.dilation, workspace=wsa,
                                                    stream=stream), steps, 1, stream)
    fl_branch = attn_flops_double_counted(w) / 2   # SWA and DSWA: equal tap-frame counts here
    fl_bwd = 2.5 * fl_branch
    att_ms = (swa_ms + dswa_ms) / 2
    achieved = fl_bwd / (att_ms / 1e3) / 1e12
    res = {"workload": "B2 H16 T21 P1560 d128 (L=32760) bf16 in, fp32 out and dL/do",
           "steps": steps, "ms_per_step": round(step_ms, 3),
           "tokens_per_s": round(w.B * w.L / (step_ms / 1e3), 1),
           "bwd_ms": round(bwd_ms, 3),
           "attn_bwd_roofline": {"bound": "mfma", "achieved": round(achieved, 2),
                                 "peak": PEAK_MFMA_BF16_TFLOPS, "unit": "TFLOP/s",
                                 "frac": round(achieved / PEAK_MFMA_BF16_TFLOPS, 4),
                                 "calls": "hta_swa_bwd, hta_dswa_bwd (prep + query pass + key pass)",
                                 "flop_per_call": fl_bwd, "avg_call_ms": round(att_ms, 4)}}
    if cpu_heads > 0:
        res["cpu_baseline"] = cpu_baseline_bwd(w, x, dout, cpu_heads)
    del saved, wsf, wsb, wsa
    torch.cuda.empty_cache()
    return res


def cpu_baseline_bwd(w, x, dout, heads: int, frames: int = 2):
    """The fp64 oracle's hybrid backward, untuned, on a bounded sample: `heads`
    heads of batch 0 over the first `frames` frames (the attention windows are
    shorter there than in the full sequence, so this over-states the oracle's
    rate on the workload). A token carries H heads: the sample is worth
    frames * P * heads / H tokens."""
    import oracle
    n = frames * w.P
    sl = (slice(0, 1), slice(0, heads), slice(0, n))
    f = lambda t: t[sl].double().cpu().numpy()
    q, k, v, a, b = f(x["q"]), f(x["k"]), f(x["v"]), f(x["alpha"]), f(x["beta"])
    do = f(dout.to(w.dtype))
    t0 = time.perf_counter()
    oracle.hybrid_bwd(q, k, v, a, b, do, frames, w.P, w.window, w.taps, w.dilation)
    dt = time.perf_counter() - t0
    tokens = n * heads / w.H
    model, nproc = cpu_info()
    return {"value": round(tokens / dt, 1), "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle", "cpu_model": model, "nproc": nproc,
            "sample": f"hybrid backward of {heads} of {w.H} heads of batch 0 over the first "
                      f"{frames} frames ({n} tokens each; = {tokens:.0f} tokens of {w.H} heads), "
                      f"{dt:.1f} s wall"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--stream-steps", type=int, default=64)
    ap.add_argument("--long-horizon-steps", type=int, default=2)
    ap.add_argument("--dilated-steps", type=int, default=3)
    ap.add_argument("--unscaled-steps", type=int, default=5)
    ap.add_argument("--project-steps", type=int, default=10)
    ap.add_argument("--train-steps", type=int, default=10)
    ap.add_argument("--peaks", type=int, default=1, help="measure the MFMA and HBM ceilings (0: skip)")
    ap.add_argument("--cpu-heads", type=int, default=8,
                    help="heads of batch 0 the CPU oracle baseline runs (0: skip it)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="CALLS",
                    help="only run CALLS copies of known size (counter calibration) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    import torch
    from hybrid_linear_temporal_hta_amd import hta
    from hybrid_linear_temporal_hta_amd.inputs import WORKLOADS, make_inputs

    w = WORKLOADS["hybrid_stream"]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    full = make_inputs(w, device=dev)                      # prefix + streamed frames
    nP = w.T * w.P
    x = {k: (t[:, :, :nP].contiguous() if k in ("q", "k", "v", "alpha", "beta") else t)
         for k, t in full.items()}
    _, state, o, ws = setup(hta, w, x, dev)
    stream = torch.cuda.current_stream()
    side = concurrent_side(hta, dev, lambda s: hybrid_call(
        hta, w, x, state, o, ws, hta.make_params(w.window, w.taps, w.dilation, w.chunk, side=s), stream))
    prm = hta.make_params(w.window, w.taps, w.dilation, w.chunk, side=side)
    # The metric: the library's hybrid forward, the attention pass on the side stream.
    ms_per_step = timed_wall(hybrid_call(hta, w, x, state, o, ws, prm, stream), args.steps,
                             args.warmup)
    tokens = w.B * w.L
    value = tokens / (ms_per_step / 1e3)
    # The same call with every launch on one stream (no side stream), for context.
    prm1 = hta.make_params(w.window, w.taps, w.dilation, w.chunk)
    ms_single = timed_wall(hybrid_call(hta, w, x, state, o, ws, prm1, stream), args.steps, 1)
    # Roofline of the dominant kernel: the hybrid's attention pass (both windows in
    # one launch), alone on the stream, timed with HIP events on that stream.
    wsa = attn_ws(hta, w, x, o, prm1, dev)
    attn_ms = timed_events(lambda: hta.hta_swa_dswa_fwd_ex(x["q"], x["k"], x["v"], o, w.P, prm1,
                                                           workspace=wsa, stream=stream),
                           args.steps, 1, stream)
    # The GLA branch alone (prep + scan), for its own HBM fraction.
    gla_ms = timed_events(lambda: hta.hta_gla_fwd(x["q"], x["k"], x["v"], x["alpha"], x["beta"],
                                                  state, o, w.P, w.chunk, 0.0, ws, stream),
                          args.steps, 1, stream)

    fl = attn_flops(w)
    launch_ms = attn_ms / ATTN_LAUNCHES
    fl_launch = fl / ATTN_LAUNCHES
    achieved = fl_launch / (launch_ms / 1e3) / 1e12
    dbl = attn_flops_double_counted(w) / ATTN_LAUNCHES / (launch_ms / 1e3) / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_MFMA_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_MFMA_BF16_TFLOPS, 4),
                "traffic": pmc_traffic(PMC_FILE, ATTN_SRC), "kernel": ATTN_KERNEL,
                "launches_per_step": ATTN_LAUNCHES, "flop_per_launch": fl_launch,
                "avg_launch_ms": round(launch_ms, 4),
                "double_counted_TFLOPs": round(dbl, 2),
                "double_counted_frac": round(dbl / PEAK_MFMA_BF16_TFLOPS, 4),
                "mfma_busy_frac_profiled": profiled_mfma_busy(ATTN_MFMA, ATTN_SRC)}
    gb = gla_bytes(w)
    gla = {"kernels": "gla_prep2_kernel + gla_scan3_kernel", "avg_ms": round(gla_ms, 4),
           "algorithmic_bytes": gb, "achieved_GBps": round(gb / (gla_ms / 1e3) / 1e9, 1),
           "frac_hbm": round(gb / (gla_ms / 1e3) / 1e9 / PEAK_HBM_GBPS, 4),
           "flop": gla_flops(w),
           "frac_mfma": round(gla_flops(w) / (gla_ms / 1e3) / 1e12 / PEAK_MFMA_BF16_TFLOPS, 4),
           "traffic_prep": pmc_traffic(GLA_PREP_PMC, GLA_SRC),
           "traffic_scan": pmc_traffic(GLA_SCAN_PMC, GLA_SRC),
           "mfma_busy_frac_profiled": {"prep": profiled_mfma_busy(GLA_PREP_MFMA, GLA_SRC),
                                       "scan": profiled_mfma_busy(GLA_SCAN_MFMA, GLA_SRC)}}
    hybrid_frac = (fl + gla_flops(w)) / (ms_per_step / 1e3) / 1e12 / PEAK_MFMA_BF16_TFLOPS

    # Streaming continuation: prefix = the 21 frames above, then one frame per step.
    sres = None
    if args.stream_steps > 0:
        st = hta.Stream(w.B, w.H, w.P, w.dk, w.dtype, prm, w.ring, device=dev)
        hta.hta_stream_init(st, x["k"], x["v"], w.T, state, stream=stream)
        frames = []
        for n in range(args.stream_steps):
            sl = slice((w.T + n) * w.P, (w.T + n + 1) * w.P)
            frames.append({k: full[k][:, :, sl].contiguous() for k in ("q", "k", "v", "alpha", "beta")})
        of = torch.empty(w.B, w.H, w.P, w.dv, dtype=torch.float32, device=dev)
        e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        torch.cuda.synchronize()
        e0.record(stream)
        for f in frames:
            hta.hta_stream_step(st, f["q"], f["k"], f["v"], f["alpha"], f["beta"], of, stream=stream)
        e1.record(stream)
        for f in frames:      # commit only (ring append + state advance), same frames again
            hta.hta_stream_step(st, f["q"], f["k"], f["v"], f["alpha"], f["beta"], None, stream=stream)
        e2.record(stream)
        torch.cuda.synchronize()
        ns = args.stream_steps
        full_ms = e0.elapsed_time(e1) / ns
        commit_ms = e1.elapsed_time(e2) / ns
        commit_bytes = w.B * w.H * (w.P * (2 * w.dk * 2 * 2 + 8) + 2 * w.dk * w.dv * 4)
        sres = {"steps": ns, "frame_tokens": w.B * w.P, "ms_per_step": round(full_ms, 4),
                "tokens_per_s": round(w.B * w.P / (full_ms / 1e3), 1),
                "commit_only_ms_per_step": round(commit_ms, 4),
                "commit_only_algorithmic_bytes": commit_bytes,
                "commit_only_frac_hbm": round(commit_bytes / (commit_ms / 1e3) / 1e9 / PEAK_HBM_GBPS, 4)}
        del frames, st
    del full
    torch.cuda.empty_cache()

    tr = train(hta, w, x, dev, args.train_steps, 2, args.cpu_heads, side) if args.train_steps > 0 else None
    lh = long_horizon(hta, dev, args.long_horizon_steps, side) if args.long_horizon_steps > 0 else None
    dl = dilated(hta, dev, args.dilated_steps, side) if args.dilated_steps > 0 else None
    un = attn_unscaled(hta, dev, args.unscaled_steps) if args.unscaled_steps > 0 else None
    proj = projection(hta, dev, args.project_steps) if args.project_steps > 0 else None
    pk = measured_peaks(dev, stream) if args.peaks else None
    if pk:
        roofline["frac_of_measured_mfma"] = round(achieved / pk["mfma_TFLOPs"], 4)
        gla["frac_of_measured_hbm"] = round(gb / (gla_ms / 1e3) / 1e9 / pk["hbm_copy_GBps"], 4)
    cpu = cpu_baseline(w, x, args.cpu_heads) if args.cpu_heads > 0 else None

    out = {"metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic",
           "config": {"workload": "hybrid forward B2 H16 T21 P1560 d128 (L=32760) bf16 in, fp32 out; "
                                  "SWA W=3, DSWA 4 taps dil 4, GLA chunk 64",
                      "global_batch": w.B, "seq_len": w.L, "heads": w.H, "head_dim": w.dk,
                      "parallelism": "single GPU"},
           "roofline": roofline, "hybrid_frac_mfma": round(hybrid_frac, 4),
           "hybrid_flop": fl + gla_flops(w), "ms_per_step_single_stream": round(ms_single, 4),
           "gla": gla, "stream": sres, "long_horizon": lh, "dilated": dl, "attn_unscaled": un,
           "project": proj, "train": tr, "peaks": pk, "cpu_baseline": cpu}
    print(json.dumps(out))


if __name__ == "__main__":
    main()
