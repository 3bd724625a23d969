"""Benchmark: hybrid temporal-attention forward tokens/s on one MI355X.

One step = one full hybrid forward (GLA branch, then SWA + DSWA with the GLA
partial added in the epilogue: the two launches hta_hybrid_fwd makes) over one
batch of the workload B=2, H=16, d=128, T=21 frames x P=1560 tokens (L=32760),
bf16 q/k/v, fp32 accumulation and output, inputs resident in HBM. After the
timed forward steps the 64-frame streaming continuation of the same workload
is timed as well (reported under "stream").

Prints ONE JSON line. With --gpus above 1 it exits: this build runs on a single
GPU (sharding is described in the design notes, not measured).
"""
from __future__ import annotations

import argparse
import hashlib
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
ATTN_KERNEL = "win_attn_bf16_kernel<2>"
PMC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic.json")
ATTN_SRC = os.path.join(ROOT, "hybrid_linear_temporal_hta_amd", "csrc", "win_attn.hip")


def attn_flops(w) -> float:
    """Algorithmic FLOPs of SWA + DSWA: 4 d P^2 per (query frame, tap frame) pair."""
    n_swa = sum(min(w.window, f + 1) for f in range(w.T))
    n_dswa = sum(sum(1 for j in range(w.taps) if f - j * w.dilation >= 0) for f in range(w.T))
    return 4.0 * w.dk * w.P * w.P * (n_swa + n_dswa) * w.B * w.H


def gla_flops(w) -> float:
    """Chunked GLA FLOPs per token (triangles at half): 5 C d + 6 d^2 + C^2 / 3."""
    C, d = w.chunk, w.dk
    return (5 * C * d + 6 * d * d + C * C / 3.0) * w.B * w.H * w.L


def gla_bytes(w, out_bytes=4) -> float:
    """Algorithmic HBM bytes of the GLA branch: q, k, v (bf16), alpha, beta, o."""
    return (3 * w.dk * 2 + 8 + w.dv * out_bytes) * w.B * w.H * w.L


def pmc_traffic():
    """HBM bytes per attention launch from the committed rocprofv3 counter runs,
    valid only while the kernel source is the one they were taken on."""
    try:
        rec = json.load(open(PMC_FILE))
        sha = hashlib.sha256(open(ATTN_SRC, "rb").read()).hexdigest()
        if rec.get("source_sha256") != sha:
            return None
        return float(rec["hbm_bytes_per_launch"])
    except Exception:
        return None


def cpu_baseline(w, x):
    """The fp64 oracle, untuned, on a bounded sample: one (batch, head) slice of
    the workload -- SWA + DSWA for all its L query rows and the GLA recurrence
    over its L tokens. That slice is 1/H of the per-token work of L tokens."""
    import numpy as np
    import oracle
    q = x["q"][0:1, 0:1].double().cpu().numpy()
    k = x["k"][0:1, 0:1].double().cpu().numpy()
    v = x["v"][0:1, 0:1].double().cpu().numpy()
    a = x["alpha"][0:1, 0:1].double().cpu().numpy()
    b = x["beta"][0:1, 0:1].double().cpu().numpy()
    rows = np.arange(w.L, dtype=np.int64)
    t0 = time.perf_counter()
    oracle.swa_rows(q, k, v, w.T, w.P, w.window, rows)
    oracle.dswa_rows(q, k, v, w.T, w.P, w.taps, w.dilation, rows)
    oracle.gla(q, k, v, a, b)
    dt = time.perf_counter() - t0
    tokens = w.L / w.H
    return {"value": tokens / dt, "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"one (batch, head) slice: SWA+DSWA for all {w.L} query rows and the GLA "
                      f"recurrence over {w.L} tokens (= {tokens:.1f} tokens x {w.H} heads), "
                      f"{dt:.1f} s wall"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--stream-steps", type=int, default=64)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

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
    prm = hta.make_params(w.window, w.taps, w.dilation, w.chunk)
    state = torch.zeros(w.B, w.H, w.dk, w.dv, device=dev)
    o = torch.empty(w.B, w.H, w.L, w.dv, dtype=torch.float32, device=dev)
    ws = torch.empty(max(hta.hta_workspace_bytes(hta.HTA_OP_GLA, hta.make_shape(x["q"], x["v"], w.P, o),
                                                 prm), 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        hta.hta_gla_fwd(x["q"], x["k"], x["v"], x["alpha"], x["beta"], state, o, w.P, w.chunk,
                        0.0, ws, stream)
        if ev is not None:
            ev[1].record(stream)
        hta.hta_swa_dswa_fwd(x["q"], x["k"], x["v"], o, w.P, prm, add=o, stream=stream)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gla_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    attn_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
    ms_per_step = wall * 1e3 / args.steps
    tokens = w.B * w.L
    value = tokens / (ms_per_step / 1e3)

    fl = attn_flops(w)
    achieved = fl / (attn_ms / 1e3) / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_MFMA_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_MFMA_BF16_TFLOPS, 4),
                "traffic": pmc_traffic(), "kernel": ATTN_KERNEL,
                "flop_per_launch": fl, "avg_launch_ms": round(attn_ms, 4)}
    gb = gla_bytes(w)
    gla = {"kernels": "gla_prep_bf16_kernel + gla_scan_bf16_kernel", "avg_ms": round(gla_ms, 4),
           "algorithmic_bytes": gb, "achieved_GBps": round(gb / (gla_ms / 1e3) / 1e9, 1),
           "frac_hbm": round(gb / (gla_ms / 1e3) / 1e9 / PEAK_HBM_GBPS, 4),
           "flop": gla_flops(w),
           "frac_mfma": round(gla_flops(w) / (gla_ms / 1e3) / 1e12 / PEAK_MFMA_BF16_TFLOPS, 4)}

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

    cpu = None if args.no_cpu_baseline else cpu_baseline(w, x)

    out = {"metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic",
           "config": {"workload": "hybrid forward B2 H16 T21 P1560 d128 (L=32760) bf16 in, fp32 out; "
                                  "SWA W=3, DSWA 4 taps dil 4, GLA chunk 64",
                      "global_batch": w.B, "seq_len": w.L, "heads": w.H, "head_dim": w.dk,
                      "parallelism": "single GPU"},
           "roofline": roofline, "gla": gla, "stream": sres, "cpu_baseline": cpu}
    print(json.dumps(out))


if __name__ == "__main__":
    main()
