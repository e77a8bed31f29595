"""Benchmark of the KDA / gated delta rule hot path on one MI355X.

Prints ONE JSON line.  Headline: chunkwise prefill (kda_chunk_fwd) on the
Gated DeltaNet workload B=4, H=16, L=4096, d_k=d_v=128, bf16 q/k/v, fp32 gates
and state; one step = one kda_chunk_fwd over that batch (o and S_final
written).  Decode leg in the same line: the KDA decode workload, 256 sequences
x 32 heads, fp32 state updated in place for 64 steps.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload N]

Inputs are seeded synthetic data (linear_attention_sequence_kda_amd.inputs),
resident in HBM before the timed region.  The CPU baseline is the fp64 oracle
(oracle/, C, all host cores of this job) timed on the same workload.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_MFMA_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 MFMA, TFLOP/s
FP32_MFMA_PEAK_TFLOPS = 157.3   # MI355X fp32 (vector / MFMA) figure, TFLOP/s
CHUNK = 64


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def esize(dt):
    return 2 if dt == "bf16" else 4


def prefill_bytes(w):
    """Compulsory HBM bytes of one kda_chunk_fwd (each tensor touched once)."""
    tok = w.B * w.H * w.L
    eq, eg = esize(w.qkv_dtype), esize(w.gate_dtype)
    b = tok * (2 * w.dk + 2 * w.dv) * eq          # q, k, v read; o written
    if w.alpha_mode == "channel":
        b += tok * w.dk * eg
    elif w.alpha_mode == "head":
        b += tok * eg
    b += tok * eg                                  # beta
    b += w.B * w.H * w.dk * w.dv * 4               # S_final written
    if w.s0_std is not None:
        b += w.B * w.H * w.dk * w.dv * 4           # S0 read
    return b


def prefill_flops(w):
    """Algorithmic flops: 6 dk dv + 2C(3 dk + 2 dv) per token-head (C = 64):
    state products Q S, W S, K^T u (2 dk dv each) and the full CxC chunk
    blocks A, P, T K, T V ("2Ld^2 + 2LCd" counted the same way)."""
    per = 6 * w.dk * w.dv + 2 * CHUNK * (3 * w.dk + 2 * w.dv)
    return w.B * w.H * w.L * per


def decode_bytes(w):
    """Compulsory HBM bytes of one decode step: state read + write, inputs, o."""
    bh = w.B * w.H
    eq, eg = esize(w.qkv_dtype), esize(w.gate_dtype)
    b = bh * w.dk * w.dv * 4 * 2
    b += bh * (2 * w.dk + w.dv) * eq + bh * w.dv * eq
    b += bh * (w.dk if w.alpha_mode == "channel" else 1) * eg + bh * eg
    return b


def to_dev(torch, arr, dt):
    if arr is None:
        return None
    if dt == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(
            torch.bfloat16).to("cuda:0")
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to("cuda:0")


def bench_prefill(torch, kda, gen, w, steps, warmup):
    log(f"prefill workload {w.name}: drawing inputs")
    x = gen.prefill_inputs(w, threads=16)
    d = {n: to_dev(torch, x[n], w.qkv_dtype if n in ("q", "k", "v") else w.gate_dtype)
         for n in ("q", "k", "v", "log_alpha", "beta")}
    S0 = to_dev(torch, x["S0"], "f32") if x["S0"] is not None else None
    o = torch.empty((w.B, w.H, w.L, w.dv), dtype=d["v"].dtype, device="cuda:0")
    Sf = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device="cuda:0")
    args = (d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], S0)
    for _ in range(warmup):
        kda.chunk_fwd(*args, o=o, S_final=Sf)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s, e in ev:
        s.record()
        kda.chunk_fwd(*args, o=o, S_final=Sf)
        e.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = [s.elapsed_time(e) for s, e in ev]
    return x, wall, kern_ms


def bench_decode(torch, kda, gen, w):
    log(f"decode workload {w.name}: drawing inputs")
    T = w.decode_steps
    steps = []
    for t in range(T):
        xt = gen.decode_inputs(w, t)
        steps.append(tuple(to_dev(torch, xt[n], w.qkv_dtype if n in ("q", "k", "v")
                                  else w.gate_dtype)
                           for n in ("q", "k", "v", "log_alpha", "beta")))
    S0 = to_dev(torch, gen.decode_state(w), "f32")
    S = S0.clone()
    o = torch.empty((w.B, w.H, w.dv), dtype=steps[0][2].dtype, device="cuda:0")
    # warm-up pass over all steps, then restore the state outside the timing
    for st in steps:
        kda.decode_step(*st, S, o=o)
    S.copy_(S0)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(T)]
    t0 = time.perf_counter()
    for st, (s, e) in zip(steps, ev):
        s.record()
        kda.decode_step(*st, S, o=o)
        e.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, [s.elapsed_time(e) for s, e in ev]


def cpu_baseline(gen, w, x):
    """The fp64 oracle (C, threads over (head, 32-column block)) on the whole
    prefill workload."""
    import oracle
    N = w.B * w.H
    f = lambda a: None if a is None else a.reshape((N,) + a.shape[2:])
    threads = oracle.default_threads()
    log(f"cpu baseline: oracle on the full workload with {threads} threads")
    t0 = time.perf_counter()
    oracle.forward(f(x["q"]), f(x["k"]), f(x["v"]), f(x["log_alpha"]), f(x["beta"]),
                   f(x["S0"]), qkv_dtype=w.qkv_dtype, gate_dtype=w.gate_dtype,
                   alpha_mode=w.alpha_mode, want_o=True, threads=threads)
    dt = time.perf_counter() - t0
    return {"value": w.B * w.L / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"full {w.name} workload ({N} heads x {w.L} tokens, all columns), "
                      f"{dt:.2f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=2, help="prefill workload number (1-4)")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 256 MiB device copy (a known-size "
                         "reference for hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (got --gpus {args.gpus}): the KDA hot path "
              "here is a single-GPU kernel library with no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch
    import linear_attention_sequence_kda_amd as kda
    from linear_attention_sequence_kda_amd import inputs as gen

    kda.library()  # fail loudly if the HIP library is missing
    if args.copy_calibration:
        src = torch.ones(64 << 20, dtype=torch.float32, device="cuda:0")  # 256 MiB
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    w = gen.WORKLOADS[args.workload]
    x, wall, kern_ms = bench_prefill(torch, kda, gen, w, args.steps, args.warmup)
    ms_per_step = wall * 1e3 / args.steps
    tokens = w.B * w.L
    value = tokens / (wall / args.steps)
    kavg = float(np.mean(kern_ms))
    bytes_ = prefill_bytes(w)
    flops = prefill_flops(w)
    gbs = bytes_ / (kavg * 1e-3) / 1e9
    tflops = flops / (kavg * 1e-3) / 1e12
    mfma_peak = BF16_MFMA_PEAK_TFLOPS if w.qkv_dtype == "bf16" else FP32_MFMA_PEAK_TFLOPS
    log(f"prefill: {ms_per_step:.4f} ms/step wall, kernel avg {kavg*1e3:.1f} us "
        f"(min {min(kern_ms)*1e3:.1f}), {gbs:.0f} GB/s, {tflops:.1f} TFLOP/s")

    out = {
        "metric": "KDA prefill tokens/s + MFMA util; decode tokens/s + HBM GB/s (1 MI355X)",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.qkv_dtype,
        "data": "synthetic (seeded; shapes and distributions of the pages' workloads)",
        "config": {"workload": w.name, "batch": w.B, "heads": w.H, "seq_len": w.L,
                   "d_k": w.dk, "d_v": w.dv, "chunk": CHUNK, "alpha": w.alpha_mode,
                   "gate_dtype": w.gate_dtype, "state_dtype": "f32"},
        "roofline": {"kernel": "kda_chunk_kernel", "bound": "hbm", "achieved": gbs,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                     "traffic": None, "algorithmic_bytes_per_launch": bytes_,
                     "avg_kernel_us": kavg * 1e3},
        "mfma": {"achieved": tflops, "peak": mfma_peak, "unit": "TFLOP/s",
                 "frac": tflops / mfma_peak, "algorithmic_flops_per_launch": flops},
    }
    if not args.no_decode:
        wd = gen.WORKLOADS[5]
        dwall, dk_ms = bench_decode(torch, kda, gen, wd)
        davg = float(np.mean(dk_ms))
        dbytes = decode_bytes(wd)
        dgbs = dbytes / (davg * 1e-3) / 1e9
        log(f"decode: {dwall*1e3/wd.decode_steps:.4f} ms/step wall, kernel avg "
            f"{davg*1e3:.1f} us, {dgbs:.0f} GB/s")
        out["decode"] = {
            "workload": wd.name, "tokens_per_s": wd.B * wd.decode_steps / dwall,
            "unit": "tokens/s", "ms_per_step": dwall * 1e3 / wd.decode_steps,
            "steps": wd.decode_steps,
            "roofline": {"kernel": "kda_decode_kernel", "bound": "hbm", "achieved": dgbs,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": dgbs / HBM_PEAK_GBS,
                         "traffic": None, "algorithmic_bytes_per_launch": dbytes,
                         "avg_kernel_us": davg * 1e3},
        }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(gen, w, x)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
