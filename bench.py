"""Benchmark of the KDA / gated delta rule hot path on one MI355X.

Prints ONE JSON line.  Headline: chunkwise KDA prefill (kda_chunk_fwd,
per-channel decay) on the long-context workload B=1, H=16, L=524288,
d_k=d_v=128, all inputs bf16, fp32 state, S_final returned; one step = one
kda_chunk_fwd over that batch.  Further legs in the same line: the Gated
DeltaNet workload (4 x 16 heads x 4096, scalar decay), the KDA workload
(2 x 32 heads x 8192), the KDA decode workload (256 sequences x 32 heads, fp32
state updated in place for 64 steps), gradients (token by token, and in
chunkwise form on the Gated DeltaNet and KDA workloads), raw inputs with fused
preprocessing, and normalized linear attention.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload N]

Inputs are seeded synthetic data (linear_attention_sequence_kda_amd.inputs),
resident in HBM before the timed region.  The CPU baseline is the fp64 oracle
(oracle/, C, all host cores of this job) timed on the headline workload.

Timing: the headline value is K back-to-back calls between two device
synchronizations (wall clock).  Every prefill leg is also timed call by call
with HIP events after a 1 GiB write has flushed the 256 MiB memory-side cache
(outside the events), which is the figure its `tokens_per_s` reports.

`roofline` covers the kernel with the most time per step, timed with the
library's HIP event pairs (kda_timing_*) on the call's stream, over K more
steps: achieved = the path's compulsory bytes per token-head (every input read
once, o and the states written once) x the token-heads one launch of that
kernel covers / its mean launch time.  `path` covers the whole call (every
launch) against HBM and against bf16 MFMA.  `traffic` is the kernel's measured
HBM bytes per launch from profiles/traffic.json (rocprofv3 FETCH_SIZE and
WRITE_SIZE passes scaled by a copy of known size), or null when there is no
measurement for the current sources.
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


def tensor_bytes(w):
    """Bytes of each compulsory tensor of one kda_chunk_fwd (touched once)."""
    tok = w.B * w.H * w.L
    eq, eg = esize(w.qkv_dtype), esize(w.gate_dtype)
    st = w.B * w.H * w.dk * w.dv * 4
    la = {"channel": tok * w.dk * eg, "head": tok * eg}.get(w.alpha_mode, 0)
    return {"q": tok * w.dk * eq, "k": tok * w.dk * eq, "v": tok * w.dv * eq,
            "o": tok * w.dv * eq, "log_alpha": la, "beta": tok * eg,
            "S0": st if w.s0_std is not None else 0, "S_final": st}


def prefill_bytes(w):
    """Compulsory HBM bytes of one kda_chunk_fwd: every input read once, o and
    S_final written once."""
    return sum(tensor_bytes(w).values())


def prefill_flops(w):
    """Algorithmic flops of the path: 6 dk dv + 2C(3 dk + 2 dv) per token-head
    (C = 64): state products Q S, W S, K^T u (2 dk dv each) and the full CxC
    chunk blocks A, P, T K, T V and P u ("2Ld^2 + 2LCd" counted the same way)."""
    per = 6 * w.dk * w.dv + 2 * CHUNK * (3 * w.dk + 2 * w.dv)
    return w.B * w.H * w.L * per


def kernel_work(w, kernel):
    """(compulsory bytes, algorithmic flops) one whole kda_chunk_fwd hands to
    `kernel`: the compulsory tensors it reads or writes (intermediate records
    in the workspace are not counted) and the products it computes."""
    t = tensor_bytes(w)
    tok = w.B * w.H * w.L
    dk, dv, C = w.dk, w.dv, CHUNK
    if kernel == "kda_intra_kernel":
        if w.alpha_mode == "channel":      # A, P, W = T K, U = T V from q, k, v, gates
            return (t["q"] + t["k"] + t["v"] + t["log_alpha"] + t["beta"],
                    tok * 2 * C * (3 * dk + dv))
        return t["k"] + t["log_alpha"] + t["beta"], tok * 2 * C * dk   # A only
    if kernel in ("kda_inter_kernel", "kda_inter_wide_kernel", "kda_inter_quad_kernel"):  # u = U - W S, o = Q S + P u, S update
        return t["o"] + t["S0"] + t["S_final"], tok * (6 * dk * dv + 2 * C * dv)
    if kernel == "kda_inter_scalar_kernel":  # X, u = T X, P, o, S update
        return (t["q"] + t["k"] + t["v"] + t["o"] + t["S0"] + t["S_final"],
                tok * (6 * dk * dv + 2 * C * dk + 4 * C * dv))
    raise KeyError(kernel)


def decode_bytes(w):
    """Compulsory HBM bytes of one decode step: state read + write, inputs, o."""
    bh = w.B * w.H
    eq, eg = esize(w.qkv_dtype), esize(w.gate_dtype)
    b = bh * w.dk * w.dv * 4 * 2
    b += bh * (2 * w.dk + w.dv) * eq + bh * w.dv * eq
    b += bh * (w.dk if w.alpha_mode == "channel" else 1) * eg + bh * eg
    return b


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter passes, or None
    when there are none for this kernel and workload or the kernel's sources
    have changed since they were taken."""
    from linear_attention_sequence_kda_amd import profiling
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh).get(f"{kernel}|{workload}")
    if not rec or rec.get("source_sha256") != profiling.source_digest(kernel):
        return None
    return rec["bytes"]


def to_dev(torch, arr, dt):
    if arr is None:
        return None
    if dt == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(
            torch.bfloat16).to("cuda:0")
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to("cuda:0")


def kernel_times(torch, kda, steps, step_fn):
    """Run step_fn `steps` times with the library's HIP event pairs on; return
    {kernel: (launches per step, mean ms per launch)} for every kernel that
    ran."""
    kda.timing_reset()
    kda.timing_enable(True)
    try:
        for _ in range(steps):
            step_fn()
        torch.cuda.synchronize()
    finally:
        kda.timing_enable(False)
    out = {}
    for name in kda.binding.KERNELS:
        n, ms = kda.timing_read(name)
        if n:
            out[name] = (n / steps, ms / n)
    kda.timing_reset()
    return out


def bench_prefill(torch, kda, gen, w, steps, warmup):
    log(f"prefill workload {w.name}: drawing inputs")
    x = gen.prefill_inputs(w, threads=16)
    d = {n: to_dev(torch, x[n], w.qkv_dtype if n in ("q", "k", "v") else w.gate_dtype)
         for n in ("q", "k", "v", "log_alpha", "beta")}
    S0 = to_dev(torch, x["S0"], "f32") if x["S0"] is not None else None
    o = torch.empty((w.B, w.H, w.L, w.dv), dtype=d["v"].dtype, device="cuda:0")
    Sf = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device="cuda:0")
    wsb = kda.chunk_fwd_workspace_bytes(d["q"], d["v"], d["log_alpha"], d["beta"])
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda:0")
    args = (d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], S0)
    call = lambda: kda.chunk_fwd(*args, o=o, S_final=Sf, workspace=ws)
    for _ in range(warmup):
        call()
    # K back-to-back calls between two synchronizations
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # the same K calls one by one, each after a 1 GiB write has flushed the
    # 256 MiB memory-side cache (as when other layers run between two calls);
    # the flush is outside the events
    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda:0")
    call_ms = []
    for _ in range(steps):
        flush.fill_(1.0)
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        call()
        e.record()
        torch.cuda.synchronize()
        call_ms.append(s.elapsed_time(e))
    del flush
    # per-kernel durations: the same steps again with the library's event
    # pairs around every launch (kept out of the regions above, whose clock
    # they would slow by a few microseconds per launch)
    kern = kernel_times(torch, kda, steps, call)
    return x, wall, call_ms, kern, wsb, (o, Sf)


def summarize_prefill(w, wall, call_ms, kern, steps):
    """tokens/s of one prefill workload, each kernel's figures, the kernel with
    the most time per step against HBM, and the whole call against both roofs.
    Call figures are the cache-flushed per-call times."""
    cavg = float(np.mean(call_ms))
    bytes_ = prefill_bytes(w)
    flops = prefill_flops(w)
    th = w.B * w.H * w.L
    gbs = bytes_ / (cavg * 1e-3) / 1e9
    tflops = flops / (cavg * 1e-3) / 1e12
    mfma_peak = BF16_MFMA_PEAK_TFLOPS if w.qkv_dtype == "bf16" else FP32_MFMA_PEAK_TFLOPS
    log(f"prefill {w.name}: {wall * 1e3 / steps:.4f} ms/step back-to-back, flushed call avg "
        f"{cavg*1e3:.1f} us (min {min(call_ms)*1e3:.1f}), {gbs:.0f} GB/s, {tflops:.1f} TFLOP/s")
    kernels = {}
    for name, (per_step, ms) in kern.items():
        kb, kf = kernel_work(w, name)
        kb, kf = kb / per_step, kf / per_step     # per launch
        kernels[name] = {"launches_per_step": per_step, "avg_us": ms * 1e3,
                         "algorithmic_bytes_per_launch": kb,
                         "algorithmic_flops_per_launch": kf,
                         "GB/s": kb / (ms * 1e-3) / 1e9, "TFLOP/s": kf / (ms * 1e-3) / 1e12}
        log(f"  {name}: {per_step:g} launch(es)/step, {ms*1e3:.1f} us avg, "
            f"{kernels[name]['GB/s']:.0f} GB/s, {kernels[name]['TFLOP/s']:.1f} TFLOP/s")
    # the dominant kernel: most time per step
    dom = max(kernels, key=lambda n: kernels[n]["avg_us"] * kernels[n]["launches_per_step"])
    kd = kernels[dom]
    path = {"avg_call_us": cavg * 1e3, "min_call_us": min(call_ms) * 1e3,
            "back_to_back_call_us": wall * 1e6 / steps,
            "hbm": {"achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": gbs / HBM_PEAK_GBS, "compulsory_bytes_per_call": bytes_,
                    "bytes_per_token_head": bytes_ / th},
            "mfma": {"achieved": tflops, "peak": mfma_peak, "unit": "TFLOP/s",
                     "frac": tflops / mfma_peak, "algorithmic_flops_per_call": flops,
                     "flops_per_token_head": flops / th}}
    # dominant kernel: the path's compulsory bytes per token-head times the
    # token-heads one launch covers, over its mean launch time (HIP events on
    # the call's stream); the prefill's arithmetic intensity is left of the
    # MI355X ridge, so HBM binds
    per_launch = bytes_ / kd["launches_per_step"]
    achieved = per_launch / (kd["avg_us"] * 1e-6) / 1e9
    roof = {"kernel": dom, "bound": "hbm", "achieved": achieved,
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
            "traffic": measured_traffic(dom, w.name),
            "algorithmic_bytes_per_launch": per_launch,
            "token_heads_per_launch": th / kd["launches_per_step"],
            "avg_kernel_us": kd["avg_us"]}
    return {"tokens_per_s": w.B * w.L / (cavg * 1e-3), "ms_per_step": cavg,
            "back_to_back_tokens_per_s": w.B * w.L / (wall / steps),
            "roofline": roof, "kernels": kernels, "path": path}


def bench_prefill_leg(torch, kda, gen, w, steps, warmup):
    """A further prefill workload in the same line (same timing as the headline)."""
    x, wall, call_ms, kern, wsb, _ = bench_prefill(torch, kda, gen, w, steps, warmup)
    del x
    out = {"workload": w.name, "unit": "tokens/s",
           "config": {"batch": w.B, "heads": w.H, "seq_len": w.L, "d_k": w.dk, "d_v": w.dv,
                      "chunk": CHUNK, "alpha": w.alpha_mode, "qkv_dtype": w.qkv_dtype,
                      "gate_dtype": w.gate_dtype, "state_dtype": "f32",
                      "S0": w.s0_std is not None, "workspace_bytes": wsb}}
    out.update(summarize_prefill(w, wall, call_ms, kern, steps))
    torch.cuda.empty_cache()
    return out


def bwd_flops(w):
    """Algorithmic flops of one kda_recurrence_bwd: 20 dk dv per token-head.
    The forward step it has to redo (S~ = diag(alpha) S, k S~, S~ + k^T u:
    5 per state element) and the reverse step (G += q^T do, k G, dq = S do^T,
    dk = G u^T - S~ ge^T, gS~ = G - k^T ge, d ln alpha = sum gS~ S~,
    G = diag(alpha) gS~: 15 per element); the recomputation of states from
    checkpoints is the kernel's own cost and is not counted."""
    return w.B * w.H * w.L * 20 * w.dk * w.dv


def bench_bwd(torch, kda, gen, w, steps, warmup):
    """Gradients of the recurrence for one prefill workload (dJ/do given,
    dJ/dS_final zero): tokens/s, and the gradient kernel against the fp32
    vector ALU peak (the kernel is a chain of per-token vector updates)."""
    log(f"gradients, workload {w.name}: drawing inputs")
    x = gen.prefill_inputs(w, threads=16)
    d = {n: to_dev(torch, x[n], w.qkv_dtype if n in ("q", "k", "v") else w.gate_dtype)
         for n in ("q", "k", "v", "log_alpha", "beta")}
    S0 = to_dev(torch, x["S0"], "f32") if x["S0"] is not None else None
    del x
    rng = np.random.default_rng(w.seed + 101)
    do = to_dev(torch, gen.to_storage(rng.normal(size=(w.B, w.H, w.L, w.dv)), w.qkv_dtype),
                w.qkv_dtype)
    wsb = kda.recurrence_bwd_workspace_bytes(d["q"], d["v"], d["log_alpha"], d["beta"])
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda:0")

    def step():
        return kda.recurrence_bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], S0, do,
                                  None, want_dS0=S0 is not None, workspace=ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern = kernel_times(torch, kda, steps, step)
    per, ms = kern["kda_bwd_kernel"]
    flops = bwd_flops(w) / per
    tflops = flops / (ms * 1e-3) / 1e12
    log(f"gradients {w.name}: {wall * 1e3 / steps:.3f} ms/step wall, kernel avg {ms:.3f} ms, "
        f"{tflops:.2f} TFLOP/s")
    out = {"workload": w.name, "tokens_per_s": w.B * w.L / (wall / steps), "unit": "tokens/s",
           "ms_per_step": wall * 1e3 / steps, "workspace_bytes": wsb,
           "kernels": {n: {"launches_per_step": pk, "avg_us": m * 1e3} for n, (pk, m) in kern.items()},
           "roofline": {"kernel": "kda_bwd_kernel", "bound": "alu", "achieved": tflops,
                        "peak": FP32_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": tflops / FP32_MFMA_PEAK_TFLOPS,
                        "traffic": measured_traffic("kda_bwd_kernel", w.name),
                        "algorithmic_flops_per_launch": flops, "avg_kernel_us": ms * 1e3}}
    del d, do, ws
    torch.cuda.empty_cache()
    return out


def chunk_grad_flops(w):
    """Algorithmic matrix-core flops of one kda_chunk_grad_kernel launch:
    per chunk of C = 64 tokens and head, 2 x (C^2 dv for dY = T^T du, 3 C dk dv
    for dO S^T, dY S^T and u G^T, 2 C^2 dv for dY u^T and dO u^T, and 4
    triangular decayed sums of C^2/2 dk each)."""
    C = 64
    nc = -(-w.L // C)
    per = 2 * (C * C * w.dv + 3 * C * w.dk * w.dv + 2 * C * C * w.dv + 2 * C * C * w.dk)
    return w.B * w.H * nc * per


def chunk_grad_bytes(w):
    """Algorithmic HBM bytes of one kda_chunk_grad_kernel launch: per chunk
    of C = 64 tokens and head, every input read once (T^T fp32; du, u, dO, v,
    q, k bf16; S and G fp32; ln alpha per channel or per token, and beta, in
    the gate type; without a decay one column of widened fp32 zeros and an
    fp32 beta) and every gradient written once (fp32)."""
    C, dk, dv = 64, w.dk, w.dv
    nc = -(-w.L // C)
    g = 2 if w.gate_dtype == "bf16" else 4
    gates = {"channel": C * dk * g + C * g, "head": 2 * C * g}.get(w.alpha_mode, 2 * C * 4)
    reads = C * C * 4 + 4 * C * dv * 2 + 2 * C * dk * 2 + gates + 2 * dk * dv * 4
    dla = {"channel": C * dk * 4, "head": C * 4}.get(w.alpha_mode, 0)
    writes = 2 * C * dk * 4 + C * dv * 4 + dla + C * 4
    return w.B * w.H * nc * (reads + writes)


def bench_chunk_bwd(torch, kda, gen, w, steps, warmup):
    """Chunkwise gradients (kda_chunk_bwd) of one prefill workload (dJ/do
    given, dJ/dS_final zero): tokens/s, every kernel's time, and the
    chunk-parallel gradient kernel against HBM (its bound: the counters read
    3.6 TB/s on the 2 x 32 x 8192 workload) and against bf16 MFMA."""
    log(f"chunkwise gradients, workload {w.name}: drawing inputs")
    x = gen.prefill_inputs(w, threads=16)
    d = {n: to_dev(torch, x[n], w.qkv_dtype if n in ("q", "k", "v") else w.gate_dtype)
         for n in ("q", "k", "v", "log_alpha", "beta")}
    S0 = to_dev(torch, x["S0"], "f32") if x["S0"] is not None else None
    del x
    rng = np.random.default_rng(w.seed + 101)
    do = to_dev(torch, gen.to_storage(rng.normal(size=(w.B, w.H, w.L, w.dv)), w.qkv_dtype),
                w.qkv_dtype)
    wsb = kda.chunk_bwd_workspace_bytes(d["q"], d["v"], d["log_alpha"], d["beta"])
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda:0")

    def step():
        return kda.chunk_bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], S0, do, None,
                             want_dS0=S0 is not None, workspace=ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern = kernel_times(torch, kda, steps, step)
    per, ms = kern["kda_chunk_grad_kernel"]
    tflops = chunk_grad_flops(w) / per / (ms * 1e-3) / 1e12
    gbs = chunk_grad_bytes(w) / per / (ms * 1e-3) / 1e9
    log(f"chunkwise gradients {w.name}: {wall * 1e3 / steps:.3f} ms/step wall; "
        + ", ".join(f"{n} {pk:g} x {m * 1e3:.1f} us" for n, (pk, m) in kern.items()))
    out = {"workload": w.name, "tokens_per_s": w.B * w.L / (wall / steps), "unit": "tokens/s",
           "ms_per_step": wall * 1e3 / steps, "workspace_bytes": wsb,
           "kernels": {n: {"launches_per_step": pk, "avg_us": m * 1e3} for n, (pk, m) in kern.items()},
           "roofline": {"kernel": "kda_chunk_grad_kernel", "bound": "hbm", "achieved": gbs,
                        "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                        "traffic": measured_traffic("kda_chunk_grad_kernel", w.name),
                        "algorithmic_bytes_per_launch": chunk_grad_bytes(w) / per,
                        "avg_kernel_us": ms * 1e3,
                        "mfma": {"achieved": tflops, "peak": BF16_MFMA_PEAK_TFLOPS,
                                 "unit": "TFLOP/s", "frac": tflops / BF16_MFMA_PEAK_TFLOPS,
                                 "algorithmic_flops_per_launch": chunk_grad_flops(w) / per}}}
    del d, do, ws
    torch.cuda.empty_cache()
    return out


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
    t0 = time.perf_counter()
    for st in steps:
        kda.decode_step(*st, S, o=o)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # per-launch durations over the same 64 steps (state restored first)
    S.copy_(S0)
    it = iter(steps)
    kern = kernel_times(torch, kda, T, lambda: kda.decode_step(*next(it), S, o=o))
    return wall, kern


def bench_prefill_raw(torch, kda, gen, w, steps, warmup):
    """The same prefill on raw inputs (unnormalized q, k, beta logits, gate
    pre-activations) with the preprocessing fused into the kernels' loads."""
    log(f"prefill workload {w.name}, raw inputs: drawing inputs")
    x = gen.prefill_inputs(w, threads=16, raw=True)
    d = {n: to_dev(torch, x[n], w.qkv_dtype if n in ("q", "k", "v") else w.gate_dtype)
         for n in ("q", "k", "v", "log_alpha", "beta")}
    S0 = to_dev(torch, x["S0"], "f32") if x["S0"] is not None else None
    o = torch.empty((w.B, w.H, w.L, w.dv), dtype=d["v"].dtype, device="cuda:0")
    Sf = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device="cuda:0")
    wsb = kda.chunk_fwd_workspace_bytes(d["q"], d["v"], d["log_alpha"], d["beta"])
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda:0")
    flags = kda.NORM_QK | kda.BETA_LOGIT | kda.GATE_RAW
    call = lambda: kda.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], S0, o=o,
                                 S_final=Sf, workspace=ws, flags=flags)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern = kernel_times(torch, kda, steps, call)
    per = {k: {"launches_per_step": n, "avg_us": ms * 1e3} for k, (n, ms) in kern.items()}
    log(f"prefill, raw inputs + fused preprocessing: {wall * 1e3 / steps:.4f} ms/step wall; "
        + ", ".join(f"{k} {v['avg_us']:.1f} us" for k, v in per.items()))
    return {"flags": "NORM_QK | BETA_LOGIT | GATE_RAW", "tokens_per_s": w.B * w.L / (wall / steps),
            "unit": "tokens/s", "ms_per_step": wall * 1e3 / steps, "kernels": per}


def bench_linear_attention(torch, kda, gen, w, steps, warmup):
    """Normalized linear attention (phi = elu + 1) on the prefill workload's
    shape: raw q, k, v drawn with the same recipe, no decay or gates."""
    wl = gen.custom(B=w.B, H=w.H, L=w.L, dk=w.dk, dv=w.dv, qkv_dtype=w.qkv_dtype,
                    gate_dtype="f32", alpha_mode="none", s0_std=None, seed=w.seed)
    log(f"linear attention on {w.B}x{w.H}x{w.L} d={w.dk}: drawing inputs")
    x = gen.prefill_inputs(wl, threads=16, raw=True)
    d = [to_dev(torch, x[n], w.qkv_dtype) for n in ("q", "k", "v")]
    o = torch.empty((w.B, w.H, w.L, w.dv), dtype=d[2].dtype, device="cuda:0")
    Sf = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device="cuda:0")
    zf = torch.empty((w.B, w.H, w.dk), dtype=torch.float32, device="cuda:0")
    call = lambda: kda.linear_attn_fwd(*d, o=o, S_final=Sf, z_final=zf)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern = kernel_times(torch, kda, steps, call)
    _, ms = kern["kda_inter_scalar_kernel"]
    e = esize(w.qkv_dtype)
    th = w.B * w.H * w.L
    # q, k, v read, o written; S_final and z_final written
    bytes_ = th * e * (2 * w.dk + 2 * w.dv) + w.B * w.H * (w.dk * w.dv + w.dk) * 4
    C = 64 if w.qkv_dtype == "bf16" else 32
    # Q S, S update (2 dk dv each), P and P V (C dk, C dv), z (C dk): flops per token-head
    flops = th * (4 * w.dk * w.dv + 2 * C * (2 * w.dk + w.dv))
    gbs = bytes_ / (ms * 1e-3) / 1e9
    tflops = flops / (ms * 1e-3) / 1e12
    fper, fms = kern.get("kda_feature_map_kernel", (0, 0.0))
    fbytes = 2 * th * w.dk * e   # q read, phi(q) written
    log(f"linear attention: {wall * 1e3 / steps:.4f} ms/step wall, state pass avg {ms * 1e3:.1f} us, "
        f"{gbs:.0f} GB/s, {tflops:.1f} TFLOP/s; feature map avg {fms * 1e3:.1f} us, "
        f"{fbytes / max(fms * 1e-3, 1e-12) / 1e9:.0f} GB/s")
    return {"shape": f"b{w.B}_h{w.H}_l{w.L}_d{w.dk}_{w.qkv_dtype}",
            "tokens_per_s": th / w.H / (wall / steps), "unit": "tokens/s",
            "ms_per_step": wall * 1e3 / steps,
            "kernel": "kda_inter_scalar_kernel (linear attention instance)",
            "avg_kernel_us": ms * 1e3, "algorithmic_bytes_per_launch": bytes_,
            "algorithmic_flops_per_launch": flops,
            "hbm_frac": gbs / HBM_PEAK_GBS, "GB/s": gbs, "TFLOP/s": tflops,
            "feature_map": {"kernel": "kda_feature_map_kernel", "avg_us": fms * 1e3,
                            "algorithmic_bytes_per_launch": fbytes,
                            "GB/s": fbytes / max(fms * 1e-3, 1e-12) / 1e9}}


def cpu_baseline(gen, w, x, outs=None, min_seconds=10.0, max_passes=64):
    """The fp64 oracle (C, one worker per (head, 32-column block), all host
    cores of the job) on the workload the headline times.  Heads run a few at
    a time, so the fp64 outputs stay within a few GB of host memory; heads are
    taken in order until every head has run once and about min_seconds of
    compute have passed (whole passes over the workload are repeated while
    they take less).  Value: the token rate this gives for the whole batch."""
    import oracle
    N = w.B * w.H
    f = lambda a: None if a is None else a.reshape((N,) + a.shape[2:])
    xf = {k: f(v) for k, v in x.items()}
    threads = oracle.default_threads()
    group = max(1, min(N, threads // max(1, w.dv // 32)))
    log(f"cpu baseline: oracle on {w.name}, {threads} threads, {group} heads at a time")
    heads_done, dt, passes = 0, 0.0, 0
    check = None
    while passes < max_passes and (heads_done < N or dt < min_seconds):
        h0 = heads_done % N
        hs = slice(h0, min(N, h0 + group))
        sl = {k: (None if v is None else np.ascontiguousarray(v[hs])) for k, v in xf.items()}
        t0 = time.perf_counter()
        o_ref, s_ref = oracle.forward(sl["q"], sl["k"], sl["v"], sl["log_alpha"], sl["beta"],
                                      sl["S0"], qkv_dtype=w.qkv_dtype, gate_dtype=w.gate_dtype,
                                      alpha_mode=w.alpha_mode, want_o=True, threads=threads)
        dt += time.perf_counter() - t0
        if check is None and outs is not None:
            # the first heads of the timed call's own outputs against the oracle
            # (outside the oracle's clock)
            check = oracle_check(w, outs, hs, o_ref, s_ref)
        heads_done += hs.stop - hs.start
        passes = heads_done // N
    # heads_done x L token-heads in dt seconds; the batch's tokens/s is that
    # rate divided by the heads each token passes through
    value = heads_done * w.L / w.H / dt
    return {"value": value, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{w.name}: {heads_done} head runs of {w.L} tokens (all {w.dv} columns, "
                      f"o and S_final; the batch has {N} heads), {group} heads at a time, "
                      f"{dt:.2f} s of oracle compute"}, check


def oracle_check(w, outs, hs, o_ref, s_ref):
    """Worst per-head relative error max|x - ref| / max|ref| of the timed
    call's o and S_final on heads hs (flattened b*H + h) against the fp64
    oracle, with the parity tests' bar for the workload's dtype."""
    import oracle
    o, Sf = outs
    N = w.B * w.H
    o_h = o.reshape(N, w.L, w.dv)[hs].float().cpu().numpy()
    s_h = Sf.reshape(N, w.dk, w.dv)[hs].cpu().numpy()
    e_o = float(oracle.slab_error(o_h, o_ref, 1))
    e_s = float(oracle.slab_error(s_h, s_ref, 1))
    tol = 2e-2 if w.qkv_dtype == "bf16" else 1e-4
    log(f"oracle check on heads {hs.start}..{hs.stop - 1}: o {e_o:.2e}, S_final {e_s:.2e} (bar {tol})")
    return {"heads": [hs.start, hs.stop], "o": e_o, "S_final": e_s, "bar": tol,
            "metric": "max|x - ref| / max|ref| per head, worst head; fp64 oracle",
            "pass": bool(e_o <= tol and e_s <= tol)}


def run_env(torch, workloads):
    """What the line was measured on: device, HIP and torch versions, a digest
    of the library's sources and of this file, the input seeds."""
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    h = hashlib.sha256()
    csrc = os.path.join(root, "linear_attention_sequence_kda_amd", "csrc")
    files = [os.path.join(csrc, f) for f in sorted(os.listdir(csrc))]
    files += [os.path.join(root, "include", "kda.h"), os.path.abspath(__file__)]
    for f in files:
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode() + b"\0" + fh.read())
    props = torch.cuda.get_device_properties(0)
    return {"gpu": torch.cuda.get_device_name(0), "arch": getattr(props, "gcnArchName", None),
            "cus": props.multi_processor_count, "hip": torch.version.hip, "torch": torch.__version__,
            "sources_sha256": h.hexdigest()[:16],
            "seeds": {w.name: w.seed for w in workloads}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=4, help="headline prefill workload number (1-4)")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-linear-attention", action="store_true")
    ap.add_argument("--no-raw", action="store_true", help="skip the raw-input prefill leg")
    ap.add_argument("--no-kda", action="store_true",
                    help="skip the KDA (per-channel decay) prefill legs, workloads 3 and 4")
    ap.add_argument("--no-bwd", action="store_true",
                    help="skip the gradient (kda_recurrence_bwd) legs")
    ap.add_argument("--no-gdn-bwd", action="store_true",
                    help="skip the Gated DeltaNet gradient leg (keep the KDA one)")
    ap.add_argument("--no-chunk-bwd", action="store_true",
                    help="skip the chunkwise gradient (kda_chunk_bwd) legs")
    ap.add_argument("--no-prefill-legs", action="store_true",
                    help="skip the prefill legs other than the headline workload's")
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
    from linear_attention_sequence_kda_amd import binding  # noqa: F401  (kda.binding)
    from linear_attention_sequence_kda_amd import inputs as gen

    kda.library()  # fail loudly if the HIP library is missing
    if args.copy_calibration:
        src = torch.ones(64 << 20, dtype=torch.float32, device="cuda:0")  # 256 MiB
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    w = gen.WORKLOADS[args.workload]
    x, wall, call_ms, kern, wsb, outs = bench_prefill(torch, kda, gen, w, args.steps, args.warmup)
    head = summarize_prefill(w, wall, call_ms, kern, args.steps)
    # the headline: K back-to-back calls between two synchronizations
    ms_per_step = wall * 1e3 / args.steps
    value = w.B * w.L / (wall / args.steps)
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
                   "qkv_dtype": w.qkv_dtype, "gate_dtype": w.gate_dtype,
                   "state_dtype": "f32", "S0": w.s0_std is not None, "S_final": True,
                   "workspace_bytes": wsb},
        "roofline": head["roofline"],
        "kernels": head["kernels"],
        # the whole kda_chunk_fwd call (every launch), against both roofs;
        # flushed per-call figures
        "path": head["path"],
        "flushed_tokens_per_s": head["tokens_per_s"],
    }
    if not args.no_decode:
        wd = gen.WORKLOADS[5]
        dwall, dkern = bench_decode(torch, kda, gen, wd)
        dper, dms = dkern["kda_decode_kernel"]
        dbytes = decode_bytes(wd)
        dgbs = dbytes / (dms * 1e-3) / 1e9
        log(f"decode: {dwall*1e3/wd.decode_steps:.4f} ms/step wall, kernel avg "
            f"{dms*1e3:.1f} us, {dgbs:.0f} GB/s")
        out["decode"] = {
            "workload": wd.name, "tokens_per_s": wd.B * wd.decode_steps / dwall,
            "unit": "tokens/s", "ms_per_step": dwall * 1e3 / wd.decode_steps,
            "steps": wd.decode_steps,
            "roofline": {"kernel": "kda_decode_kernel", "bound": "hbm", "achieved": dgbs,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": dgbs / HBM_PEAK_GBS,
                         "traffic": measured_traffic("kda_decode_kernel", wd.name),
                         "algorithmic_bytes_per_launch": dbytes,
                         "avg_kernel_us": dms * 1e3},
        }
    # further prefill workloads: Gated DeltaNet (scalar decay, 4 x 16 x 4096)
    # and the other KDA ones (2 x 32 x 8192; 1 x 16 x 524288)
    legs = [("prefill_gated_deltanet", 2)]
    if not args.no_kda:
        legs += [("prefill_kda", 3), ("prefill_kda_long_context", 4)]
    if args.no_prefill_legs:
        legs = []
    for key, n in legs:
        if n != args.workload:
            out[key] = bench_prefill_leg(torch, kda, gen, gen.WORKLOADS[n], args.steps,
                                         args.warmup)
    # gradients, raw inputs and linear attention run on the Gated DeltaNet
    # workload's shape (the gradient kernel's checkpoints of the long-context
    # workload would not fit in HBM)
    w2 = gen.WORKLOADS[2]
    if not args.no_bwd:
        if not args.no_gdn_bwd:
            out["gradients"] = bench_bwd(torch, kda, gen, w2, min(args.steps, 10), min(args.warmup, 2))
        if not args.no_kda:
            # the KDA workload's gradients (per-channel decay, 2 x 32 x 8192)
            out["gradients_kda"] = bench_bwd(torch, kda, gen, gen.WORKLOADS[3],
                                             min(args.steps, 5), min(args.warmup, 1))
    if not args.no_chunk_bwd:
        # the same gradients in chunkwise form (bf16 operands on the matrix cores)
        out["gradients_chunk"] = bench_chunk_bwd(torch, kda, gen, w2, args.steps,
                                                 min(args.warmup, 2))
        if not args.no_kda:
            out["gradients_chunk_kda"] = bench_chunk_bwd(torch, kda, gen, gen.WORKLOADS[3],
                                                         args.steps, min(args.warmup, 2))
    if not args.no_raw:
        out["prefill_raw_inputs"] = bench_prefill_raw(torch, kda, gen, w2, args.steps, args.warmup)
    if not args.no_linear_attention:
        out["linear_attention"] = bench_linear_attention(torch, kda, gen, w2, args.steps,
                                                         args.warmup)
    if not args.no_cpu:
        out["cpu_baseline"], chk = cpu_baseline(gen, w, x, outs)
        if chk is not None:
            out["oracle_check"] = chk
    out["env"] = run_env(torch, [gen.WORKLOADS[n] for n in sorted({args.workload, 2, 3, 4, 5})])
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
