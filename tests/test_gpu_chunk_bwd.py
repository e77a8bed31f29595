"""Parity of kda_chunk_bwd (chunkwise gradients, HIP through the C ABI) with
oracle.backward (fp64 CPU reverse sweep of the token recurrence, pinned in
test_oracle_backward.py by finite differences and automatic differentiation).

Both sides see the same stored input values.  The chunkwise path computes
with bf16 operands on the matrix cores and fp32 accumulation (the arithmetic
of the bf16 chunked prefill), so its bar is the bf16 prefill's: per (b, h)
slab, max|x - ref| / max|ref| <= 2e-2 for every gradient.
"""

import numpy as np
import pytest

from linear_attention_sequence_kda_amd import inputs as gen

from gpu_util import device_inputs, say, to_dev, to_f64
from test_gpu_bwd import NAMES, reference, upstream

pytestmark = pytest.mark.gpu

TOL = 2e-2


def _kda():
    import linear_attention_sequence_kda_amd as kda
    return kda


def run_chunk(w, x, do, dSf, want_dS0=True):
    import torch
    kda = _kda()
    d = device_inputs(w, x)
    ddo = to_dev(do, w.qkv_dtype)
    ddSf = None if dSf is None else to_dev(dSf, gen.F32)
    got = kda.chunk_bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"], ddo, ddSf,
                        want_dS0=want_dS0)
    torch.cuda.synchronize()
    return [None if g is None else to_f64(g) for g in got]


def compare(w, x, do, dSf, got, heads, label, want_dS0=True, tol=TOL):
    refs = reference(w, x, do, dSf, heads)
    worst = {}
    for (b, h), ref in zip(heads, refs):
        for name, g, r in zip(NAMES, got, ref):
            if name == "dS0" and not want_dS0:
                assert g is None
                continue
            if r is None:
                assert g is None, name
                continue
            gh = g[b, h]
            assert np.all(np.isfinite(gh)), name
            scale = np.abs(r).max()
            err = np.abs(gh - r).max() / scale if scale > 0 else np.abs(gh).max()
            worst[name] = max(worst.get(name, 0.0), err)
    say(f"{label}: " + " ".join(f"{n}={e:.2e}" for n, e in worst.items()) + f" (tol {tol})")
    for name, e in worst.items():
        assert e <= tol, f"{name} error {e}"
    return worst


def run_and_compare(w, label, final=True, want_dS0=True, heads=None, seed=7):
    x = gen.prefill_inputs(w)
    do, dSf = upstream(w, seed, final)
    say(f"{label}: chunk_bwd B={w.B} H={w.H} L={w.L} dk={w.dk} dv={w.dv} "
        f"{w.qkv_dtype}/{w.gate_dtype}/{w.alpha_mode} S0={x['S0'] is not None} "
        f"dS_final={final} seed={w.seed}")
    got = run_chunk(w, x, do, dSf, want_dS0)
    heads = heads or [(b, h) for b in range(w.B) for h in range(w.H)]
    return compare(w, x, do, dSf, got, heads, label, want_dS0)


GATES = [("f32", "none"), ("f32", "head"), ("bf16", "head"), ("f32", "channel"),
         ("bf16", "channel")]
DIMS = [(128, 128), (64, 64), (128, 64), (64, 128)]


@pytest.mark.parametrize("gd,mode", GATES, ids=lambda x: str(x))
@pytest.mark.parametrize("dk,dv", DIMS, ids=lambda x: str(x))
@pytest.mark.parametrize("L", [1, 64, 70, 200])
def test_small_shapes(gd, mode, dk, dv, L):
    """Every decay mode and gate dtype, every head size, one chunk, a ragged
    tail and several chunks."""
    w = gen.custom(B=2, H=2, L=L, dk=dk, dv=dv, qkv_dtype="bf16", gate_dtype=gd,
                   alpha_mode=mode, seed=5000 + L + dk + 3 * dv)
    run_and_compare(w, "chunk-bwd-small")


@pytest.mark.parametrize("s0,final,want", [(False, True, True), (True, False, True),
                                           (False, False, True), (True, True, False)])
def test_optional_states(s0, final, want):
    w = gen.custom(B=1, H=3, L=137, dk=128, dv=128, qkv_dtype="bf16", gate_dtype="bf16",
                   alpha_mode="channel", s0_std=0.02 if s0 else None, seed=43)
    run_and_compare(w, "chunk-bwd-optional", final=final, want_dS0=want)


@pytest.mark.parametrize("mu,sigma", [(1.2, 0.3), (3.0, 0.3), (1.5, 1.0)])
def test_strong_decay(mu, sigma):
    """Per-channel decay of any strength: the decayed sums are split through
    anchor tokens so that no factor exceeds 1."""
    w = gen.custom(B=1, H=3, L=200, dk=128, dv=128, qkv_dtype="bf16", gate_dtype="f32",
                   alpha_mode="channel", seed=61 + int(10 * mu), la_mu=mu, la_sigma=sigma)
    run_and_compare(w, f"chunk-bwd strong decay mu={mu} sigma={sigma}")


def test_decay_wipes_and_mixed_blocks():
    w = gen.custom(B=1, H=3, L=300, dk=128, dv=128, qkv_dtype="bf16", gate_dtype="f32",
                   alpha_mode="channel", seed=78)
    x = gen.prefill_inputs(w)
    la = x["log_alpha"].copy()
    rng = np.random.default_rng(6)
    t = rng.integers(0, w.L, size=40)
    c = rng.integers(0, w.dk, size=40)
    la[0, 0, t, c] = -1000.0
    la[0, 1, 64:80, 7] = -12.0
    la[0, 2, :, :5] = -30.0
    x["log_alpha"] = la.astype(np.float32)
    do, dSf = upstream(w, 9, True)
    say("chunk-bwd wipes and mixed blocks: B=1 H=3 L=300")
    got = run_chunk(w, x, do, dSf)
    compare(w, x, do, dSf, got, [(0, 0), (0, 1), (0, 2)], "chunk-bwd wipes")


def test_agrees_with_token_kernel():
    """The two GPU implementations of the gradient on one problem: the
    token-by-token sweep (fp32) and the chunkwise form (bf16 operands)."""
    import torch
    kda = _kda()
    w = gen.custom(B=2, H=4, L=1000, dk=128, dv=128, qkv_dtype="bf16", gate_dtype="bf16",
                   alpha_mode="channel", seed=99)
    x = gen.prefill_inputs(w)
    do, dSf = upstream(w, 11, True)
    say("chunk-bwd vs recurrence_bwd: B=2 H=4 L=1000")
    got = run_chunk(w, x, do, dSf)
    d = device_inputs(w, x)
    tok = kda.recurrence_bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"],
                             to_dev(do, w.qkv_dtype), to_dev(dSf, gen.F32))
    torch.cuda.synchronize()
    tok = [to_f64(t) for t in tok]
    N = w.B * w.H
    for name, a, b in zip(NAMES, got, tok):
        a = a.reshape(N, -1)
        b = b.reshape(N, -1)
        err = (np.abs(a - b).max(axis=1) / np.abs(b).max(axis=1)).max()
        say(f"  {name}: {err:.2e}")
        assert err <= TOL, name


def test_deterministic():
    """No atomics across workgroups: two calls give the same bits."""
    w = gen.custom(B=1, H=4, L=333, dk=128, dv=128, qkv_dtype="bf16", gate_dtype="f32",
                   alpha_mode="channel", seed=12)
    x = gen.prefill_inputs(w)
    do, dSf = upstream(w, 3, True)
    say("chunk-bwd deterministic: B=1 H=4 L=333")
    a = run_chunk(w, x, do, dSf)
    b = run_chunk(w, x, do, dSf)
    for name, u, v in zip(NAMES, a, b):
        assert np.array_equal(u, v), name


def test_empty_sequence_passes_final_gradient_through():
    import torch
    kda = _kda()
    w = gen.custom(B=1, H=2, L=0, dk=128, dv=128, qkv_dtype="bf16", gate_dtype="f32",
                   alpha_mode="channel", seed=1)
    x = gen.prefill_inputs(w)
    d = device_inputs(w, x)
    dSf = np.random.default_rng(2).normal(size=(1, 2, 128, 128)).astype(np.float32)
    say("chunk-bwd L=0")
    ddo = torch.empty((1, 2, 0, 128), dtype=torch.bfloat16, device="cuda:0")
    got = kda.chunk_bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"], ddo,
                        to_dev(dSf, gen.F32))
    torch.cuda.synchronize()
    assert np.array_equal(to_f64(got[5]), dSf.astype(np.float64))
    assert all(g.numel() == 0 for g in got[:5])


@pytest.mark.parametrize("cfg", [2, 3])
def test_workload_full(cfg):
    """The full-size training workloads in one call, as bench.py times them;
    two heads against the oracle."""
    w = gen.WORKLOADS[cfg]
    heads = [(0, 0), (w.B - 1, w.H - 1)]
    run_and_compare(w, f"chunk-bwd workload {cfg}", heads=heads)


def _sweep_cases(n=12, seed=20261204):
    """Seeded random shapes for the gradients: ragged lengths, head counts,
    every head size, gate dtype and decay mode, decay strengths from almost
    none to strong, with and without an initial state and a final-state
    gradient."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        gd, mode = GATES[rng.integers(len(GATES))]
        dk, dv = DIMS[rng.integers(len(DIMS))]
        B = int(rng.integers(1, 3))
        H = int(rng.integers(1, 9))
        L = int(rng.integers(1, min(700, 8000 // (B * H)) + 1))
        mu = float(rng.uniform(-6.0, -0.05))
        s0 = [None, 0.02, 0.5][int(rng.integers(3))]
        final = bool(rng.integers(2))
        cases.append((i, B, H, L, dk, dv, gd, mode, mu, s0, final))
    return cases


@pytest.mark.parametrize("case", _sweep_cases(), ids=lambda c: f"sweep{c[0]}")
def test_random_shape_sweep(case):
    i, B, H, L, dk, dv, gd, mode, mu, s0, final = case
    w = gen.custom(B=B, H=H, L=L, dk=dk, dv=dv, qkv_dtype="bf16", gate_dtype=gd,
                   alpha_mode=mode, la_mu=mu, la_sigma=0.5, s0_std=s0, seed=6000 + i)
    run_and_compare(w, f"chunk-bwd-sweep{i} mu={mu:.2f} s0={s0}", final=final, seed=70 + i)
