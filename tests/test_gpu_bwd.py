"""Parity of kda_recurrence_bwd (HIP, through the C ABI) with oracle.backward
(fp64 CPU reverse sweep, itself pinned by finite differences and automatic
differentiation in test_oracle_backward.py).

Both sides see the same stored input values (bf16 inputs widened exactly), so
the difference is fp32 rounding in the kernel.  Metric: per (b, h) slab,
max|x - ref| / max|ref| for each gradient, worst slab.  Bar: 1e-4.
"""

import numpy as np
import pytest

import oracle
from linear_attention_sequence_kda_amd import inputs as gen

from gpu_util import device_inputs, say, to_dev, to_f64

pytestmark = pytest.mark.gpu

TOL = 1e-4
NAMES = ["dq", "dk", "dv", "dlog_alpha", "dbeta", "dS0"]


def _kda():
    import linear_attention_sequence_kda_amd as kda
    return kda


def upstream(w: gen.Workload, seed: int, final: bool):
    """Seeded upstream gradients: do in the qkv storage type, dS_final fp32."""
    rng = np.random.default_rng(seed)
    do = gen.to_storage(rng.normal(size=(w.B, w.H, w.L, w.dv)), w.qkv_dtype)
    dSf = rng.normal(size=(w.B, w.H, w.dk, w.dv)).astype(np.float32) if final else None
    return do, dSf


def reference(w, x, do, dSf, heads):
    """oracle.backward per listed (b, h) on the widened stored values."""
    out = []
    for b, h in heads:
        la = gen.widen(x["log_alpha"][b, h], w.gate_dtype) if x["log_alpha"] is not None else None
        s0 = None if x["S0"] is None else np.asarray(x["S0"][b, h], dtype=np.float64)
        out.append(oracle.backward(gen.widen(x["q"][b, h], w.qkv_dtype),
                                   gen.widen(x["k"][b, h], w.qkv_dtype),
                                   gen.widen(x["v"][b, h], w.qkv_dtype), la,
                                   gen.widen(x["beta"][b, h], w.gate_dtype), s0,
                                   gen.widen(do[b, h], w.qkv_dtype),
                                   None if dSf is None else dSf[b, h].astype(np.float64)))
    return out


def run_and_compare(w: gen.Workload, label: str, final=True, want_dS0=True, heads=None,
                    seed=7):
    import torch
    kda = _kda()
    x = gen.prefill_inputs(w)
    do, dSf = upstream(w, seed, final)
    d = device_inputs(w, x)
    ddo = to_dev(do, w.qkv_dtype)
    ddSf = None if dSf is None else to_dev(dSf, gen.F32)
    say(f"{label}: recurrence_bwd B={w.B} H={w.H} L={w.L} dk={w.dk} dv={w.dv} "
        f"{w.qkv_dtype}/{w.gate_dtype}/{w.alpha_mode} S0={x['S0'] is not None} "
        f"dS_final={final} seed={w.seed}")
    got = kda.recurrence_bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"], ddo,
                             ddSf, want_dS0=want_dS0)
    torch.cuda.synchronize()
    got = [None if g is None else to_f64(g) for g in got]
    heads = heads or [(b, h) for b in range(w.B) for h in range(w.H)]
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
            scale = np.abs(r).max()
            err = np.abs(gh - r).max() / scale if scale > 0 else np.abs(gh).max()
            worst[name] = max(worst.get(name, 0.0), err)
    say(f"{label}: " + " ".join(f"{n}={e:.2e}" for n, e in worst.items()) + f" (tol {TOL})")
    for name, e in worst.items():
        assert e <= TOL, f"{name} error {e}"
    return got


DTYPES = [("f32", "f32", "none"), ("f32", "f32", "head"), ("f32", "f32", "channel"),
          ("bf16", "f32", "head"), ("bf16", "bf16", "channel"), ("bf16", "bf16", "none"),
          ("f32", "bf16", "channel")]
DIMS = [(64, 64), (128, 128), (128, 64), (64, 128)]


@pytest.mark.parametrize("qd,gd,mode", DTYPES, ids=lambda x: str(x))
@pytest.mark.parametrize("dk,dv", DIMS, ids=lambda x: str(x))
@pytest.mark.parametrize("L", [1, 13, 70])
def test_small_shapes(qd, gd, mode, dk, dv, L):
    w = gen.custom(B=2, H=2, L=L, dk=dk, dv=dv, qkv_dtype=qd, gate_dtype=gd, alpha_mode=mode,
                   seed=3000 + L + dk + dv)
    run_and_compare(w, "bwd-small")


@pytest.mark.parametrize("s0,final,want", [(False, True, True), (True, False, True),
                                           (False, False, True), (True, True, False)])
def test_optional_states(s0, final, want):
    w = gen.custom(B=1, H=3, L=37, dk=128, dv=128, qkv_dtype="bf16", gate_dtype="bf16",
                   alpha_mode="channel", s0_std=0.02 if s0 else None, seed=41)
    run_and_compare(w, "bwd-optional", final=final, want_dS0=want)


@pytest.mark.parametrize("L", [7, 8, 9, 64, 1003])
def test_checkpoint_boundaries(L):
    w = gen.custom(B=1, H=2, L=L, dk=128, dv=128, qkv_dtype="bf16", gate_dtype="f32",
                   alpha_mode="head", seed=L)
    run_and_compare(w, "bwd-boundary")


def test_empty_sequence_passes_final_gradient_through():
    import torch
    kda = _kda()
    w = gen.custom(B=2, H=2, L=0, dk=64, dv=64, qkv_dtype="f32", gate_dtype="f32",
                   alpha_mode="channel", seed=5)
    x = gen.prefill_inputs(w)
    d = device_inputs(w, x)
    rng = np.random.default_rng(3)
    dSf = rng.normal(size=(2, 2, 64, 64)).astype(np.float32)
    ddo = torch.empty((2, 2, 0, 64), dtype=torch.float32, device="cuda:0")
    say("bwd-empty: L=0")
    got = kda.recurrence_bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"], ddo,
                             to_dev(dSf, gen.F32))
    torch.cuda.synchronize()
    assert np.array_equal(to_f64(got[5]), dSf.astype(np.float64))
    assert all(g.numel() == 0 for g in got[:5])


def test_repeatable_outputs():
    """dv and dS0 have one writer per element: bitwise equal across runs; the
    atomically summed gradients agree within the bar."""
    import torch
    kda = _kda()
    w = gen.custom(B=1, H=4, L=300, dk=128, dv=128, qkv_dtype="bf16", gate_dtype="bf16",
                   alpha_mode="channel", seed=77)
    x = gen.prefill_inputs(w)
    do, dSf = upstream(w, 9, True)
    d = device_inputs(w, x)
    args = (d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"],
            to_dev(do, w.qkv_dtype), to_dev(dSf, gen.F32))
    say("bwd-repeat: two calls")
    a = kda.recurrence_bwd(*args)
    b = kda.recurrence_bwd(*args)
    torch.cuda.synchronize()
    assert torch.equal(a[2], b[2]) and torch.equal(a[5], b[5])
    for i in (0, 1, 3, 4):
        ref = to_f64(a[i])
        assert np.abs(to_f64(b[i]) - ref).max() <= 1e-5 * np.abs(ref).max()


@pytest.mark.parametrize("cfg", [2, 3])
def test_workload_full_sampled_heads(cfg):
    """The full-size prefill workloads (4 x 16 x 4096 Gated DeltaNet, 2 x 32 x
    8192 KDA) in the launch the benchmark times; the oracle checks two heads."""
    w = gen.WORKLOADS[cfg]
    run_and_compare(w, f"bwd-workload{cfg}", heads=[(0, 0), (w.B - 1, w.H - 1)])


# ---- raw inputs (kda_recurrence_bwd_ex) ---------------------------------------

ALL = oracle.NORM_QK | oracle.BETA_LOGIT | oracle.GATE_RAW


def _mixed(w, flags):
    """The raw draw where a flag asks for it, the preprocessed draw elsewhere."""
    x, r = gen.prefill_inputs(w), gen.prefill_inputs(w, raw=True)
    out = dict(x)
    if flags & oracle.NORM_QK:
        out["q"], out["k"] = r["q"], r["k"]
    if flags & oracle.BETA_LOGIT:
        out["beta"] = r["beta"]
    if flags & oracle.GATE_RAW and w.alpha_mode != gen.ALPHA_NONE:
        out["log_alpha"] = r["log_alpha"]
    return out


@pytest.mark.parametrize("flags", [ALL, oracle.NORM_QK, oracle.BETA_LOGIT | oracle.GATE_RAW])
@pytest.mark.parametrize("qd,gd,mode", [("bf16", "bf16", "channel"), ("f32", "f32", "head"),
                                        ("bf16", "f32", "none")])
@pytest.mark.parametrize("dk,dv", [(128, 64), (64, 128)])
def test_raw_inputs_against_oracle(flags, qd, gd, mode, dk, dv):
    import torch
    kda = _kda()
    w = gen.custom(B=2, H=2, L=77, dk=dk, dv=dv, qkv_dtype=qd, gate_dtype=gd, alpha_mode=mode,
                   seed=500 + flags + dk)
    x = _mixed(w, flags)
    do, dSf = upstream(w, 17, True)
    d = device_inputs(w, x)
    say(f"bwd-raw: recurrence_bwd_ex flags={flags} {qd}/{gd}/{mode} L={w.L}")
    got = kda.recurrence_bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"],
                             to_dev(do, w.qkv_dtype), to_dev(dSf, gen.F32), flags=flags)
    torch.cuda.synchronize()
    got = [None if g is None else to_f64(g) for g in got]
    worst = {}
    for b in range(w.B):
        for h in range(w.H):
            la = None if x["log_alpha"] is None else gen.widen(x["log_alpha"][b, h], w.gate_dtype)
            ref = oracle.backward_raw(gen.widen(x["q"][b, h], w.qkv_dtype),
                                      gen.widen(x["k"][b, h], w.qkv_dtype),
                                      gen.widen(x["v"][b, h], w.qkv_dtype), la,
                                      gen.widen(x["beta"][b, h], w.gate_dtype),
                                      np.asarray(x["S0"][b, h], dtype=np.float64),
                                      gen.widen(do[b, h], w.qkv_dtype),
                                      dSf[b, h].astype(np.float64), flags)
            for name, g, r in zip(NAMES, got, ref):
                if r is None:
                    assert g is None, name
                    continue
                err = np.abs(g[b, h] - r).max() / np.abs(r).max()
                worst[name] = max(worst.get(name, 0.0), err)
    say("bwd-raw: " + " ".join(f"{n}={e:.2e}" for n, e in worst.items()))
    for name, e in worst.items():
        assert e <= TOL, f"{name} error {e}"
