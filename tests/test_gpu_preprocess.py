"""Parity of the fused input preprocessing (kda_chunk_fwd_ex, kda_decode_step_ex,
kda_decode_step_slots_ex) with the fp64 oracle applied to the same raw inputs.

The kernels L2-normalize q and k, take beta = sigmoid(logit) and
ln alpha = -exp(g) as they load the raw values; the oracle widens the same
stored raw values to fp64, preprocesses them there and runs the recurrence.
Metric and bar as for the plain entry points: worst (b, h) slab of
max|x - ref| / max|ref|, 1e-4 for fp32 inputs, 2e-2 for bf16 inputs.
"""

import numpy as np
import pytest

import oracle
from linear_attention_sequence_kda_amd import inputs as gen

from gpu_util import TOL, flat_heads, say, to_dev, to_f64

pytestmark = pytest.mark.gpu

ALL = oracle.NORM_QK | oracle.BETA_LOGIT | oracle.GATE_RAW


def _kda():
    import linear_attention_sequence_kda_amd as kda
    return kda


def mixed_inputs(w, flags, draw):
    """Inputs for a flag set: the raw draw where a bit asks for it, the
    default (already preprocessed) draw of the same stream elsewhere."""
    x, r = draw(False), draw(True)
    out = dict(x)
    if flags & oracle.NORM_QK:
        out["q"], out["k"] = r["q"], r["k"]
    if flags & oracle.BETA_LOGIT:
        out["beta"] = r["beta"]
    if flags & oracle.GATE_RAW and w.alpha_mode != gen.ALPHA_NONE:
        out["log_alpha"] = r["log_alpha"]
    return out


def oracle_raw(w, xf, flags, S0=None):
    q, k, v, la, b = oracle.preprocess(xf["q"], xf["k"], xf["v"], xf["log_alpha"], xf["beta"],
                                       flags, qkv_dtype=w.qkv_dtype, gate_dtype=w.gate_dtype)
    return oracle.forward(q, k, v, la, b, xf["S0"] if S0 is None else S0, qkv_dtype="f64",
                          gate_dtype="f64", alpha_mode=w.alpha_mode)


def _dev(w, x):
    g = lambda n: to_dev(x[n], w.qkv_dtype if n in ("q", "k", "v") else w.gate_dtype)
    return {n: g(n) for n in ("q", "k", "v", "log_alpha", "beta")} | {
        "S0": to_dev(x["S0"], gen.F32) if x.get("S0") is not None else None}


def run_prefill(w, flags, label, edit=None):
    import torch
    kda = _kda()
    x = mixed_inputs(w, flags, lambda raw: gen.prefill_inputs(w, raw=raw))
    if edit is not None:
        x = edit(x)
    d = _dev(w, x)
    say(f"{label}: chunk_fwd_ex flags={flags} B={w.B} H={w.H} L={w.L} dk={w.dk} dv={w.dv} "
        f"{w.qkv_dtype}/{w.gate_dtype}/{w.alpha_mode} seed={w.seed}")
    o, Sf = kda.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"],
                          flags=flags)
    torch.cuda.synchronize()
    N = w.B * w.H
    o_ref, S_ref = oracle_raw(w, flat_heads(x, N), flags)
    tol = TOL[w.qkv_dtype]
    e_o = oracle.slab_error(to_f64(o).reshape(N, w.L, w.dv), o_ref, 1)
    e_s = oracle.slab_error(to_f64(Sf).reshape(N, w.dk, w.dv), S_ref, 1)
    say(f"{label}: err o={e_o:.3e} S={e_s:.3e} (tol {tol})")
    assert e_o <= tol, f"o error {e_o}"
    assert e_s <= tol, f"S_final error {e_s}"
    return o, Sf


DTYPES = [("f32", "f32", "none"), ("f32", "f32", "head"), ("f32", "f32", "channel"),
          ("bf16", "f32", "head"), ("bf16", "bf16", "channel"), ("bf16", "f32", "channel"),
          ("bf16", "bf16", "head")]
DIMS = [(64, 64), (128, 128), (128, 64), (64, 128)]


@pytest.mark.parametrize("qd,gd,mode", DTYPES, ids=lambda x: str(x))
@pytest.mark.parametrize("dk,dv", DIMS, ids=lambda x: str(x))
@pytest.mark.parametrize("L", [1, 130])
def test_prefill_raw_small(qd, gd, mode, dk, dv, L):
    w = gen.custom(B=2, H=2, L=L, dk=dk, dv=dv, qkv_dtype=qd, gate_dtype=gd, alpha_mode=mode,
                   seed=3000 + L + dk + dv)
    run_prefill(w, ALL, "raw-small")


@pytest.mark.parametrize("flags", list(range(8)))
@pytest.mark.parametrize("qd,gd,mode", [("bf16", "bf16", "channel"), ("bf16", "f32", "head"),
                                        ("f32", "f32", "channel")], ids=lambda x: str(x))
def test_prefill_flag_subsets(flags, qd, gd, mode):
    w = gen.custom(B=1, H=3, L=200, dk=128, dv=128, qkv_dtype=qd, gate_dtype=gd,
                   alpha_mode=mode, seed=41 + flags)
    run_prefill(w, flags, "subset")


@pytest.mark.parametrize("qd,mode", [("bf16", "channel"), ("bf16", "head"), ("f32", "none")])
def test_prefill_zero_rows(qd, mode):
    """A zero raw q row gives o = 0 for that token; a zero raw k row writes
    nothing (the 1e-12 floor keeps both zero, no NaN)."""
    import torch
    w = gen.custom(B=1, H=2, L=150, dk=128, dv=128, qkv_dtype=qd, gate_dtype="f32",
                   alpha_mode=mode, seed=9)

    def edit(x):
        x = dict(x)
        x["q"] = x["q"].copy()
        x["k"] = x["k"].copy()
        x["q"][:, :, [0, 5, 64, 149]] = 0
        x["k"][:, :, [3, 63, 100]] = 0
        return x
    o, Sf = run_prefill(w, ALL, "zero-rows", edit=edit)
    assert bool(torch.isfinite(o.float()).all()) and bool(torch.isfinite(Sf).all())
    assert torch.count_nonzero(o[:, :, [0, 5, 64, 149]]) == 0


@pytest.mark.parametrize("qd,gd,mode", [("bf16", "bf16", "channel"), ("bf16", "f32", "head"),
                                        ("f32", "f32", "none")], ids=lambda x: str(x))
def test_prefill_flags_zero_is_plain_entry(qd, gd, mode):
    """kda_chunk_fwd_ex with flags = 0 is kda_chunk_fwd, bit for bit."""
    import torch
    kda = _kda()
    w = gen.custom(B=2, H=4, L=333, dk=128, dv=128, qkv_dtype=qd, gate_dtype=gd,
                   alpha_mode=mode, seed=5)
    d = _dev(w, gen.prefill_inputs(w))
    say(f"flags0-vs-plain {qd}/{gd}/{mode}")
    o1, s1 = kda.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"])
    o2, s2 = kda.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"], flags=0)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


@pytest.mark.parametrize("cfg", [2, 3])
def test_prefill_raw_workload(cfg):
    """The full-size prefill workloads, drawn raw (same streams) and
    preprocessed by the kernels."""
    run_prefill(gen.WORKLOADS[cfg], ALL, f"raw-workload{cfg}")


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------

def run_decode(w, steps, flags, label):
    import torch
    kda = _kda()
    S0 = gen.decode_state(w)
    S = to_dev(S0, gen.F32) if S0 is not None else torch.zeros(
        (w.B, w.H, w.dk, w.dv), dtype=torch.float32, device="cuda:0")
    outs, per_step = [], []
    for t in range(steps):
        x = mixed_inputs(w, flags, lambda raw: gen.decode_inputs(w, t, raw=raw))
        per_step.append(x)
        d = _dev(w, x)
        if t == 0:
            say(f"{label}: decode_ex flags={flags} B={w.B} H={w.H} dk={w.dk} dv={w.dv} "
                f"{w.qkv_dtype}/{w.gate_dtype}/{w.alpha_mode} steps={steps}")
        outs.append(kda.decode_step(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], S,
                                    flags=flags))
    torch.cuda.synchronize()
    N = w.B * w.H
    stack = lambda key: None if per_step[0][key] is None else np.stack(
        [p[key] for p in per_step], axis=2).reshape((N, steps) + per_step[0][key].shape[2:])
    xf = {n: stack(n) for n in ("q", "k", "v", "log_alpha", "beta")}
    xf["S0"] = None if S0 is None else S0.reshape(N, w.dk, w.dv)
    o_ref, S_ref = oracle_raw(w, xf, flags)
    og = np.stack([to_f64(o) for o in outs], axis=2).reshape(N, steps, w.dv)
    e_o = oracle.slab_error(og, o_ref, 1)
    e_s = oracle.slab_error(to_f64(S).reshape(N, w.dk, w.dv), S_ref, 1)
    tol = TOL[w.qkv_dtype]
    say(f"{label}: err o={e_o:.3e} S={e_s:.3e} (tol {tol})")
    assert e_o <= tol and e_s <= tol


@pytest.mark.parametrize("qd,gd,mode", DTYPES, ids=lambda x: str(x))
@pytest.mark.parametrize("dk,dv", DIMS, ids=lambda x: str(x))
def test_decode_raw_small(qd, gd, mode, dk, dv):
    w = gen.custom(B=3, H=4, L=1, dk=dk, dv=dv, qkv_dtype=qd, gate_dtype=gd, alpha_mode=mode,
                   seed=500 + dk + dv).replace(decode_steps=5)
    run_decode(w, 5, ALL, "decode-raw")


@pytest.mark.parametrize("flags", list(range(8)))
def test_decode_flag_subsets(flags):
    w = gen.custom(B=2, H=8, L=1, dk=128, dv=128, qkv_dtype="bf16", gate_dtype="f32",
                   alpha_mode="channel", seed=60 + flags).replace(decode_steps=3)
    run_decode(w, 3, flags, "decode-subset")


def test_decode_raw_workload():
    """The serving-size decode workload (256 sequences x 32 heads), 4 steps."""
    run_decode(gen.WORKLOADS[5], 4, ALL, "decode-raw-workload")


@pytest.mark.parametrize("mode", ["channel", "head"])
def test_decode_slots_raw(mode):
    """kda_decode_step_slots_ex equals kda_decode_step_ex on the gathered
    states, bit for bit, and leaves idle sequences at o = 0."""
    import torch
    kda = _kda()
    B, H, n_slots = 5, 4, 8
    w = gen.custom(B=B, H=H, L=1, dk=128, dv=128, qkv_dtype="bf16", gate_dtype="f32",
                   alpha_mode=mode, seed=78).replace(decode_steps=1)
    pool_w = w.replace(B=n_slots)
    pool0 = to_dev(gen.decode_state(pool_w), "f32")
    xt = gen.decode_inputs(w, 0, raw=True)
    d = _dev(w, xt)
    args = [d[n] for n in ("q", "k", "v", "log_alpha", "beta")]
    slots_h = [2, 7, 0, -1, 5]
    slots = torch.tensor(slots_h, dtype=torch.int32, device="cuda:0")
    say(f"decode slots raw {mode}")
    pool = pool0.clone()
    o = kda.decode_step_slots(*args, pool, slots, flags=ALL)
    live = [b for b, sl in enumerate(slots_h) if sl >= 0]
    S_g = pool0[[slots_h[b] for b in live]].contiguous()
    o_ref = kda.decode_step(*[t[live].contiguous() for t in args], S_g, flags=ALL)
    torch.cuda.synchronize()
    assert torch.equal(o[live], o_ref)
    assert torch.count_nonzero(o[3]) == 0
    for b in live:
        assert torch.equal(pool[slots_h[b]], S_g[live.index(b)])
    # and the oracle on the live sequences
    N = len(live) * H
    f = lambda a: None if a is None else np.ascontiguousarray(a[live]).reshape(
        (N, 1) + a.shape[2:])
    xf = {n: f(xt[n]) for n in ("q", "k", "v", "log_alpha", "beta")}
    xf["S0"] = gen.decode_state(pool_w)[[slots_h[b] for b in live]].reshape(N, 128, 128)
    o_or, S_or = oracle_raw(w, xf, ALL)
    assert oracle.slab_error(to_f64(o[live]).reshape(N, 1, 128), o_or, 1) <= TOL["bf16"]
    S_new = torch.stack([pool[slots_h[b]] for b in live]).reshape(N, 128, 128)
    assert oracle.slab_error(to_f64(S_new), S_or, 1) <= TOL["bf16"]


@pytest.mark.parametrize("gd,dk", [("f32", 128), ("bf16", 64)])
def test_prefill_raw_gate_strong(gd, dk):
    """Raw gates g up to about 4.5 give ln(alpha) = -exp(g) down to about -90:
    every sub-block's decay leaves the range of the kernel's factored split
    and takes its direct path."""
    w = gen.custom(B=1, H=3, L=150, dk=dk, dv=128, qkv_dtype="bf16", gate_dtype=gd,
                   alpha_mode="channel", seed=91 + dk, la_mu=3.0, la_sigma=0.6)
    run_prefill(w, oracle.GATE_RAW | oracle.NORM_QK | oracle.BETA_LOGIT, "raw strong gate")
