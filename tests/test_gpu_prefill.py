"""Parity of kda_chunk_fwd (HIP, through the C ABI) with the fp64 CPU oracle.

Metric: per (b, h) slab, max|x - ref| / max|ref|, worst slab; o and S_final
each.  Bar: 1e-4 for fp32 inputs, 2e-2 for bf16 inputs.
"""

import numpy as np
import pytest

import oracle
from linear_attention_sequence_kda_amd import inputs as gen

from gpu_util import TOL, device_inputs, flat_heads, oracle_prefill, say, to_dev, to_f64

pytestmark = pytest.mark.gpu


def _kda():
    import linear_attention_sequence_kda_amd as kda
    return kda


def run_and_compare(w: gen.Workload, label: str, tol=None):
    import torch
    kda = _kda()
    x = gen.prefill_inputs(w)
    N = w.B * w.H
    d = device_inputs(w, x)
    say(f"{label}: chunk_fwd B={w.B} H={w.H} L={w.L} dk={w.dk} dv={w.dv} "
        f"{w.qkv_dtype}/{w.gate_dtype}/{w.alpha_mode} seed={w.seed}")
    o, Sf = kda.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"])
    torch.cuda.synchronize()
    xf = flat_heads(x, N)
    o_ref, S_ref = oracle_prefill(w, xf)
    tol = TOL[w.qkv_dtype] if tol is None else tol
    e_o = oracle.slab_error(to_f64(o).reshape(N, w.L, w.dv), o_ref, 1)
    e_s = oracle.slab_error(to_f64(Sf).reshape(N, w.dk, w.dv), S_ref, 1)
    say(f"{label}: err o={e_o:.3e} S={e_s:.3e} (tol {tol})")
    assert e_o <= tol, f"o error {e_o}"
    assert e_s <= tol, f"S_final error {e_s}"
    return o, Sf


DTYPES = [("f32", "f32", "none"), ("f32", "f32", "head"), ("f32", "f32", "channel"),
          ("bf16", "f32", "head"), ("bf16", "bf16", "channel"), ("bf16", "f32", "channel"),
          ("bf16", "bf16", "none"), ("f32", "bf16", "channel")]
DIMS = [(64, 64), (128, 128), (128, 64), (64, 128)]


@pytest.mark.parametrize("qd,gd,mode", DTYPES, ids=lambda x: str(x))
@pytest.mark.parametrize("dk,dv", DIMS, ids=lambda x: str(x))
@pytest.mark.parametrize("L", [1, 65, 200])
def test_small_shapes(qd, gd, mode, dk, dv, L):
    w = gen.custom(B=2, H=2, L=L, dk=dk, dv=dv, qkv_dtype=qd, gate_dtype=gd, alpha_mode=mode,
                   seed=1000 + L + dk + dv)
    run_and_compare(w, "small")


@pytest.mark.parametrize("L", [63, 64, 127, 128, 129, 640])
def test_chunk_boundaries(L):
    w = gen.custom(B=1, H=3, L=L, dk=128, dv=128, qkv_dtype="bf16", gate_dtype="bf16",
                   alpha_mode="channel", seed=L)
    run_and_compare(w, "boundary")


@pytest.mark.parametrize("B,H,dk,dv,qd", [(2, 32, 128, 128, "bf16"),    # 32-column slices
                                          (4, 16, 128, 64, "bf16"),     # 32-column slices, dv 64
                                          (4, 64, 64, 64, "bf16"),      # 64-column slices
                                          (2, 64, 64, 128, "f32"),      # fp32, 32-column slices
                                          (2, 64, 128, 128, "f32")])
def test_slice_widths(B, H, dk, dv, qd):
    w = gen.custom(B=B, H=H, L=150, dk=dk, dv=dv, qkv_dtype=qd, gate_dtype="f32",
                   alpha_mode="channel", seed=B * H)
    run_and_compare(w, "slices")


# per-channel decay in bf16 runs a state pass whose slice width follows the
# number of heads: 16 columns up to 63 heads (d_v = 128), 32 up to 127, 64
# beyond; each width, with d_k = 64 and 128 and d_v = 64 too
@pytest.mark.parametrize("B,H,dk,dv", [(1, 5, 128, 128), (2, 48, 128, 128), (4, 40, 128, 128),
                                       (2, 70, 64, 128), (3, 50, 128, 64), (5, 60, 64, 64),
                                       (1, 3, 64, 64)])
def test_kda_state_pass_slice_widths(B, H, dk, dv):
    w = gen.custom(B=B, H=H, L=150, dk=dk, dv=dv, qkv_dtype="bf16", gate_dtype="bf16",
                   alpha_mode="channel", s0_std=0.02, seed=B * H + dk + dv)
    run_and_compare(w, "kda slices")


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_workload_full(cfg):
    run_and_compare(gen.WORKLOADS[cfg], f"workload{cfg}")


def test_long_context_full():
    """The long-context workload (1 x 16 heads x 524,288 tokens, per-channel
    decay, S_final returned) at full size, in the launch configuration the
    benchmark times, against the oracle on every head and every column of o
    and S_final.  The oracle runs a few heads at a time (each head's fp64 o
    is 537 MB) with one worker per (head, 32-column block)."""
    import torch
    kda = _kda()
    w = gen.WORKLOADS[4]
    say("workload4: drawing inputs")
    x = gen.prefill_inputs(w, threads=16)
    d = device_inputs(w, x)
    say("workload4: chunk_fwd full size")
    o, Sf = kda.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"])
    torch.cuda.synchronize()
    del d
    assert torch.isfinite(o).all() and torch.isfinite(Sf).all()
    o_h = o[0].cpu()            # [H, L, dv] in bf16
    s_h = to_f64(Sf[0])         # [H, dk, dv]
    del o
    torch.cuda.empty_cache()
    threads = oracle.default_threads()
    group = max(1, min(w.H, threads // max(1, w.dv // 32)))
    worst_o = worst_s = 0.0
    for h0 in range(0, w.H, group):
        hs = list(range(h0, min(w.H, h0 + group)))
        xs = {k: (None if v is None else np.ascontiguousarray(v[0, hs])) for k, v in x.items()}
        say(f"workload4: oracle on heads {hs[0]}..{hs[-1]}")
        o_ref, S_ref = oracle.forward(xs["q"], xs["k"], xs["v"], xs["log_alpha"], xs["beta"],
                                      None, qkv_dtype="bf16", gate_dtype="bf16",
                                      alpha_mode="channel", threads=threads)
        e_o = oracle.slab_error(o_h[hs].float().numpy().astype(np.float64), o_ref, 1)
        e_s = oracle.slab_error(s_h[hs], S_ref, 1)
        del o_ref, S_ref
        say(f"workload4: heads {hs[0]}..{hs[-1]} err o={e_o:.3e} S={e_s:.3e}")
        worst_o, worst_s = max(worst_o, e_o), max(worst_s, e_s)
    say(f"workload4: worst err o={worst_o:.3e} S={worst_s:.3e} (tol {TOL['bf16']})")
    assert worst_o <= TOL["bf16"], f"o error {worst_o}"
    assert worst_s <= TOL["bf16"], f"S_final error {worst_s}"


# ---------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------

def test_empty_sequence_returns_initial_state():
    import torch
    kda = _kda()
    w = gen.custom(B=2, H=3, L=0, dk=128, dv=128, qkv_dtype="bf16", gate_dtype="f32")
    q = torch.empty((2, 3, 0, 128), dtype=torch.bfloat16, device="cuda:0")
    la = torch.empty((2, 3, 0, 128), dtype=torch.float32, device="cuda:0")
    beta = torch.empty((2, 3, 0), dtype=torch.float32, device="cuda:0")
    S0 = torch.randn((2, 3, 128, 128), device="cuda:0")
    say("empty: L=0")
    o, Sf = kda.chunk_fwd(q, q, q, la, beta, S0)
    torch.cuda.synchronize()
    assert o.shape == (2, 3, 0, 128)
    assert torch.equal(Sf, S0)
    o, Sf = kda.chunk_fwd(q, q, q, la, beta, None)
    torch.cuda.synchronize()
    assert torch.count_nonzero(Sf) == 0


def test_zero_inputs_keep_state_bitwise():
    import torch
    kda = _kda()
    B, H, L, d = 1, 4, 100, 128
    z = torch.zeros((B, H, L, d), dtype=torch.bfloat16, device="cuda:0")
    la = torch.zeros((B, H, L, d), dtype=torch.bfloat16, device="cuda:0")
    beta = torch.rand((B, H, L), device="cuda:0").to(torch.bfloat16)
    S0 = torch.randn((B, H, d, d), device="cuda:0")
    say("zeros")
    o, Sf = kda.chunk_fwd(z, z, z, la, beta, S0)
    torch.cuda.synchronize()
    assert torch.count_nonzero(o) == 0
    assert torch.equal(Sf, S0)


def test_exact_replacement_on_gpu():
    """beta = 1 and q = k (unit keys) must read back each value."""
    import torch
    kda = _kda()
    w = gen.custom(B=1, H=4, L=130, dk=128, dv=128, qkv_dtype="f32", gate_dtype="f32",
                   alpha_mode="channel", seed=9)
    x = gen.prefill_inputs(w)
    d = device_inputs(w, x)
    ones = torch.ones_like(d["beta"])
    say("replacement")
    o, _ = kda.chunk_fwd(d["k"], d["k"], d["v"], d["log_alpha"], ones, d["S0"])
    torch.cuda.synchronize()
    v = to_f64(d["v"])
    err = np.abs(to_f64(o) - v).max() / np.abs(v).max()
    assert err <= 1e-4


def test_in_place_final_state():
    import torch
    kda = _kda()
    w = gen.custom(B=2, H=4, L=100, dk=128, dv=128, qkv_dtype="bf16", gate_dtype="bf16", seed=3)
    x = gen.prefill_inputs(w)
    d = device_inputs(w, x)
    say("in-place S_final = S0")
    o1, S1 = kda.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"])
    S = d["S0"].clone()
    o2, S2 = kda.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], S, S_final=S)
    torch.cuda.synchronize()
    assert S2.data_ptr() == S.data_ptr()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


@pytest.mark.parametrize("split", [37, 64, 100])
def test_split_sequence_state_passing(split):
    import torch
    kda = _kda()
    w = gen.custom(B=1, H=4, L=200, dk=128, dv=128, qkv_dtype="bf16", gate_dtype="bf16",
                   alpha_mode="channel", seed=21)
    x = gen.prefill_inputs(w)
    d = device_inputs(w, x)
    sl = lambda t, a, b: t[:, :, a:b].contiguous()
    say(f"split at {split}")
    o1, Sm = kda.chunk_fwd(*(sl(d[n], 0, split) for n in ("q", "k", "v", "log_alpha", "beta")),
                           d["S0"])
    o2, Se = kda.chunk_fwd(*(sl(d[n], split, 200) for n in ("q", "k", "v", "log_alpha", "beta")),
                           Sm)
    torch.cuda.synchronize()
    xf = flat_heads(x, 4)
    o_ref, S_ref = oracle_prefill(w, xf)
    og = np.concatenate([to_f64(o1), to_f64(o2)], axis=2).reshape(4, 200, 128)
    assert oracle.slab_error(og, o_ref, 1) <= TOL["bf16"]
    assert oracle.slab_error(to_f64(Se).reshape(4, 128, 128), S_ref, 1) <= TOL["bf16"]


def test_nan_stays_in_its_head():
    import torch
    kda = _kda()
    w = gen.custom(B=1, H=4, L=130, dk=128, dv=128, qkv_dtype="bf16", gate_dtype="bf16", seed=5)
    x = gen.prefill_inputs(w)
    d = device_inputs(w, x)
    d["v"][0, 2, 70, 5] = float("nan")
    say("nan confinement")
    o, Sf = kda.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"])
    torch.cuda.synchronize()
    for h in (0, 1, 3):
        assert torch.isfinite(o[0, h]).all() and torch.isfinite(Sf[0, h]).all()
    assert not torch.isfinite(o[0, 2]).all()


def test_deterministic():
    import torch
    kda = _kda()
    w = gen.custom(B=2, H=32, L=300, dk=128, dv=128, qkv_dtype="bf16", gate_dtype="bf16", seed=8)
    x = gen.prefill_inputs(w)
    d = device_inputs(w, x)
    say("determinism")
    ref = kda.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"])
    for _ in range(5):
        o, Sf = kda.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"])
        torch.cuda.synchronize()
        assert torch.equal(o, ref[0]) and torch.equal(Sf, ref[1])


def _strong_decay_case(w, x, label):
    import torch
    kda = _kda()
    N = w.B * w.H
    d = device_inputs(w, x)
    say(f"{label}: B={w.B} H={w.H} L={w.L} dk={w.dk} dv={w.dv} {w.qkv_dtype}/{w.gate_dtype} "
        f"ln(alpha) in [{float(np.min(gen.widen(x['log_alpha'], w.gate_dtype))):.1f}, "
        f"{float(np.max(gen.widen(x['log_alpha'], w.gate_dtype))):.3f}]")
    o, Sf = kda.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"])
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_prefill(w, flat_heads(x, N))
    tol = TOL[w.qkv_dtype]
    e_o = oracle.slab_error(to_f64(o).reshape(N, w.L, w.dv), o_ref, 1)
    e_s = oracle.slab_error(to_f64(Sf).reshape(N, w.dk, w.dv), S_ref, 1)
    say(f"{label}: err o={e_o:.3e} S={e_s:.3e}")
    assert e_o <= tol and e_s <= tol, (e_o, e_s)


# ln(alpha) = -exp(N(mu, sigma)): mu = 1.2 reaches about -5, mu = 3.0 about
# -20 (every 16-token sub-block leaves the split's range), mu = 1.5 with
# sigma = 1 mixes weak and very strong channels within one sub-block
@pytest.mark.parametrize("mu,sigma", [(1.2, 0.3), (3.0, 0.3), (1.5, 1.0)])
@pytest.mark.parametrize("qd,gd,dk", [("bf16", "f32", 128), ("bf16", "bf16", 64),
                                      ("f32", "f32", 128)])
def test_strong_decay(mu, sigma, qd, gd, dk):
    """Per-channel decay of any strength meets the bar: nothing in the
    factored decay may overflow (the oracle has no limit either)."""
    w = gen.custom(B=1, H=4, L=200, dk=dk, dv=128, qkv_dtype=qd, gate_dtype=gd,
                   alpha_mode="channel", seed=31 + int(10 * mu) + dk, la_mu=mu, la_sigma=sigma)
    _strong_decay_case(w, gen.prefill_inputs(w), f"strong decay mu={mu} sigma={sigma}")


def test_decay_wipes_and_mixed_sub_blocks():
    """Single tokens that wipe a channel (ln(alpha) = -1000) inside otherwise
    weakly decaying sub-blocks, and sub-blocks where only one channel leaves
    the split's range."""
    w = gen.custom(B=1, H=3, L=300, dk=128, dv=128, qkv_dtype="bf16", gate_dtype="f32",
                   alpha_mode="channel", seed=77)
    x = gen.prefill_inputs(w)
    la = x["log_alpha"].copy()
    rng = np.random.default_rng(5)
    t = rng.integers(0, w.L, size=40)
    c = rng.integers(0, w.dk, size=40)
    la[0, 0, t, c] = -1000.0                      # wipes on head 0
    la[0, 1, 64:80, 7] = -12.0                    # one channel of one sub-block on head 1
    la[0, 2, :, :5] = -30.0                       # five channels everywhere on head 2
    x["log_alpha"] = la.astype(np.float32)
    _strong_decay_case(w, x, "wipes and mixed sub-blocks")


def test_head_gate_equals_broadcast_channel_gate():
    """A per-head gate and the same gate broadcast over channels are the same
    recurrence; the two kernel paths (decay on results vs decay in operands)
    must each meet the bar against the oracle and agree with each other."""
    import torch
    kda = _kda()
    w = gen.custom(B=1, H=4, L=150, dk=128, dv=128, qkv_dtype="bf16", gate_dtype="f32",
                   alpha_mode="head", seed=12)
    x = gen.prefill_inputs(w)
    d = device_inputs(w, x)
    la_c = d["log_alpha"][..., None].expand(1, 4, 150, 128).contiguous()
    say("head vs channel gate")
    a = kda.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"])
    b = kda.chunk_fwd(d["q"], d["k"], d["v"], la_c, d["beta"], d["S0"])
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_prefill(w, flat_heads(x, 4))
    for o, Sf in (a, b):
        assert oracle.slab_error(to_f64(o).reshape(4, 150, 128), o_ref, 1) <= TOL["bf16"]
        assert oracle.slab_error(to_f64(Sf).reshape(4, 128, 128), S_ref, 1) <= TOL["bf16"]
    assert oracle.slab_error(to_f64(a[0]).reshape(4, 150, 128),
                             to_f64(b[0]).reshape(4, 150, 128), 1) <= 2 * TOL["bf16"]


@pytest.mark.parametrize("mode,gd,L", [("channel", "bf16", 100_000), ("head", "f32", 330_000)])
def test_few_heads_several_spans(mode, gd, L):
    """Two heads and a sequence long enough for several record spans (4 with
    per-channel decay; 2 with one decay per token, the second only 37 chunks),
    with 16-column state slices.  Checked against the oracle on a block of
    state columns, with and without S_final (the state then crosses spans
    through the workspace), and bit for bit across repeated calls."""
    import torch
    kda = _kda()
    w = gen.custom(B=1, H=2, L=L, dk=128, dv=128, qkv_dtype="bf16", gate_dtype=gd,
                   alpha_mode=mode, s0_std=0.02, seed=L + 5)
    x = gen.prefill_inputs(w, threads=16)
    d = device_inputs(w, x)
    args = (d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"])
    say(f"few heads, several spans: {mode} L={L}")
    o1, S1 = kda.chunk_fwd(*args)
    o2, S2 = kda.chunk_fwd(*args)
    o3, none = kda.chunk_fwd(*args, output_final_state=False)
    torch.cuda.synchronize()
    assert none is None
    assert torch.equal(o1, o2) and torch.equal(S1, S2) and torch.equal(o1, o3)
    col0, ncols = 72, 16
    xs = {k: (None if v is None else np.ascontiguousarray(v[0])) for k, v in x.items()}
    say(f"few heads, several spans {mode}: oracle on a column block")
    o_ref, S_ref = oracle.forward(xs["q"], xs["k"], xs["v"], xs["log_alpha"], xs["beta"],
                                  np.ascontiguousarray(xs["S0"]), qkv_dtype="bf16",
                                  gate_dtype=gd, alpha_mode=mode, col0=col0, ncols=ncols)
    e_o = oracle.slab_error(to_f64(o1[0, :, :, col0:col0 + ncols]), o_ref, 1)
    e_s = oracle.slab_error(to_f64(S1[0, :, :, col0:col0 + ncols]), S_ref, 1)
    say(f"few heads, several spans {mode}: err o={e_o:.3e} S={e_s:.3e}")
    assert e_o <= TOL["bf16"] and e_s <= TOL["bf16"]


def test_multi_span_call_follows_the_callers_stream():
    """A multi-span call on a non-default stream starts after the work queued
    before it there and ends before the work queued after it.  Here an input
    is written on that stream behind a long GPU sleep, the call follows, and
    a copy of o and S_final is taken on it right after; all must match a
    call on settled inputs bit for bit."""
    import torch
    kda = _kda()
    w = gen.custom(B=1, H=2, L=100_000, dk=128, dv=128, qkv_dtype="bf16", gate_dtype="bf16",
                   alpha_mode="channel", s0_std=0.02, seed=613)
    x = gen.prefill_inputs(w, threads=16)
    d = device_inputs(w, x)
    say("multi-span call on a caller's stream")
    o_ref, S_ref = kda.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"])
    k2 = torch.zeros_like(d["k"])
    torch.cuda.synchronize()
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        torch.cuda._sleep(20_000_000)  # a few milliseconds of GPU time
        k2.copy_(d["k"])
        o, S = kda.chunk_fwd(d["q"], k2, d["v"], d["log_alpha"], d["beta"], d["S0"])
        o_copy, S_copy = o.clone(), S.clone()
    st.synchronize()
    assert torch.equal(o_copy, o_ref) and torch.equal(S_copy, S_ref)


def test_caller_workspace_and_multi_span_state_area():
    """A caller-supplied workspace of exactly the queried size gives the same
    bits as the binding's own; a smaller one is rejected before any launch.
    Without S_final, a multi-span call (KDA records, 2 spans here) carries the
    state through the workspace's state area and must give the same o."""
    import torch
    kda = _kda()
    from linear_attention_sequence_kda_amd.binding import KdaError
    w = gen.custom(B=2, H=32, L=2048, dk=128, dv=128, qkv_dtype="bf16", gate_dtype="bf16",
                   alpha_mode="channel", seed=31)
    x = gen.prefill_inputs(w)
    d = device_inputs(w, x)
    args = (d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"])
    say("caller workspace / multi-span state area")
    wsb = kda.chunk_fwd_workspace_bytes(d["q"], d["v"], d["log_alpha"], d["beta"])
    assert wsb > 0
    o_ref, S_ref = kda.chunk_fwd(*args)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda:0")
    o1, S1 = kda.chunk_fwd(*args, workspace=ws)
    o2, none = kda.chunk_fwd(*args, output_final_state=False, workspace=ws)
    torch.cuda.synchronize()
    assert none is None
    assert torch.equal(o1, o_ref) and torch.equal(S1, S_ref)
    assert torch.equal(o2, o_ref)
    small = torch.empty(wsb - 256, dtype=torch.uint8, device="cuda:0")
    with pytest.raises(KdaError) as ei:
        kda.chunk_fwd(*args, workspace=small)
    assert ei.value.status == 6
    N = w.B * w.H
    o_or, _ = oracle_prefill(w, flat_heads(x, N))
    assert oracle.slab_error(to_f64(o2).reshape(N, w.L, w.dv), o_or, 1) <= TOL["bf16"]


def test_kernel_timing_counts_launches():
    """kda_timing_* sees one intra-chunk and one inter-chunk launch per
    single-span call and one decode launch per step, with positive times."""
    import torch
    kda = _kda()
    w = gen.custom(B=1, H=4, L=300, dk=128, dv=128, qkv_dtype="bf16", gate_dtype="f32",
                   alpha_mode="head", seed=41)
    d = device_inputs(w, gen.prefill_inputs(w))
    say("kernel timing")
    kda.timing_reset()
    kda.timing_enable(True)
    try:
        for _ in range(2):
            kda.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"])
        S = torch.zeros((1, 4, 128, 128), dtype=torch.float32, device="cuda:0")
        kda.decode_step(d["q"][:, :, 0].contiguous(), d["k"][:, :, 0].contiguous(),
                        d["v"][:, :, 0].contiguous(), d["log_alpha"][:, :, 0].contiguous(),
                        d["beta"][:, :, 0].contiguous(), S)
        torch.cuda.synchronize()
    finally:
        kda.timing_enable(False)
    got = {k: kda.timing_read(k) for k in kda.binding.KERNELS}
    kda.timing_reset()
    assert got["kda_intra_kernel"][0] == 2 and got["kda_inter_scalar_kernel"][0] == 2
    assert got["kda_decode_kernel"][0] == 1 and got["kda_inter_kernel"][0] == 0
    for k in ("kda_intra_kernel", "kda_inter_scalar_kernel", "kda_decode_kernel"):
        assert got[k][1] > 0.0
    assert kda.timing_read("kda_intra_kernel") == (0, 0.0)


_PLAN_LOG_PROG = r"""
import sys
sys.path.insert(0, {root!r})
import torch
import linear_attention_sequence_kda_amd as kda
from linear_attention_sequence_kda_amd import inputs as gen
sys.path.insert(0, {tests!r})
from gpu_util import device_inputs
w = gen.custom(B=1, H=3, L=200, dk=128, dv=128, qkv_dtype="bf16", gate_dtype="bf16",
               alpha_mode="channel", seed=5)
d = device_inputs(w, gen.prefill_inputs(w))
kda.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"])
torch.cuda.synchronize()
print("done", flush=True)
"""


def test_log_reports_the_prefill_plan():
    """KDA_LOG=1 in a child process: a prefill call logs its shape and its plan
    (chunks, spans, record bytes, the state pass and its slice width)."""
    import os
    import subprocess
    import sys
    here = os.path.dirname(os.path.abspath(__file__))
    root = os.path.dirname(here)
    env = dict(os.environ, KDA_LOG="1")
    say("KDA_LOG plan line (child process)")
    p = subprocess.run([sys.executable, "-c", _PLAN_LOG_PROG.format(root=root, tests=here)],
                       env=env, capture_output=True, text=True, timeout=300)
    assert p.returncode == 0 and "done" in p.stdout, p.stderr[-2000:]
    lines = [x for x in p.stderr.splitlines() if x.startswith("[kda] ")]
    assert any("kda_chunk_fwd: B=1 H=3 L=200 dk=128 dv=128 qkv=bf16 gate=bf16 alpha=channel" in x
               for x in lines), lines
    assert any("kda_chunk_fwd: 4 chunks of 64 in 1 span(s) of 4" in x and
               "state pass kda_inter_quad_kernel, 16-column slices" in x for x in lines), lines
    assert not any("status" in x for x in lines), lines


def test_longest_sequence_fp32():
    """The longest sequence the ABI accepts (L = INT_MAX / 512 = 4,194,303
    tokens, one head): with fp32 q, k, v and per-channel gates every head's
    rows span just under 2 GiB, where the kernels' 32-bit byte offsets are at
    their limit; the last chunk is ragged (31 of 32 tokens).  Every column of
    o and S_final against the oracle."""
    import torch
    kda = _kda()
    L = (2 ** 31 - 1) // 512
    w = gen.custom(B=1, H=1, L=L, dk=128, dv=128, qkv_dtype="f32", gate_dtype="f32",
                   alpha_mode="channel", seed=77)
    say(f"longest sequence: drawing inputs L={L}")
    x = gen.prefill_inputs(w, threads=16)
    d = device_inputs(w, x)
    say("longest sequence: chunk_fwd")
    o, Sf = kda.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"])
    torch.cuda.synchronize()
    del d
    o_h = o[0].cpu().numpy().astype(np.float64)
    s_h = to_f64(Sf[0])
    del o
    torch.cuda.empty_cache()
    say("longest sequence: oracle")
    xf = flat_heads(x, 1)
    o_ref, S_ref = oracle_prefill(w, xf)
    e_o = oracle.slab_error(o_h, o_ref, 1)
    e_s = oracle.slab_error(s_h, S_ref, 1)
    say(f"longest sequence: err o={e_o:.3e} S={e_s:.3e} (tol {TOL['f32']})")
    assert e_o <= TOL["f32"], f"o error {e_o}"
    assert e_s <= TOL["f32"], f"S_final error {e_s}"


def _sweep_cases(n=20, seed=20261203):
    """Seeded random shapes: head counts on both sides of each state-pass slice
    width, ragged lengths, every dtype and decay mode, decay strengths from
    almost none to strong, with and without an initial state."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        qd, gd, mode = DTYPES[rng.integers(len(DTYPES))]
        dk, dv = DIMS[rng.integers(len(DIMS))]
        B = int(rng.integers(1, 4))
        H = int(rng.integers(1, 72 // B + 1))
        L = int(rng.integers(1, max(2, 30_000 // (B * H)) + 1))
        L = min(L, 1500)
        mu = float(rng.uniform(-6.0, -0.05))
        s0 = [None, 0.02, 0.5][int(rng.integers(3))]
        cases.append((i, B, H, L, dk, dv, qd, gd, mode, mu, s0))
    return cases


@pytest.mark.parametrize("case", _sweep_cases(), ids=lambda c: f"sweep{c[0]}")
def test_random_shape_sweep(case):
    i, B, H, L, dk, dv, qd, gd, mode, mu, s0 = case
    w = gen.custom(B=B, H=H, L=L, dk=dk, dv=dv, qkv_dtype=qd, gate_dtype=gd, alpha_mode=mode,
                   la_mu=mu, la_sigma=0.5, s0_std=s0, seed=5000 + i)
    run_and_compare(w, f"sweep{i} mu={mu:.2f} s0={s0}")
