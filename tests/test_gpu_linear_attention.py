"""Parity of kda_linear_attn_fwd (normalized linear attention, phi = elu + 1,
through the C ABI) with the fp64 oracle on the same seeded raw inputs.

Metric and bar as for the delta rule: worst (b, h) slab of max|x - ref| /
max|ref|, 1e-4 for fp32 inputs, 2e-2 for bf16 inputs; o, S_final and z_final.
"""

import numpy as np
import pytest

import oracle
from linear_attention_sequence_kda_amd import inputs as gen

from gpu_util import TOL, say, to_dev, to_f64

pytestmark = pytest.mark.gpu


def _kda():
    import linear_attention_sequence_kda_amd as kda
    return kda


def _init(B, H, dk, dv, seed):
    """A running state and normalizer of plausible size: S0 ~ N(0, 4),
    z0 ~ U(5, 50) (a normalizer sums positive features)."""
    r = np.random.default_rng(seed)
    return ((r.standard_normal((B, H, dk, dv)) * 4.0).astype(np.float32),
            r.uniform(5.0, 50.0, (B, H, dk)).astype(np.float32))


def run_la(B, H, L, dk, dv, qd, init=True, seed=0, label="la", in_place=False):
    import torch
    kda = _kda()
    w = gen.custom(B=B, H=H, L=L, dk=dk, dv=dv, qkv_dtype=qd, gate_dtype="f32",
                   alpha_mode="none", s0_std=None, seed=seed)
    x = gen.prefill_inputs(w, raw=True)
    S0n, z0n = _init(B, H, dk, dv, seed + 1) if init else (None, None)
    d = {n: to_dev(x[n], qd) for n in ("q", "k", "v")}
    S0 = to_dev(S0n, "f32") if init else None
    z0 = to_dev(z0n, "f32") if init else None
    say(f"{label}: linear_attn B={B} H={H} L={L} dk={dk} dv={dv} {qd} init={init} "
        f"in_place={in_place} seed={seed}")
    if in_place:
        o, Sf, zf = kda.linear_attn_fwd(d["q"], d["k"], d["v"], S0, z0, S_final=S0, z_final=z0)
        assert Sf.data_ptr() == S0.data_ptr() and zf.data_ptr() == z0.data_ptr()
    else:
        o, Sf, zf = kda.linear_attn_fwd(d["q"], d["k"], d["v"], S0, z0)
    torch.cuda.synchronize()
    N = B * H
    fl = lambda a, tail: None if a is None else a.reshape((N,) + tail)
    o_ref, S_ref, z_ref = oracle.linear_attention(
        fl(x["q"], (L, dk)), fl(x["k"], (L, dk)), fl(x["v"], (L, dv)),
        fl(S0n, (dk, dv)), fl(z0n, (dk,)), qkv_dtype=qd)
    tol = TOL[qd]
    e_o = oracle.slab_error(to_f64(o).reshape(N, L, dv), o_ref, 1) if L else 0.0
    e_s = oracle.slab_error(to_f64(Sf).reshape(N, dk, dv), S_ref, 1)
    e_z = oracle.slab_error(to_f64(zf).reshape(N, 1, dk), z_ref[:, None, :], 1)
    say(f"{label}: err o={e_o:.3e} S={e_s:.3e} z={e_z:.3e} (tol {tol})")
    assert e_o <= tol and e_s <= tol and e_z <= tol
    return o, Sf, zf


@pytest.mark.parametrize("qd", ["bf16", "f32"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (128, 64), (64, 128)],
                         ids=lambda x: str(x))
@pytest.mark.parametrize("L", [0, 1, 65, 200])
@pytest.mark.parametrize("init", [True, False])
def test_linear_attention_small(qd, dk, dv, L, init):
    run_la(2, 2, L, dk, dv, qd, init=init, seed=7 * L + dk + dv)


@pytest.mark.parametrize("B,H,qd", [(2, 32, "bf16"), (4, 16, "bf16"), (4, 64, "bf16"),
                                    (2, 64, "f32")])
def test_linear_attention_slice_widths(B, H, qd):
    """Head counts that select each state-column slice width."""
    run_la(B, H, 150, 128, 128, qd, seed=B * H)


def test_linear_attention_in_place_state():
    run_la(2, 4, 333, 128, 128, "bf16", in_place=True, seed=3)


def test_linear_attention_gated_deltanet_shape():
    """The prefill workload's shape (4 x 16 heads, 4096 tokens, d = 128, bf16)."""
    run_la(4, 16, 4096, 128, 128, "bf16", seed=2, label="la-4x16x4096")


def test_linear_attention_chaining():
    """Two calls chained through (S, z) agree with one call over the whole
    sequence (within the bf16 bar; the chunk grid differs at the split)."""
    import torch
    kda = _kda()
    w = gen.custom(B=2, H=4, L=300, dk=128, dv=128, qkv_dtype="bf16", gate_dtype="f32",
                   alpha_mode="none", s0_std=None, seed=9)
    x = gen.prefill_inputs(w, raw=True)
    d = {n: to_dev(x[n], "bf16") for n in ("q", "k", "v")}
    say("la chaining split at 100")
    o, S, z = kda.linear_attn_fwd(d["q"], d["k"], d["v"])
    part = lambda t, a, b: t[:, :, a:b].contiguous()
    o1, S1, z1 = kda.linear_attn_fwd(*(part(d[n], 0, 100) for n in ("q", "k", "v")))
    o2, S2, z2 = kda.linear_attn_fwd(*(part(d[n], 100, 300) for n in ("q", "k", "v")), S1, z1)
    torch.cuda.synchronize()
    oc = to_f64(torch.cat([o1, o2], dim=2)).reshape(8, 300, 128)
    assert oracle.slab_error(oc, to_f64(o).reshape(8, 300, 128), 1) <= TOL["bf16"]
    assert oracle.slab_error(to_f64(S2).reshape(8, 128, 128),
                             to_f64(S).reshape(8, 128, 128), 1) <= 1e-5
    assert oracle.slab_error(to_f64(z2).reshape(8, 1, 128), to_f64(z).reshape(8, 1, 128),
                             1) <= 1e-5


@pytest.mark.parametrize("qd", ["bf16", "f32"])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 128), (128, 64), (64, 64)],
                         ids=lambda x: str(x))
def test_linear_attention_prefill_then_decode(qd, dk, dv):
    """Serving: prefill a prompt, then decode steps continue its (S, z) in
    place; every output against the oracle over prompt + generated tokens."""
    import torch
    kda = _kda()
    B, H, L, steps = 3, 4, 130, 5
    w = gen.custom(B=B, H=H, L=L + steps, dk=dk, dv=dv, qkv_dtype=qd, gate_dtype="f32",
                   alpha_mode="none", s0_std=None, seed=41 + dk)
    x = gen.prefill_inputs(w, raw=True)
    d = {n: to_dev(x[n], qd) for n in ("q", "k", "v")}
    say(f"la prefill {L} then {steps} decode steps {qd} dk={dk} dv={dv}")
    pre = {n: t[:, :, :L].contiguous() for n, t in d.items()}
    o, S, z = kda.linear_attn_fwd(pre["q"], pre["k"], pre["v"])
    outs = [to_f64(o)]
    for t in range(L, L + steps):
        step = {n: d[n][:, :, t].contiguous() for n in d}
        outs.append(to_f64(kda.linear_attn_decode_step(step["q"], step["k"], step["v"], S, z))
                    [:, :, None])
    torch.cuda.synchronize()
    N = B * H
    og = np.concatenate(outs, axis=2).reshape(N, L + steps, dv)
    fl = lambda a, tail: a.reshape((N,) + tail)
    o_ref, S_ref, z_ref = oracle.linear_attention(fl(x["q"], (L + steps, dk)),
                                                  fl(x["k"], (L + steps, dk)),
                                                  fl(x["v"], (L + steps, dv)), qkv_dtype=qd)
    tol = TOL[qd]
    assert oracle.slab_error(og, o_ref, 1) <= tol
    assert oracle.slab_error(to_f64(S).reshape(N, dk, dv), S_ref, 1) <= tol
    assert oracle.slab_error(to_f64(z).reshape(N, 1, dk), z_ref[:, None, :], 1) <= tol


def test_linear_attention_decode_serving_size():
    """256 sequences x 32 heads, d = 128 (the decode workload's size), 3 steps
    from a given (S, z)."""
    import torch
    kda = _kda()
    B, H, d, steps = 256, 32, 128, 3
    S0n, z0n = _init(B, H, d, d, 5)
    S = to_dev(S0n, "f32")
    z = to_dev(z0n, "f32")
    w = gen.custom(B=B, H=H, L=1, dk=d, dv=d, qkv_dtype="bf16", gate_dtype="f32",
                   alpha_mode="none", s0_std=None, seed=6).replace(decode_steps=steps)
    say("la decode 256x32 3 steps")
    xs, outs = [], []
    for t in range(steps):
        xt = gen.decode_inputs(w, t, raw=True)
        xs.append(xt)
        outs.append(to_f64(kda.linear_attn_decode_step(*(to_dev(xt[n], "bf16")
                                                         for n in ("q", "k", "v")), S, z)))
    torch.cuda.synchronize()
    N = B * H
    cat = lambda key, dd: np.stack([xt[key] for xt in xs], axis=2).reshape(N, steps, dd)
    o_ref, S_ref, z_ref = oracle.linear_attention(cat("q", d), cat("k", d), cat("v", d),
                                                  S0n.reshape(N, d, d), z0n.reshape(N, d),
                                                  qkv_dtype="bf16")
    og = np.stack(outs, axis=2).reshape(N, steps, d)
    assert oracle.slab_error(og, o_ref, 1) <= TOL["bf16"]
    assert oracle.slab_error(to_f64(S).reshape(N, d, d), S_ref, 1) <= TOL["bf16"]
    assert oracle.slab_error(to_f64(z).reshape(N, 1, d), z_ref[:, None, :], 1) <= TOL["bf16"]
