"""Parity of kda_chunk_fwd_varlen (packed variable-length sequences, through
the C ABI) with the fp64 oracle run on each sequence alone.

Each sequence is drawn with the workload recipe on its own seed, packed along
the token axis of [H, T, d] tensors, and compared slab by slab (per sequence
and head) with the oracle's recurrence over that sequence: 1e-4 for fp32
inputs, 2e-2 for bf16 inputs, as for the dense entry point.
"""

import numpy as np
import pytest

import oracle
from linear_attention_sequence_kda_amd import inputs as gen

from gpu_util import TOL, flat_heads, oracle_prefill, say, to_dev, to_f64

pytestmark = pytest.mark.gpu

ALL = oracle.NORM_QK | oracle.BETA_LOGIT | oracle.GATE_RAW


def _kda():
    import linear_attention_sequence_kda_amd as kda
    return kda


def packed_inputs(lens, H, dk, dv, qd, gd, mode, s0=True, seed=0, raw=False):
    """Per-sequence draws (one workload of B = 1 each) and their packing."""
    seqs = []
    for i, L in enumerate(lens):
        w = gen.custom(B=1, H=H, L=L, dk=dk, dv=dv, qkv_dtype=qd, gate_dtype=gd,
                       alpha_mode=mode, s0_std=0.02 if s0 else None, seed=seed * 1000 + i)
        seqs.append((w, gen.prefill_inputs(w, raw=raw)))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    packed = {}
    for key in ("q", "k", "v", "log_alpha", "beta"):
        if seqs[0][1][key] is None:
            packed[key] = None
            continue
        packed[key] = np.ascontiguousarray(np.concatenate([x[key][0] for _, x in seqs], axis=1))
    if s0:
        packed["S0"] = np.ascontiguousarray(np.concatenate([x["S0"] for _, x in seqs], axis=0))
    else:
        packed["S0"] = None
    return seqs, cu, packed


def run_varlen(lens, H=4, dk=128, dv=128, qd="bf16", gd="bf16", mode="channel", s0=True,
               seed=0, flags=0, final_state=True, max_seqlen=None, label="varlen"):
    import torch
    kda = _kda()
    seqs, cu, x = packed_inputs(lens, H, dk, dv, qd, gd, mode, s0, seed, raw=flags != 0)
    dq = lambda n: to_dev(x[n], qd if n in ("q", "k", "v") else gd)
    d = {n: dq(n) for n in ("q", "k", "v", "log_alpha", "beta")}
    S0 = to_dev(x["S0"], "f32") if x["S0"] is not None else None
    cu_d = torch.from_numpy(cu).to("cuda:0")
    m = max(lens) if max_seqlen is None else max_seqlen
    say(f"{label}: varlen lens={lens} H={H} dk={dk} dv={dv} {qd}/{gd}/{mode} flags={flags} "
        f"S0={s0} final={final_state} max={m}")
    o, Sf = kda.chunk_fwd_varlen(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], cu_d, m,
                                 S0, output_final_state=final_state, flags=flags)
    torch.cuda.synchronize()
    og = to_f64(o)
    sg = to_f64(Sf) if final_state else None
    tol = TOL[qd]
    worst = 0.0
    for i, (w, xi) in enumerate(seqs):
        xf = flat_heads(xi, H)
        if flags:
            qq, kk, vv, la, bb = oracle.preprocess(xf["q"], xf["k"], xf["v"], xf["log_alpha"],
                                                   xf["beta"], flags, qkv_dtype=qd,
                                                   gate_dtype=gd)
            o_ref, S_ref = oracle.forward(qq, kk, vv, la, bb, xf["S0"], qkv_dtype="f64",
                                          gate_dtype="f64", alpha_mode=mode)
        else:
            o_ref, S_ref = oracle_prefill(w, xf)
        L = lens[i]
        if L:
            e_o = oracle.slab_error(og[:, cu[i]:cu[i + 1]], o_ref, 1)
            worst = max(worst, e_o)
            assert e_o <= tol, f"sequence {i}: o error {e_o}"
        if final_state:
            e_s = oracle.slab_error(sg[i], S_ref, 1)
            worst = max(worst, e_s)
            assert e_s <= tol, f"sequence {i}: S_final error {e_s}"
    say(f"{label}: worst err {worst:.3e} (tol {tol})")
    return o, Sf


@pytest.mark.parametrize("qd,gd,mode", [("bf16", "bf16", "channel"), ("bf16", "f32", "head"),
                                        ("f32", "f32", "none"), ("f32", "f32", "channel")],
                         ids=lambda x: str(x))
@pytest.mark.parametrize("lens", [[1, 64, 65, 130], [200, 0, 37, 64, 1], [129]],
                         ids=lambda x: "-".join(map(str, x)))
def test_varlen_small(qd, gd, mode, lens):
    run_varlen(lens, qd=qd, gd=gd, mode=mode, seed=len(lens))


@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64)])
def test_varlen_dims(dk, dv):
    run_varlen([100, 7, 300], H=3, dk=dk, dv=dv, mode="channel", seed=dk + dv)
    run_varlen([100, 7, 300], H=3, dk=dk, dv=dv, qd="bf16", gd="f32", mode="head",
               seed=dk + dv + 1)


@pytest.mark.parametrize("mode,final", [("channel", True), ("channel", False),
                                        ("head", False)])
def test_varlen_several_spans(mode, final):
    """Lengths long enough for several record spans (5 with per-channel decay,
    2 with one decay per token): the short sequence ends in the first span and
    must pass its state through the later ones."""
    lens = [4000, 700, 2500] if mode == "channel" else [8000, 700, 2500]
    run_varlen(lens, H=32, mode=mode, gd="bf16" if mode == "channel" else "f32",
               final_state=final, seed=7)


def test_varlen_no_initial_state_and_slack_max():
    """No S0 (zero state) and a max_seqlen above the longest sequence."""
    run_varlen([90, 300, 5], H=8, s0=False, max_seqlen=700, seed=3)


@pytest.mark.parametrize("mode", ["channel", "head"])
def test_varlen_raw_inputs(mode):
    run_varlen([150, 64, 1, 333], H=4, qd="bf16", gd="bf16" if mode == "channel" else "f32",
               mode=mode, flags=ALL, seed=11)


@pytest.mark.parametrize("qd,gd,mode", [("bf16", "bf16", "channel"), ("bf16", "f32", "head"),
                                        ("f32", "f32", "none")], ids=lambda x: str(x))
def test_varlen_equal_lengths_is_dense(qd, gd, mode):
    """Equal lengths pack the same work as a dense [N, H, L] call with the same
    launch plan: the results agree bit for bit."""
    import torch
    kda = _kda()
    N, H, L = 3, 8, 333
    w = gen.custom(B=N, H=H, L=L, dk=128, dv=128, qkv_dtype=qd, gate_dtype=gd, alpha_mode=mode,
                   seed=21)
    x = gen.prefill_inputs(w)
    dt = lambda n: qd if n in ("q", "k", "v") else gd
    dense = {n: to_dev(x[n], dt(n)) for n in ("q", "k", "v", "log_alpha", "beta")}
    S0 = to_dev(x["S0"], "f32")
    # [N, H, L, d] -> [H, N L, d]
    pk = {n: (None if t is None else t.transpose(0, 1).reshape((H, N * L) + t.shape[3:])
              .contiguous()) for n, t in dense.items()}
    cu = torch.arange(0, N * L + 1, L, dtype=torch.int32, device="cuda:0")
    say(f"varlen equal lengths vs dense {qd}/{gd}/{mode}")
    o1, s1 = kda.chunk_fwd(dense["q"], dense["k"], dense["v"], dense["log_alpha"],
                           dense["beta"], S0)
    o2, s2 = kda.chunk_fwd_varlen(pk["q"], pk["k"], pk["v"], pk["log_alpha"], pk["beta"], cu,
                                  L, S0)
    torch.cuda.synchronize()
    assert torch.equal(o2, o1.transpose(0, 1).reshape(H, N * L, 128))
    assert torch.equal(s2, s1)


def test_varlen_prefill_then_slot_decode():
    """Serving loop: packed prefill of three prompts into a state pool, then
    decode steps on the pool by slot; every output against the oracle run over
    prompt + generated tokens of each sequence."""
    import torch
    kda = _kda()
    H, lens, steps = 4, [77, 130, 5], 4
    seqs, cu, x = packed_inputs(lens, H, 128, 128, "bf16", "f32", "channel", True, seed=31)
    dq = lambda n: to_dev(x[n], "bf16" if n in ("q", "k", "v") else "f32")
    d = {n: dq(n) for n in ("q", "k", "v", "log_alpha", "beta")}
    S0 = to_dev(x["S0"], "f32")
    cu_d = torch.from_numpy(cu).to("cuda:0")
    say("varlen prefill -> slot decode")
    # pool of 5 slots; the three sequences live in slots 4, 0, 2
    slots_h = [4, 0, 2]
    pool = torch.zeros((5, H, 128, 128), dtype=torch.float32, device="cuda:0")
    _, Sf = kda.chunk_fwd_varlen(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], cu_d,
                                 max(lens), S0)
    pool[slots_h] = Sf
    slots = torch.tensor(slots_h, dtype=torch.int32, device="cuda:0")
    wd = gen.custom(B=3, H=H, L=1, dk=128, dv=128, qkv_dtype="bf16", gate_dtype="f32",
                    alpha_mode="channel", seed=32).replace(decode_steps=steps)
    outs, dec = [], []
    for t in range(steps):
        xt = gen.decode_inputs(wd, t)
        dec.append(xt)
        dd = [to_dev(xt[n], "bf16" if n in ("q", "k", "v") else "f32")
              for n in ("q", "k", "v", "log_alpha", "beta")]
        outs.append(to_f64(kda.decode_step_slots(*dd, pool, slots)))
    torch.cuda.synchronize()
    for i, (w, xi) in enumerate(seqs):
        cat = lambda key: np.concatenate(
            [xi[key][0]] + [p[key][i][:, None] for p in dec], axis=1)
        o_ref, S_ref = oracle.forward(cat("q"), cat("k"), cat("v"), cat("log_alpha"),
                                      cat("beta"), xi["S0"][0], qkv_dtype="bf16",
                                      gate_dtype="f32", alpha_mode="channel")
        og = np.stack([o[i] for o in outs], axis=1)  # [H, steps, dv]
        assert oracle.slab_error(og, o_ref[:, lens[i]:], 1) <= TOL["bf16"]
        assert oracle.slab_error(to_f64(pool[slots_h[i]]), S_ref, 1) <= TOL["bf16"]


def _sweep_cases(n=10, seed=20261205):
    """Seeded random packings: 1-40 sequences of lengths drawn from a long-tailed
    mix (empty, single tokens, a chunk and one more, a few thousand), random
    head counts, head sizes, dtypes and decay modes, with and without S0."""
    rng = np.random.default_rng(seed)
    modes = [("bf16", "bf16", "channel"), ("bf16", "f32", "head"), ("f32", "f32", "none"),
             ("f32", "f32", "channel"), ("bf16", "bf16", "none"), ("f32", "bf16", "head")]
    dims = [(64, 64), (128, 128), (64, 128), (128, 64)]
    cases = []
    for i in range(n):
        nseq = int(rng.integers(1, 41))
        lens = [int(x) for x in np.minimum(rng.lognormal(4.0, 1.5, nseq).astype(np.int64), 3000)]
        lens[int(rng.integers(nseq))] = [0, 1, 65][int(rng.integers(3))]
        qd, gd, mode = modes[i % len(modes)]
        dk, dv = dims[rng.integers(len(dims))]
        H = int(rng.integers(1, 9))
        cases.append((i, lens, H, dk, dv, qd, gd, mode, bool(rng.integers(2))))
    return cases


@pytest.mark.parametrize("case", _sweep_cases(), ids=lambda c: f"sweep{c[0]}")
def test_varlen_random_sweep(case):
    i, lens, H, dk, dv, qd, gd, mode, s0 = case
    run_varlen(lens, H=H, dk=dk, dv=dv, qd=qd, gd=gd, mode=mode, s0=s0, seed=900 + i,
               label=f"varlen-sweep{i}")
