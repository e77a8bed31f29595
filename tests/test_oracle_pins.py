"""Pins of the CPU oracle to what the pages and the mathematics fix.

None of these compare the oracle with itself: each checks a hand-worked value,
a closed form, an invariant, a special case that reduces to a simpler textbook
computation, or a second evaluation order.
"""

import json
import os

import numpy as np
import pytest

import oracle
from linear_attention_sequence_kda_amd import inputs as gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "handworked_d2.json")


def _rng(seed):
    return np.random.default_rng(seed)


def _unit(rng, n, d):
    x = rng.standard_normal((n, d))
    return x / np.linalg.norm(x, axis=1, keepdims=True)


def _orthonormal(rng, n, d):
    """n <= d mutually orthonormal rows."""
    qm, _ = np.linalg.qr(rng.standard_normal((d, n)))
    return qm.T.copy()


def _rand_head(seed, L=37, dk=8, dv=6, mode="channel", s0=True, la_scale=0.3):
    rng = _rng(seed)
    q = _unit(rng, L, dk)
    k = _unit(rng, L, dk)
    v = rng.standard_normal((L, dv))
    if mode == "channel":
        la = -la_scale * rng.random((L, dk))
    elif mode == "head":
        la = -la_scale * rng.random(L)
    else:
        la = None
    beta = rng.random(L)
    S0 = rng.standard_normal((dk, dv)) * 0.5 if s0 else None
    return q, k, v, la, beta, S0


def _c_forward(q, k, v, la, beta, S0, mode, delta=True):
    """Run the C oracle on fp64 test data stored as fp32 (values chosen fp32-exact
    where it matters)."""
    f = lambda x: None if x is None else np.asarray(x, dtype=np.float32)[None]
    o, sf = oracle.forward(f(q), f(k), f(v), f(la), f(beta),
                           None if S0 is None else np.asarray(S0)[None],
                           alpha_mode=mode, delta=delta, threads=2)
    return o[0], sf[0]


# ---------------------------------------------------------------------------
# hand-worked values (tests/golden)
# ---------------------------------------------------------------------------

def _golden_cases():
    with open(GOLDEN) as fh:
        return json.load(fh)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_handworked_numpy(case):
    arr = lambda key: None if case[key] is None else np.array(case[key], dtype=np.float64)
    o, S = oracle.recurrence(arr("q"), arr("k"), arr("v"), arr("log_alpha"), arr("beta"), arr("S0"))
    np.testing.assert_allclose(o, case["o"], rtol=0, atol=1e-13)
    np.testing.assert_allclose(S, case["S_final"], rtol=0, atol=1e-13)
    if "rejected_reading" in case:
        assert abs(o[-1] - np.array(case["rejected_reading"]["o_last"])).max() > 0.1


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_handworked_c_oracle(case, oracle_lib):
    arr = lambda key: None if case[key] is None else np.array(case[key], dtype=np.float64)
    o, S = _c_forward(arr("q"), arr("k"), arr("v"), arr("log_alpha"), arr("beta"), arr("S0"),
                      case["alpha_mode"])
    # inputs such as 0.6 are rounded to fp32 on the way in: 1e-6 covers that
    np.testing.assert_allclose(o, case["o"], rtol=0, atol=1e-6)
    np.testing.assert_allclose(S, case["S_final"], rtol=0, atol=1e-6)


# ---------------------------------------------------------------------------
# P1: exact replacement (unit key, beta = 1, q = k  =>  o_t = v_t)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("mode", ["none", "head", "channel"])
def test_exact_replacement(mode, oracle_lib):
    q, k, v, la, beta, S0 = _rand_head(11, L=40, dk=16, dv=5, mode=mode, la_scale=2.0)
    beta = np.ones_like(beta)
    q = k.copy()
    o, _ = oracle.recurrence(q, k, v, la, beta, S0)
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-12)
    oc, _ = _c_forward(q, k, v, la, beta, S0, mode)
    # C path: inputs rounded to fp32, so k is unit only to ~1e-7
    np.testing.assert_allclose(oc, v.astype(np.float32), rtol=0, atol=2e-5)


# ---------------------------------------------------------------------------
# P2: orthonormal keys reduce the delta rule to linear attention
# ---------------------------------------------------------------------------

def test_orthonormal_keys_linear_attention():
    rng = _rng(3)
    L, dk, dv = 12, 16, 7
    k = _orthonormal(rng, L, dk)
    q = rng.standard_normal((L, dk))
    v = rng.standard_normal((L, dv))
    beta = rng.random(L)
    o, _ = oracle.recurrence(q, k, v, None, beta)
    ref = np.tril(q @ k.T) @ (beta[:, None] * v)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


def test_associative_recall():
    """Write orthonormal keys once each (beta = 1), then read each back."""
    rng = _rng(4)
    n, dk, dv = 10, 16, 9
    keys = _orthonormal(rng, n, dk)
    vals = rng.standard_normal((n, dv))
    q = np.vstack([keys, keys[::-1]])                  # reads during and after writing
    k = np.vstack([keys, np.zeros((n, dk))])           # zero keys: pure reads
    v = np.vstack([vals, np.zeros((n, dv))])
    beta = np.ones(2 * n)
    o, _ = oracle.recurrence(q, k, v, None, beta)
    np.testing.assert_allclose(o[:n], vals, rtol=0, atol=1e-12)
    np.testing.assert_allclose(o[n:], vals[::-1], rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# P3: no-delta additive mode, alpha = 1, beta = 1: o = Q S0 + tril(Q K^T) V
# ---------------------------------------------------------------------------

def test_additive_mode_linear_attention(oracle_lib):
    q, k, v, _, _, S0 = _rand_head(5, L=23, dk=8, dv=6, mode="none")
    beta = np.ones(23)
    o, S = oracle.recurrence(q, k, v, None, beta, S0, delta=False)
    ref = q @ S0 + np.tril(q @ k.T) @ v
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(S, S0 + k.T @ v, rtol=0, atol=1e-12)
    oc, Sc = _c_forward(q, k, v, None, beta, S0, "none", delta=False)
    q32, k32, v32 = (x.astype(np.float32).astype(np.float64) for x in (q, k, v))
    np.testing.assert_allclose(oc, q32 @ S0 + np.tril(q32 @ k32.T) @ v32, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# P4: zero inputs keep S0 bit for bit
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("mode", ["none", "head", "channel"])
def test_zero_inputs_keep_state(mode, oracle_lib):
    L, dk, dv = 9, 8, 8
    S0 = _rng(6).standard_normal((dk, dv))
    z = np.zeros((L, dk))
    la = None if mode == "none" else (np.zeros((L, dk)) if mode == "channel" else np.zeros(L))
    o, S = oracle.recurrence(z, z, np.zeros((L, dv)), la, _rng(7).random(L), S0)
    assert np.all(o == 0) and np.array_equal(S, S0)
    oc, Sc = _c_forward(z, z, np.zeros((L, dv)), la, _rng(7).random(L), S0, mode)
    assert np.all(oc == 0) and np.array_equal(Sc, S0)


# ---------------------------------------------------------------------------
# P5: beta = 0 is pure decay along the key (row) axis
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("mode", ["head", "channel"])
def test_pure_decay(mode, oracle_lib):
    q, k, v, la, _, S0 = _rand_head(8, L=30, dk=8, dv=8, mode=mode, la_scale=0.5)
    beta = np.zeros(30)
    o, S = oracle.recurrence(q, k, v, la, beta, S0)
    la2 = la if la.ndim == 2 else np.repeat(la[:, None], 8, axis=1)
    g = np.cumsum(la2, axis=0)
    ref_o = (q * np.exp(g)) @ S0
    np.testing.assert_allclose(o, ref_o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(S, np.exp(g[-1])[:, None] * S0, rtol=0, atol=1e-12)
    oc, Sc = _c_forward(q, k, v, la, beta, S0, mode)
    la32 = la2.astype(np.float32).astype(np.float64)
    q32 = q.astype(np.float32).astype(np.float64)
    g32 = np.cumsum(la32, axis=0)
    np.testing.assert_allclose(oc, (q32 * np.exp(g32)) @ S0, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# P6: alpha -> 0 wipes memory (a context switch at every token)
# ---------------------------------------------------------------------------

def test_wipe(oracle_lib):
    q, k, v, _, beta, S0 = _rand_head(9, L=20, dk=8, dv=5, mode="channel")
    la = np.full((20, 8), -1e3)
    o, S = oracle.recurrence(q, k, v, la, beta, S0)
    ref = (beta * np.sum(q * k, axis=1))[:, None] * v
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(S, beta[-1] * np.outer(k[-1], v[-1]), rtol=0, atol=1e-12)
    oc, _ = _c_forward(q, k, v, la, beta, S0, "channel")
    f = lambda x: x.astype(np.float32).astype(np.float64)
    np.testing.assert_allclose(oc, (f(beta) * np.sum(f(q) * f(k), axis=1))[:, None] * f(v),
                               rtol=0, atol=1e-12)


def test_context_switch_partial():
    """Channels with alpha = 0 forget, channels with alpha = 1 keep (beta = 0)."""
    dk, dv = 6, 4
    S0 = _rng(10).standard_normal((dk, dv))
    la = np.zeros((1, dk))
    la[0, :3] = -1e3
    q = np.eye(dk)[:1] * 0
    o, S = oracle.recurrence(np.zeros((1, dk)), np.zeros((1, dk)), np.zeros((1, dv)), la,
                             np.zeros(1), S0)
    assert np.all(S[:3] == 0) and np.array_equal(S[3:], S0[3:])


# ---------------------------------------------------------------------------
# P7: alpha = 1 equals the pages' printed chunk algorithm
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("C", [4, 16, 32])
def test_pages_chunk_algorithm(C):
    q, k, v, _, beta, _ = _rand_head(12, L=64, dk=16, dv=8, mode="none", s0=False)
    o_ref, S_ref = oracle.recurrence(q, k, v, None, beta)
    o, S = oracle.pages_chunk_deltanet(q, k, v, beta, C)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(S, S_ref, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# P8: repeated key -- the second write replaces the first
# ---------------------------------------------------------------------------

def test_repeated_key():
    rng = _rng(13)
    dk, dv = 8, 5
    kk = _unit(rng, 1, dk)[0]
    other = rng.standard_normal(dk)
    other -= (other @ kk) * kk                      # orthogonal to the repeated key
    S0 = rng.standard_normal((dk, dv))
    v1, v2 = rng.standard_normal(dv), rng.standard_normal(dv)
    q = np.vstack([kk, kk])
    k = np.vstack([kk, kk])
    v = np.vstack([v1, v2])
    o, S = oracle.recurrence(q, k, v, None, np.ones(2), S0)
    np.testing.assert_allclose(o[1], v2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(kk @ S, v2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(other @ S, other @ S0, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# P9: chunkwise form equals the recurrence for any chunk size, ragged tails
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("C", [1, 2, 4, 16, 64])
@pytest.mark.parametrize("L", [1, 7, 64, 65, 130])
@pytest.mark.parametrize("mode", ["none", "head", "channel"])
def test_chunk_equals_recurrence(C, L, mode):
    q, k, v, la, beta, S0 = _rand_head(100 + L + C, L=L, dk=8, dv=6, mode=mode)
    o_ref, S_ref = oracle.recurrence(q, k, v, la, beta, S0)
    o, S = oracle.chunk_reference(q, k, v, la, beta, S0, C=C)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(S, S_ref, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# P10: forward substitution inverts (I + A)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("C", [2, 16, 64])
def test_forward_substitution_inverts(C):
    rng = _rng(C)
    A = np.tril(rng.standard_normal((C, C)) * 0.3, -1)
    T = oracle.forward_substitution(A)
    np.testing.assert_allclose(T @ (np.eye(C) + A), np.eye(C), rtol=0, atol=1e-12)
    assert np.array_equal(np.triu(T, 1), np.zeros((C, C)))
    assert np.array_equal(np.diag(T), np.ones(C))


# ---------------------------------------------------------------------------
# P11: brute force with explicit transition matrices
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("mode", ["none", "head", "channel"])
def test_brute_force(mode, oracle_lib):
    q, k, v, la, beta, S0 = _rand_head(14, L=25, dk=6, dv=4, mode=mode)
    o_b, S_b = oracle.brute_force(q, k, v, la, beta, S0)
    o, S = oracle.recurrence(q, k, v, la, beta, S0)
    np.testing.assert_allclose(o, o_b, rtol=0, atol=1e-12)
    np.testing.assert_allclose(S, S_b, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# P12: state passing -- a split sequence continues exactly; decode steps chain
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("split", [1, 13, 39])
def test_state_passing_bitwise(split, oracle_lib):
    w = gen.custom(B=1, H=2, L=40, dk=16, dv=16, qkv_dtype=gen.BF16, gate_dtype=gen.BF16,
                   alpha_mode=gen.ALPHA_CHANNEL, seed=77)
    x = gen.prefill_inputs(w)
    r = lambda a: a.reshape((2,) + a.shape[2:])
    q, k, v, la, beta, S0 = (r(x[n]) for n in ("q", "k", "v", "log_alpha", "beta", "S0"))
    kw = dict(qkv_dtype="bf16", gate_dtype="bf16", alpha_mode="channel", threads=3)
    o_full, S_full = oracle.forward(q, k, v, la, beta, S0, **kw)
    o1, S_mid = oracle.forward(q[:, :split], k[:, :split], v[:, :split], la[:, :split],
                               beta[:, :split], S0, **kw)
    o2, S_end = oracle.forward(q[:, split:], k[:, split:], v[:, split:], la[:, split:],
                               beta[:, split:], S_mid, **kw)
    assert np.array_equal(np.concatenate([o1, o2], axis=1), o_full)
    assert np.array_equal(S_end, S_full)
    # token-at-a-time (decode) chaining
    S = S0.astype(np.float64)
    outs = []
    for t in range(40):
        sl = slice(t, t + 1)
        ot, S = oracle.forward(q[:, sl], k[:, sl], v[:, sl], la[:, sl], beta[:, sl], S, **kw)
        outs.append(ot)
    assert np.array_equal(np.concatenate(outs, axis=1), o_full)
    assert np.array_equal(S, S_full)


# ---------------------------------------------------------------------------
# P13: C oracle = NumPy recurrence; column slicing and threads change nothing
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("qd,gd,mode", [("f32", "f32", "none"), ("bf16", "f32", "head"),
                                         ("bf16", "bf16", "channel"), ("f32", "bf16", "channel")])
def test_c_oracle_matches_numpy(qd, gd, mode, oracle_lib):
    w = gen.custom(B=2, H=2, L=70, dk=16, dv=48, qkv_dtype=qd, gate_dtype=gd,
                   alpha_mode=mode, seed=5)
    x = gen.prefill_inputs(w)
    N = 4
    r = lambda a: None if a is None else a.reshape((N,) + a.shape[2:])
    q, k, v, la, beta, S0 = (r(x[n]) for n in ("q", "k", "v", "log_alpha", "beta", "S0"))
    kw = dict(qkv_dtype=qd, gate_dtype=gd, alpha_mode=mode)
    o, S = oracle.forward(q, k, v, la, beta, S0, threads=1, **kw)
    o4, S4 = oracle.forward(q, k, v, la, beta, S0, threads=4, **kw)
    assert np.array_equal(o, o4) and np.array_equal(S, S4)
    oc, Sc = oracle.forward(q, k, v, la, beta, S0, col0=16, ncols=20, threads=3, **kw)
    assert np.array_equal(oc, o[..., 16:36]) and np.array_equal(Sc, S[..., 16:36])
    for n in range(N):
        wide = lambda a, dt: gen.widen(a[n], dt) if a is not None else None
        o_np, S_np = oracle.recurrence(wide(q, qd), wide(k, qd), wide(v, qd), wide(la, gd),
                                       wide(beta, gd), S0[n].astype(np.float64))
        np.testing.assert_allclose(o[n], o_np, rtol=0, atol=1e-12 * max(1, np.abs(o_np).max()))
        np.testing.assert_allclose(S[n], S_np, rtol=0, atol=1e-12 * max(1, np.abs(S_np).max()))


# ---------------------------------------------------------------------------
# P14: the transition is non-expansive (long-sequence stability)
# ---------------------------------------------------------------------------

def test_state_norm_bound():
    q, k, v, la, beta, S0 = _rand_head(15, L=400, dk=8, dv=6, mode="channel", la_scale=0.05)
    S = S0.copy()
    for t in range(400):
        prev = np.linalg.norm(S)
        _, S = oracle.recurrence(q[t:t + 1], k[t:t + 1], v[t:t + 1], la[t:t + 1],
                                 beta[t:t + 1], S)
        assert np.linalg.norm(S) <= prev + beta[t] * np.linalg.norm(v[t]) + 1e-12


# ---------------------------------------------------------------------------
# P15: scalar gate == per-channel gate with equal channels (bitwise)
# ---------------------------------------------------------------------------

def test_head_mode_equals_equal_channels(oracle_lib):
    q, k, v, la, beta, S0 = _rand_head(16, L=33, dk=8, dv=8, mode="head")
    la_c = np.repeat(la[:, None], 8, axis=1)
    a = _c_forward(q, k, v, la, beta, S0, "head")
    b = _c_forward(q, k, v, la_c, beta, S0, "channel")
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ---------------------------------------------------------------------------
# the parity metric itself
# ---------------------------------------------------------------------------

def test_slab_error_metric():
    ref = np.zeros((2, 3, 4))
    ref[0] = 2.0
    ref[1] = 4.0
    x = ref.copy()
    x[1, 0, 0] += 0.4
    assert oracle.slab_error(x, ref, slab_axes=1) == pytest.approx(0.1)
    x[0, 2, 3] = np.nan
    assert oracle.slab_error(x, ref, slab_axes=1) == float("inf")
