"""Pins of the oracle's normalized linear attention (phi = elu + 1) to what the
pages and the mathematics fix.

The pins take the function under test as a callable, so the same checks also
run on test-local copies with a planted mistake (each must fail a pin).
"""

import math

import numpy as np
import pytest

import oracle


def _heads(seed, N=3, L=29, dk=8, dv=5, scale=1.5):
    r = np.random.default_rng(seed)
    return (r.standard_normal((N, L, dk)) * scale, r.standard_normal((N, L, dk)) * scale,
            r.standard_normal((N, L, dv)))


def _la(f, q, k, v, S0=None, z0=None):
    return f(q, k, v, S0, z0, qkv_dtype="f64")


# ---------------------------------------------------------------------------
# pins, each a function of (feature map, linear attention) under test
# ---------------------------------------------------------------------------

def pin_feature_map(phi, f):
    """phi(0) = 1, phi(x) = x + 1 above 0 and e^x below, continuous, positive."""
    x = np.array([0.0, 2.0, -1.0, 1e-9, -1e-9, -30.0, 5.5])
    y = phi(x)
    assert y[0] == 1.0 and y[1] == 3.0 and abs(y[2] - math.exp(-1.0)) < 1e-16
    assert abs(y[3] - y[4]) < 1e-8
    assert np.all(y > 0) and abs(y[6] - 6.5) < 1e-15


def pin_first_token(phi, f):
    """From a zero state the first output is the first value exactly."""
    q, k, v = _heads(1)
    o, _, _ = _la(f, q, k, v)
    assert np.allclose(o[:, 0], v[:, 0], rtol=0, atol=1e-14)


def pin_constant_values(phi, f):
    """The output is a weighted average of the values seen so far: constant
    values come back unchanged at every step."""
    q, k, v = _heads(2)
    v[:] = np.array([0.5, -2.0, 3.0, 0.0, 1.25])
    o, _, _ = _la(f, q, k, v)
    assert np.allclose(o, v, rtol=0, atol=1e-13)


def pin_convex_hull(phi, f):
    """From a zero state, o_t lies between the smallest and largest v_s, s <= t
    (weights phi(q_t) . phi(k_s) are positive and sum to one after dividing)."""
    q, k, v = _heads(3, L=40)
    o, _, _ = _la(f, q, k, v)
    lo = np.minimum.accumulate(v, axis=1)
    hi = np.maximum.accumulate(v, axis=1)
    assert np.all(o >= lo - 1e-12) and np.all(o <= hi + 1e-12)


def pin_quadratic_form(phi, f):
    """The causal attention form: o = (M V + phi(Q) S0) / (M 1 + phi(Q) z0)
    with M_ts = phi(q_t) . phi(k_s) for s <= t (the pages' phi(Q)(phi(K)^T V)
    with a causal mask), a different evaluation order."""
    q, k, v = _heads(4, L=33)
    r = np.random.default_rng(44)
    S0 = r.standard_normal((3, 8, 5))
    z0 = r.uniform(0.5, 2.0, (3, 8))
    o, S, z = _la(f, q, k, v, S0, z0)
    fq, fk = oracle.elu1(q), oracle.elu1(k)
    for n in range(3):
        M = np.tril(fq[n] @ fk[n].T)
        num = M @ v[n] + fq[n] @ S0[n]
        den = M.sum(1) + fq[n] @ z0[n]
        assert np.allclose(o[n], num / den[:, None], rtol=1e-12, atol=1e-12)
        assert np.allclose(S[n], S0[n] + fk[n].T @ v[n], rtol=1e-12, atol=1e-12)
        assert np.allclose(z[n], z0[n] + fk[n].sum(0), rtol=1e-12, atol=1e-12)


def pin_one_step(phi, f):
    """One token from a given (S, z) is the pages' recurrent step: write, then
    read phi(q) S / (phi(q) . z)."""
    r = np.random.default_rng(5)
    q, k, v = r.standard_normal((1, 1, 6)), r.standard_normal((1, 1, 6)), r.standard_normal((1, 1, 4))
    S0, z0 = r.standard_normal((1, 6, 4)), r.uniform(1.0, 3.0, (1, 6))
    o, S, z = _la(f, q, k, v, S0, z0)
    fq, fk = oracle.elu1(q[0, 0]), oracle.elu1(k[0, 0])
    S1 = S0[0] + np.outer(fk, v[0, 0])
    z1 = z0[0] + fk
    assert np.allclose(o[0, 0], fq @ S1 / (fq @ z1), rtol=1e-13, atol=1e-13)


def pin_split(phi, f):
    """Chaining (S, z) across a split of the sequence changes nothing."""
    q, k, v = _heads(6, L=31)
    o, S, z = _la(f, q, k, v)
    o1, S1, z1 = _la(f, q[:, :12], k[:, :12], v[:, :12])
    o2, S2, z2 = _la(f, q[:, 12:], k[:, 12:], v[:, 12:], S1, z1)
    assert np.allclose(np.concatenate([o1, o2], axis=1), o, rtol=1e-12, atol=1e-13)
    assert np.allclose(S2, S, rtol=1e-12, atol=1e-13) and np.allclose(z2, z, rtol=1e-12)


PINS = [pin_feature_map, pin_first_token, pin_constant_values, pin_convex_hull,
        pin_quadratic_form, pin_one_step, pin_split]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_linear_attention_pin(pin, oracle_lib):
    pin(oracle.elu1, oracle.linear_attention)


def test_bf16_inputs_are_widened(oracle_lib):
    """bf16 storage is widened exactly before phi."""
    from linear_attention_sequence_kda_amd import inputs as gen
    q, k, v = _heads(7, N=2, L=9)
    qb, kb, vb = (gen.f32_to_bf16_bits(x.astype(np.float32)) for x in (q, k, v))
    o1, S1, z1 = oracle.linear_attention(qb, kb, vb, qkv_dtype="bf16")
    w = lambda x: gen.bf16_bits_to_f32(x).astype(np.float64)
    o2, S2, z2 = oracle.linear_attention(w(qb), w(kb), w(vb), qkv_dtype="f64")
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2) and np.array_equal(z1, z2)


# ---------------------------------------------------------------------------
# planted mistakes in test-local copies
# ---------------------------------------------------------------------------

def _mutant(which):
    def phi(x):
        x = np.asarray(x, dtype=np.float64)
        if which == "elu_without_one":
            return np.where(x > 0, x, np.exp(np.minimum(x, 0.0)) - 1.0)
        if which == "relu_map":
            return np.maximum(x, 0.0) + 1e-6
        if which == "exp_both_sides":
            return np.exp(np.minimum(x, 30.0))
        return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))

    def la(q, k, v, S0=None, z0=None, *, qkv_dtype="f64"):
        q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
        N, L, dk = q.shape
        dv = v.shape[-1]
        S = np.zeros((N, dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
        z = np.zeros((N, dk)) if z0 is None else np.array(z0, dtype=np.float64)
        o = np.zeros((N, L, dv))
        fq = phi(v if which == "phi_on_values" else q)
        fk = phi(k)
        for t in range(L):
            if which == "read_before_write":
                num = np.einsum("nd,nde->ne", fq[:, t], S)
                den = np.einsum("nd,nd->n", fq[:, t], z)
            S = S + np.einsum("nd,ne->nde", fk[:, t], v[:, t])
            if which != "normalizer_frozen":
                z = z + fk[:, t]
            if which != "read_before_write":
                num = np.einsum("nd,nde->ne", fq[:, t], S)
                den = np.einsum("nd,nd->n", fq[:, t], z)
            if which == "no_normalizer":
                den = np.ones_like(den)
            elif which == "normalizer_uses_k":
                den = np.einsum("nd,nd->n", fk[:, t], z)
            o[:, t] = num / np.where(den == 0, 1.0, den)[:, None]
        return o, S, z
    return phi, la


MUTATIONS = ["elu_without_one", "relu_map", "exp_both_sides", "read_before_write",
             "normalizer_frozen", "no_normalizer", "normalizer_uses_k"]


@pytest.mark.parametrize("which", MUTATIONS)
def test_linear_attention_mutation_caught(which, oracle_lib):
    phi, la = _mutant(which)
    failed = []
    with np.errstate(all="ignore"):
        for pin in PINS:
            try:
                pin(phi, la)
            except AssertionError:
                failed.append(pin.__name__)
    assert failed, f"no pin catches the planted mistake {which}"


def test_unmutated_copy_passes(oracle_lib):
    phi, la = _mutant("none")
    for pin in PINS:
        pin(phi, la)
