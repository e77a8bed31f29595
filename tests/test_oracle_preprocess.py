"""Pins of the oracle's input preprocessing (L2-normalized q and k, sigmoid
beta, alpha = exp(-exp(g))) to what the pages and the mathematics fix.

The pins take the preprocessing as a callable, so the same checks also run on
test-local copies with a planted mistake (each must fail at least one pin).
"""

import numpy as np
import pytest
from scipy.special import expit

import oracle
from linear_attention_sequence_kda_amd import inputs as gen

ALL = oracle.NORM_QK | oracle.BETA_LOGIT | oracle.GATE_RAW


def _raw_head(seed, L=23, dk=8, dv=5, mode="channel"):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((L, dk)) * rng.uniform(0.05, 20.0, (L, 1))
    k = rng.standard_normal((L, dk)) * rng.uniform(0.05, 20.0, (L, 1))
    v = rng.standard_normal((L, dv))
    g = rng.normal(-2.0, 1.0, (L, dk) if mode == "channel" else (L,))
    if mode == "none":
        g = None
    b = rng.normal(0.0, 2.0, L)
    return q, k, v, g, b


def _run(pre, q, k, v, g, b, flags, mode, S0=None):
    """preprocess + the C recurrence on one head (inputs fp64, stored as f64)."""
    qq, kk, vv, la, bb = pre(q, k, v, g, b, flags, qkv_dtype="f64", gate_dtype="f64")
    f = lambda x: None if x is None else np.ascontiguousarray(x, dtype=np.float64)[None]
    o, sf = oracle.forward(f(qq), f(kk), f(vv), f(la), f(bb),
                           None if S0 is None else np.asarray(S0)[None],
                           qkv_dtype="f64", gate_dtype="f64", alpha_mode=mode, threads=2)
    return o[0], sf[0]


# ---------------------------------------------------------------------------
# pins, each a function of the preprocessing under test
# ---------------------------------------------------------------------------

def pin_unit_rows(pre):
    """Normalized rows have length 1 and keep their direction; a zero row stays
    zero (the 1e-12 floor)."""
    q, k, v, g, b = _raw_head(1)
    q[3] = 0.0
    qq, kk, *_ = pre(q, k, v, g, b, oracle.NORM_QK, qkv_dtype="f64", gate_dtype="f64")
    nz = np.ones(len(q), bool)
    nz[3] = False
    assert np.allclose(np.linalg.norm(qq[nz], axis=1), 1.0, atol=1e-14)
    assert np.allclose(np.linalg.norm(kk, axis=1), 1.0, atol=1e-14)
    assert np.all(qq[3] == 0.0)
    # same direction: raw row = |raw row| * normalized row
    assert np.allclose(q[nz], np.linalg.norm(q[nz], axis=1, keepdims=True) * qq[nz],
                       rtol=1e-13, atol=1e-13)


def pin_scale_invariance(pre):
    """With NORM_QK, o and the state do not change when each token's raw q and
    k are multiplied by positive numbers (only directions enter)."""
    q, k, v, g, b = _raw_head(2)
    rng = np.random.default_rng(22)
    o1, s1 = _run(pre, q, k, v, g, b, ALL, "channel")
    sq = rng.uniform(1e-3, 1e3, (len(q), 1))
    sk = rng.uniform(1e-3, 1e3, (len(k), 1))
    o2, s2 = _run(pre, q * sq, k * sk, v, g, b, ALL, "channel")
    assert np.allclose(o1, o2, rtol=1e-12, atol=1e-12)
    assert np.allclose(s1, s2, rtol=1e-12, atol=1e-12)


def pin_sigmoid(pre):
    """sigmoid(0) = 1/2, sigmoid(x) + sigmoid(-x) = 1, slope 1/4 at 0, the
    library's logistic function elsewhere, and no overflow at +-1000."""
    x = np.array([0.0, 1e-3, -1e-3, 0.5, -3.0, 7.25, 40.0, -40.0, 1000.0, -1000.0])
    z = np.zeros((len(x), 2))
    one = np.ones((len(x), 2))
    _, _, _, _, s = pre(z, z, one, None, x, oracle.BETA_LOGIT, qkv_dtype="f64",
                        gate_dtype="f64")
    _, _, _, _, sn = pre(z, z, one, None, -x, oracle.BETA_LOGIT, qkv_dtype="f64",
                         gate_dtype="f64")
    assert s[0] == 0.5
    assert np.allclose(s + sn, 1.0, atol=1e-15)
    assert abs((s[1] - s[2]) / 2e-3 - 0.25) < 1e-6
    assert np.allclose(s, expit(x), rtol=1e-15, atol=0)
    assert s[-2] == 1.0 and s[-1] == 0.0


def pin_exact_readout(pre):
    """Unit keys make reading the key just written return its value exactly:
    with beta -> 1 (a logit of 40 rounds to 1 in fp64) and raw q a positive
    multiple of raw k, o_t = v_t for every t, whatever the decay."""
    q, k, v, g, b = _raw_head(3)
    q = k * np.random.default_rng(33).uniform(0.1, 10.0, (len(k), 1))
    b = np.full(len(k), 40.0)
    S0 = np.random.default_rng(34).standard_normal((q.shape[1], v.shape[1]))
    o, _ = _run(pre, q, k, v, g, b, ALL, "channel", S0=S0)
    assert np.allclose(o, v, rtol=0, atol=1e-12)


def pin_gate_limits(pre):
    """alpha = exp(-exp(g)) lies in (0, 1) and falls as g grows; g -> -inf keeps
    the state (alpha = 1: the same as no decay); g large wipes it (alpha = 0:
    o_t = beta_t (q_t . k_t) v_t, the first-token result with a zero state)."""
    q, k, v, g, b = _raw_head(4)
    gg = np.linspace(-8.0, 4.0, 25)
    z = np.zeros((25, 2))
    *_, la, _ = pre(z, z, z, gg, np.zeros(25), oracle.GATE_RAW, qkv_dtype="f64",
                    gate_dtype="f64")
    a = np.exp(la)
    assert np.all((a > 0) & (a < 1)) and np.all(np.diff(a) < 0)
    # g = 0 gives alpha = 1/e
    *_, l0, _ = pre(z[:1], z[:1], z[:1], np.zeros(1), np.zeros(1), oracle.GATE_RAW,
                    qkv_dtype="f64", gate_dtype="f64")
    assert l0[0] == -1.0
    S0 = np.random.default_rng(44).standard_normal((q.shape[1], v.shape[1]))
    keep, _ = _run(pre, q, k, v, np.full(g.shape, -60.0), b, ALL, "channel", S0=S0)
    flags = oracle.NORM_QK | oracle.BETA_LOGIT
    none, _ = _run(pre, q, k, v, None, b, flags, "none", S0=S0)
    assert np.allclose(keep, none, rtol=0, atol=1e-12)
    wipe, _ = _run(pre, q, k, v, np.full(g.shape, 8.0), b, ALL, "channel", S0=S0)
    qn, kn, _, _, bs = pre(q, k, v, None, b, flags, qkv_dtype="f64", gate_dtype="f64")
    ref = (bs * np.sum(qn * kn, axis=1))[:, None] * v
    assert np.allclose(wipe, ref, rtol=0, atol=1e-12)


def pin_head_gate(pre):
    """In head mode the gate applies -exp to the per-token scalar g as well."""
    q, k, v, g, b = _raw_head(5, mode="head")
    S0 = np.random.default_rng(55).standard_normal((q.shape[1], v.shape[1]))
    oh, sh = _run(pre, q, k, v, g, b, ALL, "head", S0=S0)
    oc, sc = _run(pre, q, k, v, np.repeat(g[:, None], q.shape[1], axis=1), b, ALL, "channel",
                  S0=S0)
    assert np.allclose(oh, oc, rtol=0, atol=1e-13)
    *_, la, _ = pre(q, k, v, g, b, oracle.GATE_RAW, qkv_dtype="f64", gate_dtype="f64")
    assert la.shape == g.shape and np.all(la < 0)


def pin_no_flags(pre):
    """flags = 0 only widens the stored values (bf16 bits exactly)."""
    w = gen.custom(B=1, H=1, L=9, dk=8, dv=8, qkv_dtype=gen.BF16, gate_dtype=gen.BF16)
    x = gen.prefill_inputs(w, raw=True)
    q, k, v, la, b = pre(x["q"][0, 0], x["k"][0, 0], x["v"][0, 0], x["log_alpha"][0, 0],
                         x["beta"][0, 0], 0, qkv_dtype="bf16", gate_dtype="bf16")
    for got, key in ((q, "q"), (k, "k"), (v, "v"), (la, "log_alpha"), (b, "beta")):
        want = gen.bf16_bits_to_f32(x[key][0, 0]).astype(np.float64)
        assert got.dtype == np.float64 and np.array_equal(got, want)


PINS = [pin_unit_rows, pin_scale_invariance, pin_sigmoid, pin_exact_readout, pin_gate_limits,
        pin_head_gate, pin_no_flags]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_preprocess_pin(pin, oracle_lib):
    pin(oracle.preprocess)


def test_raw_generator_matches_recipe():
    """The generator's raw mode draws the same streams as its default mode:
    preprocessing the raw draws in fp64 gives the default inputs up to their
    storage rounding."""
    w = gen.custom(B=2, H=2, L=17, dk=16, dv=8)
    a = gen.prefill_inputs(w)
    r = gen.prefill_inputs(w, raw=True)
    q, k, v, la, b = oracle.preprocess(r["q"], r["k"], r["v"], r["log_alpha"], r["beta"], ALL)
    for got, key in ((q, "q"), (k, "k"), (v, "v"), (la, "log_alpha"), (b, "beta")):
        assert np.allclose(got, a[key], rtol=2e-7, atol=1e-7), key


# ---------------------------------------------------------------------------
# planted mistakes, each in a test-local copy of the preprocessing
# ---------------------------------------------------------------------------

def _mutant(which):
    def pre(q, k, v, log_alpha, beta, flags, *, qkv_dtype="f32", gate_dtype="f32"):
        w = lambda x, dt: None if x is None else oracle._widen(x, dt)
        q, k, v = w(q, qkv_dtype), w(k, qkv_dtype), w(v, qkv_dtype)
        la, b = w(log_alpha, gate_dtype), w(beta, gate_dtype)
        if flags & oracle.NORM_QK:
            def nrm(x):
                if which == "norm_no_sqrt":
                    n = np.sum(x * x, axis=-1, keepdims=True)
                elif which == "norm_wrong_axis":
                    n = np.sqrt(np.sum(x * x, axis=0, keepdims=True))
                elif which == "norm_l1":
                    n = np.sum(np.abs(x), axis=-1, keepdims=True)
                else:
                    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
                return x / np.maximum(n, 1e-12)
            q = nrm(q) if which != "norm_k_only" else q
            k = nrm(k)
        if flags & oracle.BETA_LOGIT:
            b = 1.0 / (1.0 + np.exp(b if which == "sigmoid_sign" else -b))
        if flags & oracle.GATE_RAW and la is not None:
            la = np.exp(la) if which == "gate_sign" else (
                -np.exp(-la) if which == "gate_inner_sign" else -np.exp(la))
        return q, k, v, la, b
    return pre


MUTATIONS = ["norm_no_sqrt", "norm_wrong_axis", "norm_l1", "norm_k_only", "sigmoid_sign",
             "gate_sign", "gate_inner_sign"]


@pytest.mark.parametrize("which", MUTATIONS)
def test_preprocess_mutation_caught(which, oracle_lib):
    pre = _mutant(which)
    failed = []
    with np.errstate(all="ignore"):
        for pin in PINS:
            try:
                pin(pre)
            except AssertionError:
                failed.append(pin.__name__)
    assert failed, f"no pin catches the planted mistake {which}"


def test_unmutated_copy_passes(oracle_lib):
    """The test-local copy without a mistake passes every pin (so the mutation
    test measures the mistakes, not the copy)."""
    with np.errstate(over="ignore"):
        for pin in PINS:
            pin(_mutant("none"))
