"""Planted mistakes in a copy of the NumPy recurrence must each fail a pin.

This shows the pins are tight enough that a dropped term, a wrong sign, index
or axis, or a transposed operand in the oracle would not go unnoticed.  The
mistakes are planted here, in test-local copies; the oracle is untouched.
"""

import json
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "handworked_d2.json")


def _make(mutation):
    def rec(q, k, v, la, beta, S0=None):
        L, dk = q.shape
        dv = v.shape[1]
        if la is None:
            a = np.ones((L, dk))
        elif np.ndim(la) == 1:
            a = np.repeat(np.exp(la)[:, None], dk, axis=1)
        else:
            a = np.exp(la)
        S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=float)
        o = np.zeros((L, dv))
        for t in range(L):
            if mutation == "correct_then_decay":
                u = beta[t] * (v[t] - k[t] @ S)
                S = a[t][:, None] * (S + np.outer(k[t], u))
            else:
                if mutation == "decay_columns" and dk == dv:
                    S = S * a[t][None, :]
                elif mutation != "no_decay":
                    S = a[t][:, None] * S
                kS = k[t] @ S
                if mutation == "sign":
                    u = beta[t] * (v[t] + kS)
                elif mutation == "drop_beta":
                    u = v[t] - kS
                elif mutation == "drop_delta":
                    u = beta[t] * v[t]
                else:
                    u = beta[t] * (v[t] - kS)
                if mutation == "read_before_write":
                    o[t] = q[t] @ S
                S = S + (np.outer(u, k[t]) if (mutation == "transposed_write" and dk == dv)
                         else np.outer(k[t], u))
            if mutation != "read_before_write":
                o[t] = (S @ q[t]) if (mutation == "transposed_read" and dk == dv) else q[t] @ S
        return o, S
    return rec


MUTATIONS = ["correct_then_decay", "decay_columns", "no_decay", "sign", "drop_beta",
             "drop_delta", "read_before_write", "transposed_write", "transposed_read"]


def _pins_pass(rec):
    """The subset of pins that can run against a bare recurrence function."""
    with open(GOLDEN) as fh:
        cases = json.load(fh)["cases"]
    arr = lambda c, key: None if c[key] is None else np.array(c[key], dtype=float)
    for c in cases:
        o, S = rec(arr(c, "q"), arr(c, "k"), arr(c, "v"), arr(c, "log_alpha"), arr(c, "beta"),
                   arr(c, "S0"))
        if not (np.allclose(o, c["o"], atol=1e-9) and np.allclose(S, c["S_final"], atol=1e-9)):
            return False
    rng = np.random.default_rng(0)
    L, d = 20, 6
    k = rng.standard_normal((L, d))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((L, d))
    S0 = rng.standard_normal((d, d))
    la = -0.5 * rng.random((L, d))
    # P1 exact replacement
    o, _ = rec(k, k, v, la, np.ones(L), S0)
    if not np.allclose(o, v, atol=1e-9):
        return False
    # P5 pure decay along rows
    q = rng.standard_normal((L, d))
    o, S = rec(q, k, v, la, np.zeros(L), S0)
    g = np.cumsum(la, axis=0)
    if not (np.allclose(o, (q * np.exp(g)) @ S0, atol=1e-9)
            and np.allclose(S, np.exp(g[-1])[:, None] * S0, atol=1e-9)):
        return False
    return True


def test_unmutated_copy_passes():
    assert _pins_pass(_make(None))


@pytest.mark.parametrize("mutation", MUTATIONS)
def test_mutation_is_caught(mutation):
    assert not _pins_pass(_make(mutation))
