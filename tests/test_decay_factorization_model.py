"""A float32 NumPy model of how the prefill kernel factors the per-channel
decay inside the intra-chunk products (A and P), checked against the direct
definition on the CPU.

With g the chunk-relative cumulative sum of ln(alpha) per key channel, the
decayed causal products of one chunk are
    P_rj = sum_c q_rc k_jc e^(g_rc - g_jc),   A_rj = beta_r sum_c k_rc k_jc e^(g_rc - g_jc)
("22,580: From GPT-2 to Kimi K3", section 9.1 for the per-channel gate; the
chunk form of section 6.3).  An MFMA product needs the factor split into a
row part and a column part.  The kernel splits it at 16-token block
boundaries: G_R is g just before block R, Z_R = e^(G_(R+1) - G_R) the block's
decay.

* end split: row factor e^(g_r - G_(R+1)) (>= 1, up to 1 / Z_R), column
  factor e^(G_(J+1) - g_j), pair scale e^(G_(R+1) - G_(J+1)); a diagonal pair
  uses the stored operands as they are.  Used alone, 1 / Z_R overflows
  float32 once a sub-block's summed ln(alpha) drops below about -88 (about
  -5.5 per token), and 0 * inf then gives NaN.
* the kernel keeps the end split for a sub-block while Z_R >= 1e-30 in every
  channel; a sub-block below that ("flagged") takes the start split, row
  factor e^(g_r - G_R) (<= 1), pair scale e^(G_R - G_(J+1)) (<= 1), and its
  diagonal blocks are summed directly with running products of alpha (never
  an exponent above zero).

This is a model of the kernel's arithmetic (a design check), not the
oracle: the oracle is the token recurrence in oracle/.
"""

import numpy as np
import pytest

C, D, NB = 64, 32, 4
UNSAFE = np.float32(1e-30)


def inputs(la_value, seed=0):
    rng = np.random.default_rng(seed)
    q = rng.normal(size=(C, D)).astype(np.float32)
    k = rng.normal(size=(C, D)).astype(np.float32)
    q /= np.linalg.norm(q, axis=1, keepdims=True)
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    # ln(alpha) around la_value with a spread, per (token, channel)
    la = (la_value * np.exp(rng.normal(scale=0.3, size=(C, D)))).astype(np.float32)
    return q, k, la


def direct(q, k, la):
    """P and A/beta from the definition, in fp64 (lower triangle incl. diagonal)."""
    g = np.cumsum(la.astype(np.float64), axis=0)
    P = np.zeros((C, C))
    Ak = np.zeros((C, C))
    for r in range(C):
        for j in range(r + 1):
            f = np.exp(g[r] - g[j])
            P[r, j] = np.sum(q[r] * k[j] * f)
            Ak[r, j] = np.sum(k[r] * k[j] * f)
    return P, Ak


def block_terms(la):
    """x: within-block inclusive products, y: products of the later tokens
    of the block, Z: block products, all float32 running products."""
    a = np.exp(la).astype(np.float32)
    x = np.ones((C, D), np.float32)
    y = np.ones((C, D), np.float32)
    Z = np.ones((NB, D), np.float32)
    for R in range(NB):
        run = np.ones(D, np.float32)
        for s in range(16):
            run = run * a[16 * R + s]
            x[16 * R + s] = run
        Z[R] = run
        run = np.ones(D, np.float32)
        for s in range(15, -1, -1):
            y[16 * R + s] = run
            run = run * a[16 * R + s]
    return a, x, y, Z


def end_split(q, k, la):
    a, x, y, Z = block_terms(la)
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        rz = (np.float32(1) / Z).astype(np.float32)
        P = np.zeros((C, C), np.float32)
        for R in range(NB):
            for J in range(R + 1):
                rows = slice(16 * R, 16 * R + 16)
                cols = slice(16 * J, 16 * J + 16)
                qr = q[rows] * x[rows] * rz[R]
                pair = np.prod(Z[J + 1:R + 1], axis=0).astype(np.float32)
                kc = k[cols] * y[cols] * pair
                P[rows, cols] = qr @ kc.T
    return np.tril(P)


def kernel_split(q, k, la):
    a, x, y, Z = block_terms(la)
    P = np.zeros((C, C), np.float32)
    Ak = np.zeros((C, C), np.float32)
    flagged = [R for R in range(NB) if np.any(Z[R] < UNSAFE)]
    for R in range(NB):
        rows = slice(16 * R, 16 * R + 16)
        fl = R in flagged
        rz = np.float32(1) if fl else (np.float32(1) / Z[R]).astype(np.float32)
        qr, kr = q[rows] * x[rows] * rz, k[rows] * x[rows] * rz
        for J in range(R + 1):
            cols = slice(16 * J, 16 * J + 16)
            if J == R and fl:
                continue
            mend = R if fl else R + 1
            pair = np.prod(Z[J + 1:mend], axis=0).astype(np.float32)
            kcs = k[cols] * y[cols] * pair
            P[rows, cols] = qr @ kcs.T
            Ak[rows, cols] = kr @ kcs.T
        if fl:
            # direct sum with running products of alpha, one column at a time
            for jj in range(16):
                j = 16 * R + jj
                f = np.ones(D, np.float32)
                for r in range(j, 16 * R + 16):
                    if r > j:
                        f = f * a[r]
                    P[r, j] = np.sum(q[r] * k[j] * f)
                    Ak[r, j] = np.sum(k[r] * k[j] * f)
    for M in (P, Ak):
        assert np.all(np.isfinite(M))
    return np.tril(P), np.tril(Ak), flagged


def rel(x, ref):
    return float(np.max(np.abs(x - ref)) / np.max(np.abs(ref)))


@pytest.mark.parametrize("la_value", [-0.02, -1.0, -5.0, -8.0, -20.0, -1000.0])
def test_kernel_split_matches_definition(la_value):
    q, k, la = inputs(la_value, seed=int(-la_value * 7) % 1000)
    P_ref, A_ref = direct(q, k, la)
    P, Ak, unsafe = kernel_split(q, k, la)
    assert np.all(np.isfinite(P)) and np.all(np.isfinite(Ak))
    assert rel(P, P_ref) < 1e-5 and rel(Ak, A_ref) < 1e-5
    # the direct path is taken exactly when a block's decay leaves float range
    sums = np.array([la[16 * R:16 * R + 16].sum(axis=0).min() for R in range(NB)])
    if la_value >= -1.0:
        assert unsafe == []
    if la_value <= -8.0:
        assert unsafe == list(range(NB)), (unsafe, sums)


@pytest.mark.parametrize("la_value", [-0.02, -1.0, -3.0])
def test_end_split_fine_in_its_range(la_value):
    q, k, la = inputs(la_value, seed=3)
    P_ref, _ = direct(q, k, la)
    assert rel(end_split(q, k, la), P_ref) < 1e-5


@pytest.mark.parametrize("la_value", [-8.0, -20.0, -1000.0])
def test_end_split_alone_breaks_below_its_range(la_value):
    """Where the end split alone fails: its 1 / Z_R overflows and the product
    turns into inf or NaN (or the direct value is lost)."""
    q, k, la = inputs(la_value, seed=3)
    P_ref, _ = direct(q, k, la)
    P = end_split(q, k, la)
    assert (not np.all(np.isfinite(P))) or rel(P, P_ref) > 1e-2
