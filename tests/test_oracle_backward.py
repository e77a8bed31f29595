"""Pins of oracle.backward, the gradients of the gated delta rule recurrence
(CPU, fp64).

The pages give only the forward recurrence; its derivatives are pinned here by
things other than the derivation itself:
  * central finite differences of a scalar loss of the forward recurrence,
    for every input element, every decay mode, with and without S0 and an
    upstream gradient of the final state;
  * automatic differentiation (torch, float64, CPU) of an independently
    written forward: the explicit transition-matrix form
    S_t = (I - beta_t k_t^T k_t) diag(alpha_t) S_{t-1} + beta_t k_t^T v_t;
  * closed forms: beta = 0 leaves k and v without influence, and makes dS0 a
    sum of decayed outer products; a zero initial state gives the first
    token's decay no influence;
  * planted mistakes in a test-local copy of the reverse sweep, each of which
    must fail the finite-difference pin.
"""

import numpy as np
import pytest

import oracle

MODES = ["channel", "head", "none"]


def draw(L, dk, dv, mode, seed, s0=True):
    rng = np.random.default_rng(seed)
    q = rng.normal(size=(L, dk))
    k = rng.normal(size=(L, dk)) / np.sqrt(dk)
    v = rng.normal(size=(L, dv))
    la = {"channel": -np.exp(rng.normal(-1.0, 0.5, size=(L, dk))),
          "head": -np.exp(rng.normal(-1.0, 0.5, size=L)),
          "none": None}[mode]
    beta = 1.0 / (1.0 + np.exp(-rng.normal(size=L)))
    S0 = rng.normal(size=(dk, dv)) if s0 else None
    return q, k, v, la, beta, S0


def loss_fn(Wo, Ws):
    def J(q, k, v, la, beta, S0):
        o, S = oracle.recurrence(q, k, v, la, beta, S0)
        return float((o * Wo).sum() + (S * Ws).sum())
    return J


def finite_differences(J, args, h=1e-6):
    """Central differences of J w.r.t. every element of every array argument
    (None arguments give None)."""
    out = []
    for idx, arr in enumerate(args):
        if arr is None:
            out.append(None)
            continue
        arr = np.asarray(arr, dtype=np.float64)
        g = np.zeros_like(arr)
        for i in np.ndindex(arr.shape):
            ap, am = arr.copy(), arr.copy()
            ap[i] += h
            am[i] -= h
            a1, a2 = list(args), list(args)
            a1[idx], a2[idx] = ap, am
            g[i] = (J(*a1) - J(*a2)) / (2 * h)
        out.append(g)
    return out


def rel(a, b):
    return np.abs(a - b).max() / max(np.abs(b).max(), 1e-300)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("s0,final", [(True, True), (False, True), (True, False)])
def test_matches_finite_differences(mode, s0, final):
    L, dk, dv = 6, 3, 2
    q, k, v, la, beta, S0 = draw(L, dk, dv, mode, seed=11, s0=s0)
    rng = np.random.default_rng(5)
    Wo = rng.normal(size=(L, dv))
    Ws = rng.normal(size=(dk, dv)) if final else np.zeros((dk, dv))
    args = [q, k, v, la, beta, S0]
    fd = finite_differences(loss_fn(Wo, Ws), args)
    dq, dk_, dv_, dla, dbeta, dS0 = oracle.backward(q, k, v, la, beta, S0, Wo,
                                                     Ws if final else None)
    got = [dq, dk_, dv_, dla, dbeta, dS0 if s0 else None]
    for name, g, f in zip(["q", "k", "v", "log_alpha", "beta", "S0"], got, fd):
        if f is None:
            assert g is None or name == "S0"
            continue
        assert rel(g, f) <= 1e-7, (name, rel(g, f))


def _torch_transition_forward(torch, q, k, v, la, beta, S0):
    """S_t = M_t S_{t-1} + beta_t k_t^T v_t with M_t built as a d_k x d_k
    matrix (the transition form of the recurrence), o_t = q_t S_t."""
    L, dk = q.shape
    S = S0
    eye = torch.eye(dk, dtype=torch.float64)
    outs = []
    for t in range(L):
        if la is None:
            D = eye
        elif la.dim() == 1:
            D = eye * torch.exp(la[t])
        else:
            D = torch.diag(torch.exp(la[t]))
        M = (eye - beta[t] * torch.outer(k[t], k[t])) @ D
        S = M @ S + beta[t] * torch.outer(k[t], v[t])
        outs.append(q[t] @ S)
    return torch.stack(outs), S


@pytest.mark.parametrize("mode", MODES)
def test_matches_autograd_of_transition_form(mode):
    torch = pytest.importorskip("torch")
    L, dk, dv = 40, 6, 5
    q, k, v, la, beta, S0 = draw(L, dk, dv, mode, seed=21)
    rng = np.random.default_rng(8)
    Wo, Ws = rng.normal(size=(L, dv)), rng.normal(size=(dk, dv))
    T = lambda a: None if a is None else torch.tensor(a, dtype=torch.float64, requires_grad=True)
    tq, tk, tv, tla, tb, tS0 = (T(a) for a in (q, k, v, la, beta, S0))
    o, S = _torch_transition_forward(torch, tq, tk, tv, tla, tb, tS0)
    J = (o * torch.tensor(Wo)).sum() + (S * torch.tensor(Ws)).sum()
    J.backward()
    got = oracle.backward(q, k, v, la, beta, S0, Wo, Ws)
    ref = [tq.grad, tk.grad, tv.grad, None if tla is None else tla.grad, tb.grad, tS0.grad]
    for name, g, r in zip(["q", "k", "v", "log_alpha", "beta", "S0"], got, ref):
        if r is None:
            assert g is None
            continue
        assert rel(g, r.numpy()) <= 1e-10, (name, rel(g, r.numpy()))


def test_beta_zero_closed_form():
    """beta = 0: S_t = diag(prod_{s<=t} alpha_s) S0, so k and v have no
    influence and dS0 = sum_t diag(A_t) q_t^T do_t + diag(A_L) dS_final with
    A_t = prod_{s<=t} alpha_s."""
    L, dk, dv = 9, 4, 3
    q, k, v, la, _, S0 = draw(L, dk, dv, "channel", seed=3)
    beta = np.zeros(L)
    rng = np.random.default_rng(9)
    do, dSf = rng.normal(size=(L, dv)), rng.normal(size=(dk, dv))
    dq, dk_, dv_, dla, dbeta, dS0 = oracle.backward(q, k, v, la, beta, S0, do, dSf)
    assert np.all(dk_ == 0.0) and np.all(dv_ == 0.0)
    A = np.exp(np.cumsum(la, axis=0))            # [L, dk]
    want = sum(A[t][:, None] * np.outer(q[t], do[t]) for t in range(L)) + A[-1][:, None] * dSf
    assert rel(dS0, want) <= 1e-12
    # do_t = 0 and dS_final = 0 give zero gradients everywhere
    z = oracle.backward(q, k, v, la, beta, S0, np.zeros((L, dv)), None)
    assert all(np.all(g == 0.0) for g in z if g is not None)


def test_zero_initial_state_first_decay_has_no_influence():
    L, dk, dv = 7, 4, 3
    for mode in ("channel", "head"):
        q, k, v, la, beta, _ = draw(L, dk, dv, mode, seed=17)
        rng = np.random.default_rng(2)
        _, _, _, dla, _, _ = oracle.backward(q, k, v, la, beta, None, rng.normal(size=(L, dv)),
                                             rng.normal(size=(dk, dv)))
        assert np.all(np.asarray(dla[0]) == 0.0)
        assert np.abs(dla[1:]).max() > 0.0


def _reverse_sweep_with(mistake, q, k, v, la, beta, S0, do, dSf):
    """Test-local copy of the reverse sweep with one planted mistake."""
    L, dk = q.shape
    a = np.exp(la)
    S, S_in = S0.copy(), []
    for t in range(L):
        S_in.append(S)
        St = a[t][:, None] * S
        S = St + np.outer(k[t], beta[t] * (v[t] - k[t] @ St))
    out = {n: np.zeros_like(x) for n, x in (("q", q), ("k", k), ("v", v), ("la", la))}
    out["beta"] = np.zeros(L)
    G = dSf.copy()
    for t in range(L - 1, -1, -1):
        St = a[t][:, None] * S_in[t]
        e = v[t] - k[t] @ St
        u = beta[t] * e
        S_t = St + np.outer(k[t], u)
        out["q"][t] = (St if mistake == "read_before_write" else S_t) @ do[t]
        if mistake != "no_output_to_state":
            G = G + np.outer(q[t], do[t])
        gSt = G.copy()
        gk = G @ (e if mistake == "u_without_beta" else u)
        gu = k[t] @ G
        out["beta"][t] = gu @ (u if mistake == "dbeta_with_u" else e)
        ge = beta[t] * gu
        out["v"][t] = ge
        gk = gk + (St @ ge if mistake == "sign_of_correction" else -(St @ ge))
        if mistake != "no_correction_to_state":
            gSt = gSt - np.outer(k[t], ge)
        out["k"][t] = gk
        out["la"][t] = np.sum(gSt * (S_in[t] if mistake == "decay_grad_undecayed" else St), axis=1)
        G = gSt if mistake == "no_decay_in_propagation" else a[t][:, None] * gSt
    out["S0"] = G
    return out


@pytest.mark.parametrize("mistake", ["read_before_write", "no_output_to_state", "u_without_beta",
                                     "dbeta_with_u", "sign_of_correction",
                                     "no_correction_to_state", "decay_grad_undecayed",
                                     "no_decay_in_propagation"])
def test_planted_mistakes_fail_the_pin(mistake):
    L, dk, dv = 5, 3, 2
    q, k, v, la, beta, S0 = draw(L, dk, dv, "channel", seed=31)
    rng = np.random.default_rng(6)
    Wo, Ws = rng.normal(size=(L, dv)), rng.normal(size=(dk, dv))
    fd = dict(zip(["q", "k", "v", "la", "beta", "S0"],
                  finite_differences(loss_fn(Wo, Ws), [q, k, v, la, beta, S0])))
    clean = _reverse_sweep_with(None, q, k, v, la, beta, S0, Wo, Ws)
    assert max(rel(clean[n], fd[n]) for n in fd) <= 1e-7      # the copy itself is right
    bad = _reverse_sweep_with(mistake, q, k, v, la, beta, S0, Wo, Ws)
    assert max(rel(bad[n], fd[n]) for n in fd) > 1e-3, mistake


# ---- gradients with respect to raw inputs (the preprocessing steps) ----------

def _raw_draw(L, dk, dv, mode, seed):
    rng = np.random.default_rng(seed)
    q = rng.normal(size=(L, dk)) * 3.0          # raw: normalized by the op
    k = rng.normal(size=(L, dk)) * 2.0
    v = rng.normal(size=(L, dv))
    g = {"channel": rng.normal(-1.0, 0.5, size=(L, dk)), "head": rng.normal(-1.0, 0.5, size=L),
         "none": None}[mode]                    # raw gate: ln alpha = -exp(g)
    x = rng.normal(size=L)                      # beta logits
    S0 = rng.normal(size=(dk, dv))
    return q, k, v, g, x, S0


def _raw_loss(Wo, Ws, flags):
    def J(q, k, v, g, x, S0):
        qn, kn, v64, la, b = oracle.preprocess(q, k, v, g, x, flags, qkv_dtype="f64",
                                               gate_dtype="f64")
        o, S = oracle.recurrence(qn, kn, v64, la, b, S0)
        return float((o * Wo).sum() + (S * Ws).sum())
    return J


@pytest.mark.parametrize("mode", ["channel", "head"])
@pytest.mark.parametrize("flags", [oracle.NORM_QK, oracle.BETA_LOGIT, oracle.GATE_RAW,
                                   oracle.NORM_QK | oracle.BETA_LOGIT | oracle.GATE_RAW])
def test_raw_input_gradients_match_finite_differences(mode, flags):
    L, dk, dv = 6, 3, 2
    q, k, v, g, x, S0 = _raw_draw(L, dk, dv, mode, seed=13)
    if not flags & oracle.BETA_LOGIT:
        x = 1.0 / (1.0 + np.exp(-x))            # already a strength in (0, 1)
    if not flags & oracle.GATE_RAW:
        g = -np.exp(g)                           # already ln alpha
    rng = np.random.default_rng(4)
    Wo, Ws = rng.normal(size=(L, dv)), rng.normal(size=(dk, dv))
    fd = finite_differences(_raw_loss(Wo, Ws, flags), [q, k, v, g, x, S0])
    got = oracle.backward_raw(q, k, v, g, x, S0, Wo, Ws, flags)
    for name, a, f in zip(["q", "k", "v", "g", "beta", "S0"], got, fd):
        assert rel(a, f) <= 1e-6, (name, rel(a, f))


def test_raw_gradients_without_flags_equal_backward():
    q, k, v, g, x, S0 = _raw_draw(7, 4, 3, "channel", seed=2)
    la, b = -np.exp(g), 1.0 / (1.0 + np.exp(-x))
    rng = np.random.default_rng(1)
    do, dSf = rng.normal(size=(7, 3)), rng.normal(size=(4, 3))
    a = oracle.backward_raw(q, k, v, la, b, S0, do, dSf, 0)
    r = oracle.backward(q, k, v, la, b, S0, do, dSf)
    assert all(np.array_equal(x1, x2) for x1, x2 in zip(a, r))


def test_zero_raw_row_follows_the_floor():
    """A zero q row is scaled by 1 / 1e-12 (the floor), so its gradient is the
    normalized-row gradient times 1e12, not the projection."""
    q, k, v, g, x, S0 = _raw_draw(5, 3, 2, "head", seed=8)
    q[2] = 0.0
    rng = np.random.default_rng(3)
    do = rng.normal(size=(5, 2))
    dq = oracle.backward_raw(q, k, v, g, x, S0, do, None, oracle.NORM_QK | oracle.GATE_RAW
                             | oracle.BETA_LOGIT)[0]
    qn, kn, v64, la, b = oracle.preprocess(q, k, v, g, x, 7, qkv_dtype="f64", gate_dtype="f64")
    dqn = oracle.backward(qn, kn, v64, la, b, S0, do, None)[0]
    assert np.allclose(dq[2], dqn[2] * 1e12, rtol=1e-14, atol=0.0)
