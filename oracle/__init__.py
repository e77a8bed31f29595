"""CPU oracle of the KDA / gated delta rule -- TEST INFRASTRUCTURE ONLY.

Only the test-suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The HIP library never loads it, and the two share no
code: the only common module is the seeded input generator, which holds no
arithmetic of the method.

Contents
--------
``forward``            ctypes front end of the plain C fp64 token recurrence
                       (``kda_oracle.c``); the oracle proper.
``recurrence``         the same recurrence in NumPy fp64 (a second, independent
                       spelling used to cross-check the C code).
``brute_force``        the recurrence with each transition matrix
                       M_t = (I - beta_t k_t^T k_t) diag(alpha_t) built
                       explicitly, a different evaluation order.
``chunk_reference``    naive chunkwise form (per-chunk WY factors), the bridge
                       between the recurrence and the chunked GPU kernels.
``pages_chunk_deltanet`` the pages' printed alpha = 1 chunk algorithm, with its
                       batched indexing read per chunk.
``forward_substitution`` the pages' in-place inversion of (I + A).
``slab_error``         the parity metric.
``linear_attention``   normalized linear attention with phi = elu + 1 (fp64:
                       phi on the host, the C recurrence without the delta
                       term for the numerator and the state, a running sum
                       for the normalizer).
``preprocess``         the token mixer's input steps (L2-normalized q and k,
                       sigmoid beta, alpha = exp(-exp(g))) in fp64, applied to
                       raw stored inputs before ``forward``.
``backward``           gradients of the recurrence (reverse-mode through the
                       token loop) for a training backward pass: dq, dk, dv,
                       d ln(alpha), dbeta and dS0 from the gradients of o and
                       of the final state.

Every function takes fp64 NumPy arrays for one head unless said otherwise.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")

F32, BF16, F64 = 0, 1, 2
ALPHA_NONE, ALPHA_HEAD, ALPHA_CHANNEL = 0, 1, 2
_DT = {"f32": F32, "bf16": BF16, "f64": F64}
# input preprocessing bits (the same meaning as the library's input flags)
NORM_QK, BETA_LOGIT, GATE_RAW = 1, 2, 4
_AM = {"none": ALPHA_NONE, "head": ALPHA_HEAD, "channel": ALPHA_CHANNEL}


# ---------------------------------------------------------------------------
# build + load of the C oracle
# ---------------------------------------------------------------------------

def build(verbose: bool = False) -> str:
    """Compile kda_oracle.c with gcc (IEEE fp64, no contraction) in place."""
    cmd = ["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-pthread", _SRC, "-o", _LIB, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        f = lib.kda_oracle_forward
        i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        f.argtypes = [i64, i64, i64, i64, i64, i32, i32, i32,
                      vp, vp, vp, vp, vp, vp, i64, i64, i32, vp, vp, i32]
        f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def forward(q, k, v, log_alpha, beta, S0=None, *, qkv_dtype="f32", gate_dtype="f32",
            alpha_mode="channel", col0=0, ncols=None, delta=True, want_o=True,
            threads=None):
    """Run the C fp64 recurrence on stacked heads.

    q, k: [N, L, dk]; v: [N, L, dv]; log_alpha: [N, L, dk] | [N, L] | None;
    beta: [N, L]; S0: [N, dk, dv] (any float dtype, widened to fp64) or None.
    Arrays are in storage type: float32, or uint16 bf16 bits.
    Returns (o [N, L, ncols] fp64 or None, S_final [N, dk, ncols] fp64).
    """
    lib = _load()
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    beta = np.ascontiguousarray(beta)
    N, L, dk = q.shape
    dv = v.shape[-1]
    if ncols is None:
        ncols = dv - col0
    la = None if (log_alpha is None or alpha_mode == "none") else np.ascontiguousarray(log_alpha)
    s0 = None if S0 is None else np.ascontiguousarray(S0, dtype=np.float64)
    o = np.empty((N, L, ncols), dtype=np.float64) if want_o else None
    sf = np.empty((N, dk, ncols), dtype=np.float64)
    rc = lib.kda_oracle_forward(N, 1, L, dk, dv, _DT[qkv_dtype], _DT[gate_dtype],
                                _AM[alpha_mode], _ptr(q), _ptr(k), _ptr(v), _ptr(la),
                                _ptr(beta), _ptr(s0), col0, ncols, 1 if delta else 0,
                                _ptr(o), _ptr(sf),
                                threads if threads is not None else default_threads())
    if rc != 0:
        raise ValueError("kda_oracle_forward rejected its arguments")
    return o, sf


# ---------------------------------------------------------------------------
# input preprocessing of the token mixer (fp64)
# ---------------------------------------------------------------------------

def _widen(x, dtype: str):
    """Stored values as fp64: float32 as is, bf16 bits shifted into float32."""
    x = np.asarray(x)
    if dtype == "bf16":
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def l2_normalize(x):
    """x / max(|x|, 1e-12) over the last axis ("22,580: From GPT-2 to Kimi K3",
    sections 5.1-5.2: the DeltaNet layer normalizes q and k so that reading a
    stored key returns its value exactly; the 1e-12 floor keeps a zero row
    zero)."""
    x = np.asarray(x, dtype=np.float64)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / np.maximum(n, 1e-12)


def sigmoid(x):
    """1 / (1 + e^-x), evaluated on the side that does not overflow (the
    write strength beta of the delta rule, same page, section 5.2)."""
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def log_alpha_of_raw(g):
    """ln alpha = -exp(g), i.e. alpha = exp(-exp(g)) in (0, 1) ("22580: From
    GPT-2 to Kimi K3, Explained", "Key code and formulas", "KDA (per-channel
    alpha)")."""
    return -np.exp(np.asarray(g, dtype=np.float64))


def preprocess(q, k, v, log_alpha, beta, flags, *, qkv_dtype="f32", gate_dtype="f32"):
    """Raw stored inputs -> fp64 inputs of the recurrence.

    Each set bit applies one step: NORM_QK normalizes q and k per token over
    d_k, BETA_LOGIT takes beta = sigmoid(beta), GATE_RAW takes
    ln alpha = -exp(log_alpha).  Returns fp64 (q, k, v, log_alpha, beta) to
    pass to ``forward`` with qkv_dtype = gate_dtype = "f64".
    """
    q, k, v = (_widen(t, qkv_dtype) for t in (q, k, v))
    la = None if log_alpha is None else _widen(log_alpha, gate_dtype)
    b = _widen(beta, gate_dtype)
    if flags & NORM_QK:
        q, k = l2_normalize(q), l2_normalize(k)
    if flags & BETA_LOGIT:
        b = sigmoid(b)
    if flags & GATE_RAW and la is not None:
        la = log_alpha_of_raw(la)
    return q, k, v, la, b


# ---------------------------------------------------------------------------
# normalized linear attention (fp64)
# ---------------------------------------------------------------------------

def elu1(x):
    """phi(x) = elu(x) + 1: x + 1 for x > 0, e^x otherwise, so phi > 0 ("22,580:
    From GPT-2 to Kimi K3", section 04: the feature map applied to q and k
    separately before they meet)."""
    x = np.asarray(x, dtype=np.float64)
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def linear_attention(q, k, v, S0=None, z0=None, *, qkv_dtype="f32", threads=None):
    """Causal normalized linear attention on stacked heads.

    Per head, with phi = elu1 applied to the stored q and k (widened to fp64):
    S_t = S_{t-1} + phi(k_t)^T v_t, z_t = z_{t-1} + phi(k_t),
    o_t = phi(q_t) S_t / (phi(q_t) . z_t)  ("22,580: From GPT-2 to Kimi K3",
    section 04, and "22,580: GPT-2 to Kimi K3, explained" (zharfai.com),
    "Linear attention collapses history into a fixed state": state, normalizer,
    readout, division; read after the write).
    q, k: [N, L, dk]; v: [N, L, dv]; S0: [N, dk, dv] or None; z0: [N, dk] or
    None.  Returns (o [N, L, dv], S_final [N, dk, dv], z_final [N, dk]), fp64.
    """
    q, k, v = (_widen(t, qkv_dtype) for t in (q, k, v))
    fq, fk = elu1(q), elu1(k)
    N, L, dk = q.shape
    ones = np.ones((N, L))
    num, S = forward(fq, fk, v, None, ones, S0, qkv_dtype="f64", gate_dtype="f64",
                     alpha_mode="none", delta=False, threads=threads)
    z_prev = np.zeros((N, dk)) if z0 is None else np.asarray(z0, dtype=np.float64)
    z = z_prev[:, None, :] + np.cumsum(fk, axis=1)
    den = np.sum(fq * z, axis=-1)
    return num / den[:, :, None], S, (z[:, -1] if L else z_prev.copy())


# ---------------------------------------------------------------------------
# NumPy fp64 spellings (one head each)
# ---------------------------------------------------------------------------

def _decay(log_alpha, L, dk):
    """exp(log_alpha) as an [L, dk] array (broadcast in head mode, ones if None)."""
    if log_alpha is None:
        return np.ones((L, dk))
    la = np.asarray(log_alpha, dtype=np.float64)
    if la.ndim == 1:
        return np.repeat(np.exp(la)[:, None], dk, axis=1)
    return np.exp(la)


def recurrence(q, k, v, log_alpha, beta, S0=None, delta=True):
    """Token-by-token recurrence (decay, correct against the decayed state,
    write, read).  Same passages as kda_oracle.h.  Returns (o [L,dv], S)."""
    L, dk = q.shape
    dv = v.shape[1]
    a = _decay(log_alpha, L, dk)
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.zeros((L, dv))
    for t in range(L):
        S = a[t][:, None] * S
        kS = k[t] @ S if delta else 0.0
        u = beta[t] * (v[t] - kS)
        S = S + np.outer(k[t], u)
        o[t] = q[t] @ S
    return o, S


def backward(q, k, v, log_alpha, beta, S0, do, dS_final=None):
    """Gradients of the token recurrence of one head (the `recurrence` above:
    S~_t = diag(alpha_t) S_{t-1}, e_t = v_t - k_t S~_t, u_t = beta_t e_t,
    S_t = S~_t + k_t^T u_t, o_t = q_t S_t), by reverse-mode differentiation
    through the token loop.  The pages give the forward recurrence only
    ("trainable on GPUs" is their motivation for the chunk form); these are
    its derivatives, written out step by step and pinned by finite differences
    and by automatic differentiation of an independent forward.

    do: [L, dv] gradient of o; dS_final: [dk, dv] gradient of the final state
    (None: zero).  log_alpha: [L, dk] (per channel), [L] (per head) or None.
    Returns (dq [L,dk], dk [L,dk], dv [L,dv], dlog_alpha (shape of log_alpha,
    or None), dbeta [L], dS0 [dk,dv]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    L, dk = q.shape
    dv = v.shape[1]
    a = _decay(log_alpha, L, dk)
    # forward: the state entering each token
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    S_in = []
    for t in range(L):
        S_in.append(S)
        St = a[t][:, None] * S
        u = beta[t] * (v[t] - k[t] @ St)
        S = St + np.outer(k[t], u)
    dq = np.zeros((L, dk))
    dkk = np.zeros((L, dk))
    dvv = np.zeros((L, dv))
    dbeta = np.zeros(L)
    dla = np.zeros((L, dk))
    G = np.zeros((dk, dv)) if dS_final is None else np.array(dS_final, dtype=np.float64)
    for t in range(L - 1, -1, -1):
        # recompute step t
        St = a[t][:, None] * S_in[t]
        e = v[t] - k[t] @ St
        u = beta[t] * e
        S_t = St + np.outer(k[t], u)
        # o_t = q_t S_t
        dq[t] = S_t @ do[t]
        G = G + np.outer(q[t], do[t])          # total gradient of S_t
        # S_t = S~_t + k_t^T u_t
        gSt = G.copy()
        gk = G @ u
        gu = k[t] @ G
        # u_t = beta_t e_t, e_t = v_t - k_t S~_t
        dbeta[t] = gu @ e
        ge = beta[t] * gu
        dvv[t] = ge
        gk = gk - St @ ge
        gSt = gSt - np.outer(k[t], ge)
        dkk[t] = gk
        # S~_t = diag(alpha_t) S_{t-1}, alpha_t = exp(ln alpha_t)
        dla[t] = np.sum(gSt * St, axis=1)
        G = a[t][:, None] * gSt
    if log_alpha is None:
        dlog = None
    elif np.ndim(log_alpha) == 1:
        dlog = dla.sum(axis=1)
    else:
        dlog = dla
    return dq, dkk, dvv, dlog, dbeta, G


def backward_raw(q, k, v, g, b, S0, do, dS_final, flags):
    """Gradients with respect to raw inputs: the recurrence fed through the
    preprocessing steps of ``preprocess`` (the flags), all fp64, one head.

    q, k: [L, dk] (raw when NORM_QK); g: raw gate (GATE_RAW) or ln alpha,
    [L, dk], [L] or None; b: beta logits (BETA_LOGIT) or beta, [L].  The
    gradient of each step, from its definition:
      q / max(|q|, eps):  (dq_n - q_n (q_n . dq_n)) / |q| when |q| > eps,
                          dq_n / eps otherwise
      sigmoid(x):         dbeta sigmoid(x) (1 - sigmoid(x))
      -exp(g):            d ln alpha (-exp(g))
    Returns (dq, dk, dv, dg, db, dS0) like ``backward``.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    qn, kn, v64, la, beta = preprocess(q, k, v, g, b, flags, qkv_dtype="f64", gate_dtype="f64")
    dq, dk, dv, dla, dbeta, dS0 = backward(qn, kn, v64, la, beta, S0, do, dS_final)
    if flags & NORM_QK:
        def through_norm(x, xn, dxn):
            n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
            proj = dxn - xn * np.sum(xn * dxn, axis=-1, keepdims=True)
            return np.where(n > 1e-12, proj / np.maximum(n, 1e-300), dxn / 1e-12)
        dq, dk = through_norm(q, qn, dq), through_norm(k, kn, dk)
    if flags & BETA_LOGIT:
        dbeta = dbeta * beta * (1.0 - beta)
    if flags & GATE_RAW and dla is not None:
        dla = dla * la
    return dq, dk, dv, dla, dbeta, dS0


def brute_force(q, k, v, log_alpha, beta, S0=None):
    """S_t = M_t S_{t-1} + beta_t k_t^T v_t with M_t = (I - beta_t k_t^T k_t) D_t
    formed as an explicit d_k x d_k matrix ("Gated DeltaNet adds controlled
    forgetting", zharfai.com; products of Householder-like transitions,
    yichencityu.github.io section 6.3)."""
    L, dk = q.shape
    dv = v.shape[1]
    a = _decay(log_alpha, L, dk)
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.zeros((L, dv))
    eye = np.eye(dk)
    for t in range(L):
        M = (eye - beta[t] * np.outer(k[t], k[t])) @ np.diag(a[t])
        S = M @ S + beta[t] * np.outer(k[t], v[t])
        o[t] = q[t] @ S
    return o, S


def forward_substitution(A):
    """(I + A)^{-1} for strictly lower-triangular A (C x C), computed the way
    section 6.3 of yichencityu.github.io does it: start from -A and complete
    row i from the finished rows above it, then add the identity."""
    C = A.shape[0]
    T = -np.tril(A, -1)
    for i in range(1, C):
        T[i, :i] = T[i, :i] + (T[i, :, None] * T[:, :i]).sum(0)
    return T + np.eye(C)


def chunk_reference(q, k, v, log_alpha, beta, S0=None, C=64):
    """Chunkwise form of the gated delta rule with per-channel decay.

    For a chunk of n tokens entering with state S (g = cumulative sum of
    log_alpha within the chunk, per key channel):
        A_rj = beta_r sum_c k_rc k_jc exp(g_rc - g_jc)   (j < r)
        T    = (I + A)^{-1}                              (forward substitution)
        W    = T diag(beta) (K * exp(g)),   U = T diag(beta) V
        P_rj = sum_c q_rc k_jc exp(g_rc - g_jc)          (j <= r)
        u    = U - W S
        O    = (Q * exp(g)) S + P u
        S    <- diag(exp(g_n)) S + (K * exp(g_n - g))^T u
    At alpha = 1 this is the chunk algorithm of section 6.3 of
    yichencityu.github.io; the gated form is derived from the recurrence (the
    pages stop before printing it).  A short last chunk is simply shorter.
    """
    L, dk = q.shape
    dv = v.shape[1]
    la = np.zeros((L, dk))
    if log_alpha is not None:
        x = np.asarray(log_alpha, dtype=np.float64)
        la = np.repeat(x[:, None], dk, axis=1) if x.ndim == 1 else x
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.zeros((L, dv))
    for s in range(0, L, C):
        e = min(s + C, L)
        Q, K, V, bt = q[s:e], k[s:e], v[s:e], beta[s:e]
        g = np.cumsum(la[s:e], axis=0)
        n = e - s
        causal = np.tril(np.ones((n, n), dtype=bool))[:, :, None]
        dec = np.exp(np.where(causal, g[:, None, :] - g[None, :, :], -np.inf))  # [r, j, c]
        KK = np.einsum("rc,jc,rjc->rj", K, K, dec)
        QK = np.einsum("rc,jc,rjc->rj", Q, K, dec)
        A = np.tril(bt[:, None] * KK, -1)
        T = forward_substitution(A)
        W = T @ (bt[:, None] * K * np.exp(g))
        U = T @ (bt[:, None] * V)
        P = np.tril(QK)
        u = U - W @ S
        o[s:e] = (Q * np.exp(g)) @ S + P @ u
        S = np.exp(g[n - 1])[:, None] * S + (K * np.exp(g[n - 1][None, :] - g)).T @ u
    return o, S


def pages_chunk_deltanet(Q, K, V, beta, C):
    """The alpha = 1 chunk algorithm as printed in section 6.3 of
    yichencityu.github.io (zero initial state, L a multiple of C), with its
    batched triangular indexing read per chunk."""
    L, d = Q.shape
    dv = V.shape[1]
    Qc, Kc, Vc = (x.reshape(-1, C, x.shape[1]) for x in (Q, K, V))
    bc = beta.reshape(-1, C)
    K_beta = Kc * bc[..., None]
    V_beta = Vc * bc[..., None]
    T = -np.tril(K_beta @ Kc.transpose(0, 2, 1), -1)
    for i in range(1, C):
        T[:, i, :i] = T[:, i, :i] + (T[:, i, :, None] * T[:, :, :i]).sum(-2)
    T = T + np.eye(C)
    W = T @ K_beta
    U = T @ V_beta
    S = np.zeros((d, dv))
    O = np.empty_like(Vc)
    for i in range(L // C):
        q_i, k_i, w_i = Qc[i], Kc[i], W[i]
        u_i = U[i] - w_i @ S
        o_inter = q_i @ S
        A_i = np.tril(q_i @ k_i.T)
        O[i] = A_i @ u_i + o_inter
        S = S + k_i.T @ u_i
    return O.reshape(L, dv), S


# ---------------------------------------------------------------------------
# parity metric
# ---------------------------------------------------------------------------

def slab_error(x, ref, slab_axes=2):
    """Worst per-slab relative error max|x - ref| / max|ref|.

    The leading ``slab_axes`` axes index slabs (e.g. (b, h)); the metric is
    taken over each slab and the worst slab is returned.  Any NaN or Inf in
    x gives inf.  A slab whose reference is all zero is judged by its absolute
    error.
    """
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if x.shape != ref.shape:
        raise ValueError(f"shape mismatch {x.shape} vs {ref.shape}")
    if x.size == 0:
        return 0.0
    if not np.all(np.isfinite(x)):
        return float("inf")
    lead = int(np.prod(x.shape[:slab_axes])) if slab_axes else 1
    xs = x.reshape(lead, -1)
    rs = ref.reshape(lead, -1)
    num = np.max(np.abs(xs - rs), axis=1)
    den = np.max(np.abs(rs), axis=1)
    den = np.where(den > 0, den, 1.0)
    return float(np.max(num / den))
