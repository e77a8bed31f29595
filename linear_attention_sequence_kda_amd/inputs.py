"""Seeded synthetic inputs for the KDA / gated delta rule workloads.

This module only draws random numbers and rounds them to their storage type.
It holds none of the recurrence's arithmetic, and both the HIP path (through
the tests and the benchmark) and the CPU oracle consume exactly the arrays it
returns.

Recipe (shared by every workload):

* generator: ``numpy.random.Generator(PCG64(SeedSequence(entropy)))`` with
  ``entropy = [seed, tensor_id, b, h]`` for prefill tensors and
  ``[seed, tensor_id, step]`` for decode tensors, so every (b, h) head block can
  be drawn on its own and host memory stays bounded at any sequence length;
* q, k: N(0, 1) in fp64, then L2-normalised per token over d_k;
* v: N(0, 1);
* log_alpha (the natural log of the decay, always <= 0): -exp(N(mu, sigma));
  one value per token-head in head mode, one per token-head-channel in channel
  mode, absent in "none" mode (alpha = 1);
* beta: sigmoid(N(0, 1));
* S0: N(0, std) in fp32 when the workload has one, otherwise absent (zero).

Raw mode (``raw=True``, the inputs of the fused preprocessing) draws from the
same streams and stores the values before the last step: q, k are the N(0, 1)
rows unnormalised, log_alpha holds g ~ N(mu, sigma) (the op takes
ln alpha = -exp(g)) and beta holds the N(0, 1) logits.

N(mu, sigma) names the mean and the standard deviation.  Storage rounding is
fp64 -> fp32 (round to nearest even) and, for bf16 tensors, fp32 -> bf16
(round to nearest even).  bf16 tensors are returned as their raw ``uint16``
bit patterns; fp32 tensors as ``float32``.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

F32 = "f32"
BF16 = "bf16"

ALPHA_NONE = "none"
ALPHA_HEAD = "head"
ALPHA_CHANNEL = "channel"

_TENSOR_IDS = {"q": 1, "k": 2, "v": 3, "log_alpha": 4, "beta": 5, "S0": 6}


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes, storage types and value distributions."""

    name: str
    B: int
    H: int
    L: int  # tokens per sequence for prefill; 1 for decode
    dk: int
    dv: int
    qkv_dtype: str  # dtype of q, k, v and of the output o
    gate_dtype: str  # dtype of log_alpha and beta
    alpha_mode: str
    la_mu: float = 0.0  # log_alpha = -exp(N(la_mu, la_sigma))
    la_sigma: float = 0.0
    s0_std: Optional[float] = None  # None: no initial state (zero)
    seed: int = 0
    decode_steps: int = 0  # > 0: a decode workload of this many steps

    @property
    def is_decode(self) -> bool:
        return self.decode_steps > 0

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads the method is measured on (sizes from the pages' configs).
WORKLOADS = {
    1: Workload("deltanet_fp32_b1_h1_l256_d64", 1, 1, 256, 64, 64, F32, F32,
                ALPHA_NONE, seed=1),
    2: Workload("gated_deltanet_bf16_b4_h16_l4096_d128", 4, 16, 4096, 128, 128,
                BF16, F32, ALPHA_HEAD, -4.0, 0.5, seed=2),
    3: Workload("kda_bf16_b2_h32_l8192_d128", 2, 32, 8192, 128, 128, BF16, BF16,
                ALPHA_CHANNEL, -4.0, 0.5, s0_std=0.02, seed=3),
    4: Workload("kda_long_bf16_b1_h16_l524288_d128", 1, 16, 524288, 128, 128,
                BF16, BF16, ALPHA_CHANNEL, -5.0, 0.5, seed=4),
    5: Workload("kda_decode_bf16_b256_h32_d128_x64", 256, 32, 1, 128, 128, BF16,
                F32, ALPHA_CHANNEL, -4.0, 0.5, s0_std=0.02, seed=5,
                decode_steps=64),
}


# --------------------------------------------------------------------------
# rounding helpers (storage conversion only)
# --------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest even) and return the uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # round half to even on the 16 dropped bits; only NaN patterns can wrap
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    out = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 exactly."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def to_storage(x64: np.ndarray, dtype: str) -> np.ndarray:
    """fp64 -> storage array (float32, or uint16 bf16 bits)."""
    x32 = np.asarray(x64, dtype=np.float64).astype(np.float32)
    if dtype == F32:
        return x32
    if dtype == BF16:
        return f32_to_bf16_bits(x32)
    raise ValueError(f"unknown dtype {dtype!r}")


def widen(x: Optional[np.ndarray], dtype: str) -> Optional[np.ndarray]:
    """Storage array -> exact fp64 values."""
    if x is None:
        return None
    if dtype == BF16:
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# draws
# --------------------------------------------------------------------------

def _rng(*entropy: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(
        [int(e) for e in entropy])))


def _unit_rows(rng: np.random.Generator, shape, raw: bool = False) -> np.ndarray:
    x = rng.standard_normal(shape)
    if raw:
        return x
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / n


def _log_alpha(rng, shape, mu, sigma, raw: bool = False) -> np.ndarray:
    g = rng.normal(mu, sigma, size=shape)
    return g if raw else -np.exp(g)


def _sigmoid_normal(rng, shape, raw: bool = False) -> np.ndarray:
    x = rng.standard_normal(shape)
    return x if raw else 1.0 / (1.0 + np.exp(-x))


def head_inputs(w: Workload, b: int, h: int, raw: bool = False) -> dict:
    """Inputs of one (b, h) head of a prefill workload, in storage types.

    Returns q [L,dk], k [L,dk], v [L,dv], log_alpha ([L,dk], [L] or None),
    beta [L] and S0 ([dk,dv] float32 or None).  ``raw``: see the module notes.
    """
    L, dk, dv = w.L, w.dk, w.dv
    out = {
        "q": to_storage(_unit_rows(_rng(w.seed, _TENSOR_IDS["q"], b, h), (L, dk), raw),
                        w.qkv_dtype),
        "k": to_storage(_unit_rows(_rng(w.seed, _TENSOR_IDS["k"], b, h), (L, dk), raw),
                        w.qkv_dtype),
        "v": to_storage(_rng(w.seed, _TENSOR_IDS["v"], b, h).standard_normal((L, dv)), w.qkv_dtype),
    }
    if w.alpha_mode == ALPHA_NONE:
        out["log_alpha"] = None
    else:
        shape = (L, dk) if w.alpha_mode == ALPHA_CHANNEL else (L,)
        out["log_alpha"] = to_storage(
            _log_alpha(_rng(w.seed, _TENSOR_IDS["log_alpha"], b, h), shape, w.la_mu, w.la_sigma,
                       raw), w.gate_dtype)
    out["beta"] = to_storage(_sigmoid_normal(_rng(w.seed, _TENSOR_IDS["beta"], b, h), (L,), raw),
                             w.gate_dtype)
    if w.s0_std is None:
        out["S0"] = None
    else:
        out["S0"] = (_rng(w.seed, _TENSOR_IDS["S0"], b, h).standard_normal((dk, dv))
                     * w.s0_std).astype(np.float32)
    return out


def prefill_inputs(w: Workload, heads=None, threads: int = 8, raw: bool = False) -> dict:
    """Stack head_inputs over all (b, h) (or the given list of (b, h) pairs).

    With ``heads=None`` the arrays are [B, H, ...]; with a list of n pairs they
    are [n, ...] in the order given.  Heads are drawn on ``threads`` threads
    (each head has its own generator, so the result does not depend on it).
    """
    pairs = heads if heads is not None else [(b, h) for b in range(w.B) for h in range(w.H)]
    if threads > 1 and len(pairs) > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(min(threads, len(pairs))) as ex:
            blocks = list(ex.map(lambda bh: head_inputs(w, *bh, raw=raw), pairs))
    else:
        blocks = [head_inputs(w, b, h, raw=raw) for (b, h) in pairs]
    out = {}
    for key in ("q", "k", "v", "log_alpha", "beta", "S0"):
        if blocks[0][key] is None:
            out[key] = None
            continue
        arr = np.stack([blk[key] for blk in blocks])
        if heads is None:
            arr = arr.reshape((w.B, w.H) + arr.shape[1:])
        out[key] = arr
    return out


def decode_state(w: Workload) -> Optional[np.ndarray]:
    """Initial fp32 state [B,H,dk,dv] of a decode workload (None: zero)."""
    if w.s0_std is None:
        return None
    return (_rng(w.seed, _TENSOR_IDS["S0"], 0, 0).standard_normal((w.B, w.H, w.dk, w.dv))
            * w.s0_std).astype(np.float32)


def decode_inputs(w: Workload, step: int, raw: bool = False) -> dict:
    """Inputs of one decode step: q,k [B,H,dk], v [B,H,dv], log_alpha
    ([B,H,dk], [B,H] or None), beta [B,H].  ``raw``: see the module notes."""
    B, H, dk, dv = w.B, w.H, w.dk, w.dv
    out = {
        "q": to_storage(_unit_rows(_rng(w.seed, _TENSOR_IDS["q"], step), (B, H, dk), raw),
                        w.qkv_dtype),
        "k": to_storage(_unit_rows(_rng(w.seed, _TENSOR_IDS["k"], step), (B, H, dk), raw),
                        w.qkv_dtype),
        "v": to_storage(_rng(w.seed, _TENSOR_IDS["v"], step).standard_normal((B, H, dv)), w.qkv_dtype),
    }
    if w.alpha_mode == ALPHA_NONE:
        out["log_alpha"] = None
    else:
        shape = (B, H, dk) if w.alpha_mode == ALPHA_CHANNEL else (B, H)
        out["log_alpha"] = to_storage(
            _log_alpha(_rng(w.seed, _TENSOR_IDS["log_alpha"], step), shape, w.la_mu, w.la_sigma,
                       raw), w.gate_dtype)
    out["beta"] = to_storage(_sigmoid_normal(_rng(w.seed, _TENSOR_IDS["beta"], step), (B, H),
                                             raw), w.gate_dtype)
    return out


def custom(B=1, H=1, L=64, dk=64, dv=64, qkv_dtype=F32, gate_dtype=F32,
           alpha_mode=ALPHA_CHANNEL, la_mu=-4.0, la_sigma=0.5, s0_std=0.02,
           seed=1234) -> Workload:
    """A workload of arbitrary shape drawn with the same recipe."""
    return Workload(f"custom_b{B}_h{H}_l{L}_dk{dk}_dv{dv}", B, H, L, dk, dv,
                    qkv_dtype, gate_dtype, alpha_mode, la_mu, la_sigma, s0_std, seed)
