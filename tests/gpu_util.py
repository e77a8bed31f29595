"""Helpers shared by the GPU parity tests (host-side marshalling only)."""

from __future__ import annotations

import sys

import numpy as np

import oracle
from linear_attention_sequence_kda_amd import inputs as gen

TOL = {"f32": 1e-4, "bf16": 2e-2}


def say(msg: str):
    """Name the case before each GPU step, flushed, so a failing run shows it."""
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def to_dev(arr, dtype: str):
    import torch
    if arr is None:
        return None
    if dtype == gen.BF16:
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.to("cuda:0")


def to_f64(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def device_inputs(w: gen.Workload, x: dict) -> dict:
    return {
        "q": to_dev(x["q"], w.qkv_dtype),
        "k": to_dev(x["k"], w.qkv_dtype),
        "v": to_dev(x["v"], w.qkv_dtype),
        "log_alpha": to_dev(x["log_alpha"], w.gate_dtype),
        "beta": to_dev(x["beta"], w.gate_dtype),
        "S0": to_dev(x["S0"], gen.F32) if x["S0"] is not None else None,
    }


def flat_heads(x: dict, N: int) -> dict:
    """[B,H,...] -> [B*H, ...] views of the stacked storage arrays."""
    return {k: (None if v is None else v.reshape((N,) + v.shape[2:])) for k, v in x.items()}


def oracle_prefill(w: gen.Workload, xf: dict, col0=0, ncols=None, S0=None):
    s0 = xf["S0"] if S0 is None else S0
    return oracle.forward(xf["q"], xf["k"], xf["v"], xf["log_alpha"], xf["beta"], s0,
                          qkv_dtype=w.qkv_dtype, gate_dtype=w.gate_dtype,
                          alpha_mode=w.alpha_mode, col0=col0, ncols=ncols)
