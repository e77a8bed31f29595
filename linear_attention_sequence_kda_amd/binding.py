"""ctypes binding of libkda.so -- argument marshalling only.

Every step of the computation runs in the HIP kernels behind the C ABI
(``include/kda.h``).  PyTorch supplies device memory and the current stream.
There is no fallback: if the library is missing, or a tensor is not on a
GPU, the call raises.
"""

from __future__ import annotations

import ctypes
import os
import re
from typing import Optional, Tuple

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libkda.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "kda.h")

KDA_F32, KDA_BF16 = 0, 1
KDA_ALPHA_NONE, KDA_ALPHA_HEAD, KDA_ALPHA_CHANNEL = 0, 1, 2
STATUS = {0: "KDA_OK", 1: "KDA_ERR_NULL", 2: "KDA_ERR_SHAPE", 3: "KDA_ERR_DTYPE",
          4: "KDA_ERR_ALPHA_MODE", 5: "KDA_ERR_ALIGN", 6: "KDA_ERR_WORKSPACE",
          7: "KDA_ERR_ALIAS", 8: "KDA_ERR_HIP", 9: "KDA_ERR_FLAGS", 10: "KDA_ERR_SCRATCH"}
# kda_input_flags: preprocessing applied by the kernels as they load raw inputs
NORM_QK, BETA_LOGIT, GATE_RAW = 1, 2, 4


class KdaShape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("H", ctypes.c_int64), ("L", ctypes.c_int64),
                ("dk", ctypes.c_int64), ("dv", ctypes.c_int64),
                ("qkv_dtype", ctypes.c_int32), ("gate_dtype", ctypes.c_int32),
                ("alpha_mode", ctypes.c_int32)]


class KdaError(RuntimeError):
    def __init__(self, status: int, text: str):
        super().__init__(f"{STATUS.get(status, status)}: {text}")
        self.status = status


_lib = None


def library() -> ctypes.CDLL:
    """Load libkda.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it first (python -m "
                "linear_attention_sequence_kda_amd.build, or __graft_entry__.build())")
        lib = ctypes.CDLL(LIB_PATH)
        vp, sz = ctypes.c_void_p, ctypes.c_size_t
        sp = ctypes.POINTER(KdaShape)
        lib.kda_chunk_fwd.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.kda_chunk_fwd.restype = ctypes.c_int
        lib.kda_chunk_fwd_workspace_bytes.argtypes = [sp]
        lib.kda_chunk_fwd_workspace_bytes.restype = sz
        lib.kda_decode_step.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.kda_decode_step.restype = ctypes.c_int
        lib.kda_decode_step_slots.argtypes = [sp, vp, vp, vp, vp, vp, vp, ctypes.c_int64, vp, vp,
                                              vp]
        lib.kda_decode_step_slots.restype = ctypes.c_int
        u32 = ctypes.c_uint32
        i64 = ctypes.c_int64
        lib.kda_chunk_fwd_varlen.argtypes = [sp, u32, vp, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                             sz, vp]
        lib.kda_chunk_fwd_varlen.restype = ctypes.c_int
        lib.kda_linear_attn_fwd.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.kda_linear_attn_fwd.restype = ctypes.c_int
        lib.kda_linear_attn_decode_step.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp]
        lib.kda_linear_attn_decode_step.restype = ctypes.c_int
        lib.kda_linear_attn_fwd_workspace_bytes.argtypes = [sp]
        lib.kda_linear_attn_fwd_workspace_bytes.restype = sz
        lib.kda_chunk_fwd_varlen_workspace_bytes.argtypes = [sp, i64]
        lib.kda_chunk_fwd_varlen_workspace_bytes.restype = sz
        lib.kda_chunk_fwd_ex.argtypes = [sp, u32, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.kda_chunk_fwd_ex.restype = ctypes.c_int
        lib.kda_chunk_fwd_noalloc.argtypes = [sp, u32, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.kda_chunk_fwd_noalloc.restype = ctypes.c_int
        lib.kda_decode_step_ex.argtypes = [sp, u32, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.kda_decode_step_ex.restype = ctypes.c_int
        lib.kda_decode_step_slots_ex.argtypes = [sp, u32, vp, vp, vp, vp, vp, vp, ctypes.c_int64,
                                                 vp, vp, vp]
        lib.kda_decode_step_slots_ex.restype = ctypes.c_int
        lib.kda_recurrence_bwd.argtypes = [sp] + [vp] * 15 + [sz, vp]
        lib.kda_recurrence_bwd.restype = ctypes.c_int
        lib.kda_recurrence_bwd_workspace_bytes.argtypes = [sp]
        lib.kda_recurrence_bwd_workspace_bytes.restype = sz
        lib.kda_recurrence_bwd_ex.argtypes = [sp, u32] + [vp] * 15 + [sz, vp]
        lib.kda_recurrence_bwd_ex.restype = ctypes.c_int
        lib.kda_recurrence_bwd_ex_workspace_bytes.argtypes = [sp, u32]
        lib.kda_recurrence_bwd_ex_workspace_bytes.restype = sz
        lib.kda_chunk_bwd.argtypes = [sp] + [vp] * 15 + [sz, vp]
        lib.kda_chunk_bwd.restype = ctypes.c_int
        lib.kda_chunk_bwd_workspace_bytes.argtypes = [sp]
        lib.kda_chunk_bwd_workspace_bytes.restype = sz
        lib.kda_strerror.argtypes = [ctypes.c_int]
        lib.kda_strerror.restype = ctypes.c_char_p
        lib.kda_last_error.argtypes = []
        lib.kda_last_error.restype = ctypes.c_char_p
        lib.kda_abi_version.argtypes = []
        lib.kda_abi_version.restype = ctypes.c_int
        lib.kda_timing_enable.argtypes = [ctypes.c_int]
        lib.kda_timing_enable.restype = ctypes.c_int
        lib.kda_timing_reset.argtypes = []
        lib.kda_timing_reset.restype = ctypes.c_int
        lib.kda_timing_read.argtypes = [ctypes.c_char_p, ctypes.POINTER(ctypes.c_int64),
                                        ctypes.POINTER(ctypes.c_double)]
        lib.kda_timing_read.restype = ctypes.c_int
        _lib = lib
    return _lib


def header_functions():
    """Names of the functions declared in include/kda.h."""
    with open(HEADER) as fh:
        text = fh.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_]+)\s*\(", text)))


def _check(rc: int):
    if rc != 0:
        lib = library()
        text = lib.kda_strerror(rc).decode()
        extra = lib.kda_last_error().decode()
        raise KdaError(rc, text + (f" ({extra})" if extra else ""))


# ---------------------------------------------------------------------------
# torch front end
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    if t.dtype == torch.float32:
        return KDA_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _require(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(t) -> int:
    torch = _torch()
    return torch.cuda.current_stream(t.device).cuda_stream


KERNELS = ("kda_intra_kernel", "kda_inter_kernel", "kda_inter_scalar_kernel",
           "kda_inter_wide_kernel", "kda_inter_quad_kernel", "kda_feature_map_kernel",
           "kda_decode_kernel", "kda_bwd_kernel", "kda_inter_wide_scan",
           "kda_chunk_grad_kernel", "kda_gate_widen_kernel")


def timing_enable(on: bool = True) -> None:
    """Bracket every later kernel launch with HIP events on its stream."""
    _check(library().kda_timing_enable(1 if on else 0))


def timing_reset() -> None:
    """Drop the kept event pairs."""
    _check(library().kda_timing_reset())


def timing_read(kernel: str) -> Tuple[int, float]:
    """(launches, summed milliseconds) of one kernel since the last reset."""
    n, ms = ctypes.c_int64(0), ctypes.c_double(0.0)
    _check(library().kda_timing_read(kernel.encode(), ctypes.byref(n), ctypes.byref(ms)))
    return n.value, ms.value


def chunk_fwd_workspace_bytes(q, v, log_alpha, beta) -> int:
    """Device workspace bytes chunk_fwd needs for these inputs."""
    return library().kda_chunk_fwd_workspace_bytes(ctypes.byref(_chunk_shape(q, v, log_alpha,
                                                                             beta)))


def _chunk_shape(q, v, log_alpha, beta) -> KdaShape:
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    if log_alpha is None:
        mode = KDA_ALPHA_NONE
    elif log_alpha.dim() == 3:
        mode = KDA_ALPHA_HEAD
    else:
        mode = KDA_ALPHA_CHANNEL
    return KdaShape(B, H, L, dk, dv, _dtype_code(q),
                    _dtype_code(log_alpha if log_alpha is not None else beta), mode)


def chunk_fwd(q, k, v, log_alpha, beta, S0=None, *, output_final_state: bool = True,
              o=None, S_final=None, workspace=None,
              flags: Optional[int] = None) -> Tuple[object, Optional[object]]:
    """Chunkwise prefill: returns (o [B,H,L,dv], S_final [B,H,dk,dv] fp32 or None).

    q, k: [B,H,L,dk]; v: [B,H,L,dv] (bf16 or fp32, same dtype);
    log_alpha: None (alpha = 1), [B,H,L] (one decay per head) or [B,H,L,dk]
    (one per key channel); beta: [B,H,L] (same dtype as log_alpha, or any
    float dtype when log_alpha is None); S0: [B,H,dk,dv] fp32 or None.
    ``o`` / ``S_final`` may be given to write into existing buffers
    (S_final may be S0 itself); ``workspace`` may be a uint8 GPU tensor of at
    least chunk_fwd_workspace_bytes() bytes (else one is allocated per call).
    ``flags`` (a set of NORM_QK | BETA_LOGIT | GATE_RAW) calls kda_chunk_fwd_ex
    on raw inputs; None calls kda_chunk_fwd.
    """
    torch = _torch()
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    for name, t in (("q", q), ("k", k), ("v", v), ("beta", beta), ("log_alpha", log_alpha),
                    ("S0", S0)):
        if t is not None:
            _require(t, name)
    if o is None:
        o = torch.empty((B, H, L, dv), dtype=v.dtype, device=v.device)
    if output_final_state and S_final is None:
        S_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=v.device)
    if S0 is not None and S0.dtype != torch.float32:
        raise TypeError("S0 must be float32")
    shape = _chunk_shape(q, v, log_alpha, beta)
    lib = library()
    ws = lib.kda_chunk_fwd_workspace_bytes(ctypes.byref(shape))
    if workspace is None:
        workspace = torch.empty(ws, dtype=torch.uint8, device=v.device) if ws else None
    else:
        _require(workspace, "workspace")
    ws_given = workspace.numel() * workspace.element_size() if workspace is not None else 0
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S0), _ptr(o),
            _ptr(S_final) if output_final_state else None, _ptr(workspace), ws_given,
            _stream(v))
    if flags is None:
        rc = lib.kda_chunk_fwd(ctypes.byref(shape), *args)
    else:
        rc = lib.kda_chunk_fwd_ex(ctypes.byref(shape), flags, *args)
    _check(rc)
    return o, (S_final if output_final_state else None)


def chunk_fwd_noalloc(q, k, v, log_alpha, beta, S0=None, *, output_final_state: bool = True,
                      o=None, S_final=None, flags: int = 0) -> Tuple[object, Optional[object]]:
    """Chunkwise prefill through kda_chunk_fwd_noalloc: the library keeps its
    work memory in a static device buffer, so the call itself allocates
    nothing on the device (pass ``o`` and, if wanted, ``S_final`` to avoid
    the two output allocations made here otherwise).  Arguments and results
    as chunk_fwd with ``flags`` (0 = preprocessed inputs)."""
    torch = _torch()
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    for name, t in (("q", q), ("k", k), ("v", v), ("beta", beta), ("log_alpha", log_alpha),
                    ("S0", S0)):
        if t is not None:
            _require(t, name)
    if o is None:
        o = torch.empty((B, H, L, dv), dtype=v.dtype, device=v.device)
    if output_final_state and S_final is None:
        S_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=v.device)
    if S0 is not None and S0.dtype != torch.float32:
        raise TypeError("S0 must be float32")
    shape = _chunk_shape(q, v, log_alpha, beta)
    rc = library().kda_chunk_fwd_noalloc(
        ctypes.byref(shape), flags, _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
        _ptr(S0), _ptr(o), _ptr(S_final) if output_final_state else None, _stream(v))
    _check(rc)
    return o, (S_final if output_final_state else None)


def recurrence_bwd_workspace_bytes(q, v, log_alpha, beta) -> int:
    shape = _chunk_shape(q, v, log_alpha, beta)
    return int(library().kda_recurrence_bwd_workspace_bytes(ctypes.byref(shape)))


def recurrence_bwd(q, k, v, log_alpha, beta, S0, do, dS_final=None, *, want_dS0: bool = True,
                   workspace=None, flags: Optional[int] = None):
    """Gradients of the recurrence (kda_recurrence_bwd): returns
    (dq, dk, dv, dlog_alpha or None, dbeta, dS0 or None), all fp32.

    Inputs as for chunk_fwd (preprocessed values); do: [B,H,L,dv] in v's dtype;
    dS_final: [B,H,dk,dv] fp32 or None.  ``workspace`` may be a uint8 GPU
    tensor of at least recurrence_bwd_workspace_bytes() bytes.  ``flags`` (a
    set of NORM_QK | BETA_LOGIT | GATE_RAW) calls kda_recurrence_bwd_ex on raw
    inputs, whose gradients are then with respect to the raw values.
    """
    torch = _torch()
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    for name, t in (("q", q), ("k", k), ("v", v), ("beta", beta), ("log_alpha", log_alpha),
                    ("S0", S0), ("do", do), ("dS_final", dS_final)):
        if t is not None:
            _require(t, name)
    for name, t in (("S0", S0), ("dS_final", dS_final)):
        if t is not None and t.dtype != torch.float32:
            raise TypeError(name + " must be float32")
    dev, f32 = v.device, torch.float32
    dq = torch.empty((B, H, L, dk), dtype=f32, device=dev)
    dk_ = torch.empty((B, H, L, dk), dtype=f32, device=dev)
    dv_ = torch.empty((B, H, L, dv), dtype=f32, device=dev)
    dla = None if log_alpha is None else torch.empty(log_alpha.shape, dtype=f32, device=dev)
    dbeta = torch.empty((B, H, L), dtype=f32, device=dev)
    dS0 = torch.empty((B, H, dk, dv), dtype=f32, device=dev) if want_dS0 else None
    shape = _chunk_shape(q, v, log_alpha, beta)
    lib = library()
    if flags is None:
        ws = lib.kda_recurrence_bwd_workspace_bytes(ctypes.byref(shape))
    else:
        ws = lib.kda_recurrence_bwd_ex_workspace_bytes(ctypes.byref(shape), flags)
    if workspace is None:
        workspace = torch.empty(ws, dtype=torch.uint8, device=dev) if ws else None
    else:
        _require(workspace, "workspace")
    ws_given = workspace.numel() * workspace.element_size() if workspace is not None else 0
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S0), _ptr(do),
            _ptr(dS_final), _ptr(dq), _ptr(dk_), _ptr(dv_), _ptr(dla), _ptr(dbeta), _ptr(dS0),
            _ptr(workspace), ws_given, _stream(v))
    if flags is None:
        _check(lib.kda_recurrence_bwd(ctypes.byref(shape), *args))
    else:
        _check(lib.kda_recurrence_bwd_ex(ctypes.byref(shape), flags, *args))
    return dq, dk_, dv_, dla, dbeta, dS0


def chunk_bwd_workspace_bytes(q, v, log_alpha, beta) -> int:
    shape = _chunk_shape(q, v, log_alpha, beta)
    return int(library().kda_chunk_bwd_workspace_bytes(ctypes.byref(shape)))


def chunk_bwd(q, k, v, log_alpha, beta, S0, do, dS_final=None, *, want_dS0: bool = True,
              workspace=None):
    """Chunkwise gradients (kda_chunk_bwd): the outputs of recurrence_bwd,
    (dq, dk, dv, dlog_alpha or None, dbeta, dS0 or None), all fp32; q, k, v
    and do bf16.  ``workspace`` may be a uint8 GPU tensor of at least
    chunk_bwd_workspace_bytes() bytes."""
    torch = _torch()
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    for name, t in (("q", q), ("k", k), ("v", v), ("beta", beta), ("log_alpha", log_alpha),
                    ("S0", S0), ("do", do), ("dS_final", dS_final)):
        if t is not None:
            _require(t, name)
    for name, t in (("S0", S0), ("dS_final", dS_final)):
        if t is not None and t.dtype != torch.float32:
            raise TypeError(name + " must be float32")
    dev, f32 = v.device, torch.float32
    dq = torch.empty((B, H, L, dk), dtype=f32, device=dev)
    dk_ = torch.empty((B, H, L, dk), dtype=f32, device=dev)
    dv_ = torch.empty((B, H, L, dv), dtype=f32, device=dev)
    dla = None if log_alpha is None else torch.empty(log_alpha.shape, dtype=f32, device=dev)
    dbeta = torch.empty((B, H, L), dtype=f32, device=dev)
    dS0 = torch.empty((B, H, dk, dv), dtype=f32, device=dev) if want_dS0 else None
    shape = _chunk_shape(q, v, log_alpha, beta)
    lib = library()
    ws = lib.kda_chunk_bwd_workspace_bytes(ctypes.byref(shape))
    if workspace is None:
        workspace = torch.empty(ws, dtype=torch.uint8, device=dev) if ws else None
    else:
        _require(workspace, "workspace")
    ws_given = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.kda_chunk_bwd(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha),
                             _ptr(beta), _ptr(S0), _ptr(do), _ptr(dS_final), _ptr(dq), _ptr(dk_),
                             _ptr(dv_), _ptr(dla), _ptr(dbeta), _ptr(dS0), _ptr(workspace),
                             ws_given, _stream(v)))
    return dq, dk_, dv_, dla, dbeta, dS0


def _varlen_shape(q, v, log_alpha, beta, n_seq: int) -> KdaShape:
    H, T, dk = q.shape
    dv = v.shape[-1]
    if log_alpha is None:
        mode = KDA_ALPHA_NONE
    elif log_alpha.dim() == 2:
        mode = KDA_ALPHA_HEAD
    else:
        mode = KDA_ALPHA_CHANNEL
    return KdaShape(n_seq, H, T, dk, dv, _dtype_code(q),
                    _dtype_code(log_alpha if log_alpha is not None else beta), mode)


def chunk_fwd_varlen(q, k, v, log_alpha, beta, cu_seqlens, max_seqlen: int, S0=None, *,
                     output_final_state: bool = True, o=None, S_final=None, workspace=None,
                     flags: int = 0) -> Tuple[object, Optional[object]]:
    """Prefill of N packed sequences: returns (o [H,T,dv], S_final [N,H,dk,dv] or None).

    q, k: [H,T,dk]; v: [H,T,dv]; log_alpha: None, [H,T] or [H,T,dk]; beta:
    [H,T]; sequence i owns tokens cu_seqlens[i] .. cu_seqlens[i+1]-1
    (cu_seqlens: int32 [N+1] on the GPU); max_seqlen: an int >= every length;
    S0: [N,H,dk,dv] fp32 or None.  ``flags`` as for chunk_fwd.
    """
    torch = _torch()
    H, T, dk = q.shape
    dv = v.shape[-1]
    for name, t in (("q", q), ("k", k), ("v", v), ("beta", beta), ("log_alpha", log_alpha),
                    ("S0", S0), ("cu_seqlens", cu_seqlens)):
        if t is not None:
            _require(t, name)
    if cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    n_seq = cu_seqlens.numel() - 1
    if o is None:
        o = torch.empty((H, T, dv), dtype=v.dtype, device=v.device)
    if output_final_state and S_final is None:
        S_final = torch.empty((n_seq, H, dk, dv), dtype=torch.float32, device=v.device)
    if S0 is not None and S0.dtype != torch.float32:
        raise TypeError("S0 must be float32")
    shape = _varlen_shape(q, v, log_alpha, beta, n_seq)
    lib = library()
    ws = lib.kda_chunk_fwd_varlen_workspace_bytes(ctypes.byref(shape), int(max_seqlen))
    if workspace is None:
        workspace = torch.empty(ws, dtype=torch.uint8, device=v.device) if ws else None
    else:
        _require(workspace, "workspace")
    ws_given = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = lib.kda_chunk_fwd_varlen(ctypes.byref(shape), flags, _ptr(cu_seqlens), int(max_seqlen),
                                  _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                                  _ptr(S0), _ptr(o),
                                  _ptr(S_final) if output_final_state else None,
                                  _ptr(workspace), ws_given, _stream(v))
    _check(rc)
    return o, (S_final if output_final_state else None)


def linear_attn_fwd(q, k, v, S0=None, z0=None, *, output_final_state: bool = True, o=None,
                    S_final=None, z_final=None, workspace=None):
    """Normalized linear attention, phi = elu + 1: returns (o, S_final, z_final).

    q, k: [B,H,L,dk] raw (before phi); v: [B,H,L,dv] (bf16 or fp32, same
    dtype); S0: [B,H,dk,dv] fp32 or None; z0: [B,H,dk] fp32 or None.  The
    final state and normalizer are fp32 (None unless output_final_state).
    ``workspace``: a uint8 GPU tensor of at least
    kda_linear_attn_fwd_workspace_bytes bytes (else one is allocated per call).
    """
    torch = _torch()
    B, H, L, dk = q.shape
    dv = v.shape[-1]
    for name, t in (("q", q), ("k", k), ("v", v), ("S0", S0), ("z0", z0)):
        if t is not None:
            _require(t, name)
    for name, t in (("S0", S0), ("z0", z0)):
        if t is not None and t.dtype != torch.float32:
            raise TypeError(f"{name} must be float32")
    if o is None:
        o = torch.empty((B, H, L, dv), dtype=v.dtype, device=v.device)
    if output_final_state:
        if S_final is None:
            S_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=v.device)
        if z_final is None:
            z_final = torch.empty((B, H, dk), dtype=torch.float32, device=v.device)
    shape = KdaShape(B, H, L, dk, dv, _dtype_code(q), KDA_F32, KDA_ALPHA_NONE)
    lib = library()
    ws = lib.kda_linear_attn_fwd_workspace_bytes(ctypes.byref(shape))
    if workspace is None:
        workspace = torch.empty(ws, dtype=torch.uint8, device=v.device) if ws else None
    else:
        _require(workspace, "workspace")
    ws_given = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = lib.kda_linear_attn_fwd(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(S0),
                                 _ptr(z0), _ptr(o),
                                 _ptr(S_final) if output_final_state else None,
                                 _ptr(z_final) if output_final_state else None,
                                 _ptr(workspace), ws_given, _stream(v))
    _check(rc)
    if not output_final_state:
        return o, None, None
    return o, S_final, z_final


def linear_attn_decode_step(q, k, v, S, z, *, o=None):
    """One normalized linear attention step (phi = elu + 1) for every (b, h):
    S [B,H,dk,dv] and z [B,H,dk] fp32 are updated in place.  q, k: [B,H,dk]
    raw; v: [B,H,dv].  Returns o [B,H,dv]."""
    torch = _torch()
    B, H, dk = q.shape
    dv = v.shape[-1]
    for name, t in (("q", q), ("k", k), ("v", v), ("S", S), ("z", z)):
        _require(t, name)
    if S.dtype != torch.float32 or z.dtype != torch.float32:
        raise TypeError("S and z must be float32")
    if o is None:
        o = torch.empty((B, H, dv), dtype=v.dtype, device=v.device)
    shape = KdaShape(B, H, 1, dk, dv, _dtype_code(q), KDA_F32, KDA_ALPHA_NONE)
    rc = library().kda_linear_attn_decode_step(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v),
                                               _ptr(S), _ptr(z), _ptr(o), _stream(v))
    _check(rc)
    return o


def decode_step(q, k, v, log_alpha, beta, S, *, o=None, flags: Optional[int] = None):
    """One decode step for every (b, h); S [B,H,dk,dv] fp32 is updated in place.

    q, k: [B,H,dk]; v: [B,H,dv]; log_alpha: None, [B,H] or [B,H,dk];
    beta: [B,H].  Returns o [B,H,dv].  ``flags`` as in chunk_fwd
    (kda_decode_step_ex).
    """
    torch = _torch()
    B, H, dk = q.shape
    dv = v.shape[-1]
    if log_alpha is None:
        mode = KDA_ALPHA_NONE
    elif log_alpha.dim() == 2:
        mode = KDA_ALPHA_HEAD
    else:
        mode = KDA_ALPHA_CHANNEL
    for name, t in (("q", q), ("k", k), ("v", v), ("beta", beta), ("log_alpha", log_alpha),
                    ("S", S)):
        if t is not None:
            _require(t, name)
    if S.dtype != torch.float32:
        raise TypeError("S must be float32")
    if o is None:
        o = torch.empty((B, H, dv), dtype=v.dtype, device=v.device)
    shape = KdaShape(B, H, 1, dk, dv, _dtype_code(q),
                     _dtype_code(log_alpha if log_alpha is not None else beta), mode)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S), _ptr(o),
            _stream(v))
    if flags is None:
        rc = library().kda_decode_step(ctypes.byref(shape), *args)
    else:
        rc = library().kda_decode_step_ex(ctypes.byref(shape), flags, *args)
    _check(rc)
    return o


def decode_step_slots(q, k, v, log_alpha, beta, S_pool, slots, *, o=None,
                      flags: Optional[int] = None):
    """One decode step where sequence b uses state slot slots[b] of S_pool.

    q, k: [B,H,dk]; v: [B,H,dv]; log_alpha: None, [B,H] or [B,H,dk];
    beta: [B,H]; S_pool: [n_slots,H,dk,dv] fp32, updated in place at the used
    slots; slots: int32 [B] on the GPU (a slot outside [0, n_slots) marks an
    idle sequence whose o is zero).  Returns o [B,H,dv].  ``flags`` as in
    chunk_fwd (kda_decode_step_slots_ex).
    """
    torch = _torch()
    B, H, dk = q.shape
    dv = v.shape[-1]
    if log_alpha is None:
        mode = KDA_ALPHA_NONE
    elif log_alpha.dim() == 2:
        mode = KDA_ALPHA_HEAD
    else:
        mode = KDA_ALPHA_CHANNEL
    for name, t in (("q", q), ("k", k), ("v", v), ("beta", beta), ("log_alpha", log_alpha),
                    ("S_pool", S_pool), ("slots", slots)):
        if t is not None:
            _require(t, name)
    if S_pool.dtype != torch.float32:
        raise TypeError("S_pool must be float32")
    if slots.dtype != torch.int32:
        raise TypeError("slots must be int32")
    if o is None:
        o = torch.empty((B, H, dv), dtype=v.dtype, device=v.device)
    shape = KdaShape(B, H, 1, dk, dv, _dtype_code(q),
                     _dtype_code(log_alpha if log_alpha is not None else beta), mode)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S_pool),
            S_pool.shape[0], _ptr(slots), _ptr(o), _stream(v))
    if flags is None:
        rc = library().kda_decode_step_slots(ctypes.byref(shape), *args)
    else:
        rc = library().kda_decode_step_slots_ex(ctypes.byref(shape), flags, *args)
    _check(rc)
    return o
