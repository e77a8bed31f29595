"""The C ABI without a GPU: the library loads, exports what kda.h declares, and
rejects bad arguments on the host before any HIP call.

Pointers here are plain integers that are never dereferenced: every call made
below fails validation (or is an empty problem) and returns before touching
the device.
"""

import ctypes

import pytest

from linear_attention_sequence_kda_amd import binding

BASE = 0x7F0000000000  # 16-byte aligned fake device addresses, never dereferenced
MB = 1 << 20


@pytest.fixture(scope="module")
def lib():
    return binding.library()


def test_exports_every_declared_function(lib):
    names = binding.header_functions()
    assert set(names) >= {"kda_chunk_fwd", "kda_decode_step", "kda_chunk_fwd_workspace_bytes",
                          "kda_strerror", "kda_last_error", "kda_abi_version"}
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_strings(lib):
    assert lib.kda_abi_version() == 1
    for code in range(11):
        assert lib.kda_strerror(code)
    assert lib.kda_strerror(0) == b"ok"
    assert lib.kda_last_error() == b""


def shape(B=2, H=3, L=100, dk=128, dv=128, qd=binding.KDA_BF16, gd=binding.KDA_F32,
          mode=binding.KDA_ALPHA_CHANNEL):
    return binding.KdaShape(B, H, L, dk, dv, qd, gd, mode)


def bufs():
    """Disjoint fake buffers, 64 MiB apart (the workspace last, 1 GiB)."""
    names = ["q", "k", "v", "la", "beta", "S0", "o", "Sf", "ws"]
    return {n: BASE + i * 64 * MB for i, n in enumerate(names)}


def chunk(lib, s, b, wsb=1 << 30):
    return lib.kda_chunk_fwd(ctypes.byref(s) if s is not None else None, b["q"], b["k"], b["v"],
                             b["la"], b["beta"], b["S0"], b["o"], b["Sf"], b["ws"], wsb, None)


def decode(lib, s, b):
    return lib.kda_decode_step(ctypes.byref(s) if s is not None else None, b["q"], b["k"],
                               b["v"], b["la"], b["beta"], b["S0"], b["o"], None)


def test_workspace_query(lib):
    # one record per (head, chunk) of a span of chunks, plus a state area when
    # the sequence runs as several spans
    s = shape(B=2, H=3, L=100)
    ws = lib.kda_chunk_fwd_workspace_bytes(ctypes.byref(s))
    assert ws > 0 and ws % 256 == 0
    assert lib.kda_chunk_fwd_workspace_bytes(ctypes.byref(shape(L=10 ** 6))) <= (160 << 20) + 6 * 128 * 128 * 4
    assert lib.kda_chunk_fwd_workspace_bytes(ctypes.byref(shape(B=0))) == 0
    assert lib.kda_chunk_fwd_workspace_bytes(ctypes.byref(shape(L=0))) == 0
    assert lib.kda_chunk_fwd_workspace_bytes(None) == 0
    bad = shape()
    bad.dk = 96
    assert lib.kda_chunk_fwd_workspace_bytes(ctypes.byref(bad)) == 0


def test_workspace_too_small(lib):
    s = shape()
    ws = lib.kda_chunk_fwd_workspace_bytes(ctypes.byref(s))
    assert chunk(lib, s, bufs(), wsb=ws - 1) == 6  # KDA_ERR_WORKSPACE
    b = bufs()
    b["ws"] = None
    assert chunk(lib, s, b) == 6


def test_workspace_overlap(lib):
    b = bufs()
    b["ws"] = b["v"] + 4096
    assert chunk(lib, shape(), b) == 7


def test_long_sequence_rejected(lib):
    # one head's [L, d] tensors must stay addressable with 32-bit byte offsets
    assert chunk(lib, shape(B=1, H=1, L=1 << 23), bufs()) == 2


def test_null_shape(lib):
    assert chunk(lib, None, bufs()) == 1  # KDA_ERR_NULL
    assert decode(lib, None, bufs()) == 1


@pytest.mark.parametrize("field,value,code", [
    ("qkv_dtype", 7, 3), ("gate_dtype", -1, 3), ("alpha_mode", 3, 4), ("dk", 96, 2),
    ("dv", 32, 2), ("B", -1, 2), ("L", -5, 2), ("H", 1 << 40, 2)])
def test_bad_shape_fields(lib, field, value, code):
    s = shape()
    setattr(s, field, value)
    assert chunk(lib, s, bufs()) == code


def test_decode_requires_L1(lib):
    s = shape(L=2)
    assert decode(lib, s, bufs()) == 2
    s = shape(L=0)
    assert decode(lib, s, bufs()) == 2


@pytest.mark.parametrize("name", ["q", "k", "v", "beta", "o"])
def test_null_pointers(lib, name):
    b = bufs()
    b[name] = None
    assert chunk(lib, shape(), b) == 1


def test_null_log_alpha_only_allowed_without_decay(lib):
    b = bufs()
    b["la"] = None
    assert chunk(lib, shape(mode=binding.KDA_ALPHA_HEAD), b) == 1
    # with alpha_mode NONE, log_alpha is ignored; misalign something else to stop
    # the call before any launch
    b["q"] += 2
    assert chunk(lib, shape(mode=binding.KDA_ALPHA_NONE), b) == 5


@pytest.mark.parametrize("name", ["q", "k", "v", "la", "beta", "S0", "o", "Sf"])
def test_misaligned(lib, name):
    b = bufs()
    b[name] += 8
    assert chunk(lib, shape(), b) == 5


def test_aliasing(lib):
    b = bufs()
    b["o"] = b["q"] + 1024          # o overlaps q
    assert chunk(lib, shape(), b) == 7
    b = bufs()
    b["Sf"] = b["S0"] + 4096        # partial overlap of S_final and S0
    assert chunk(lib, shape(), b) == 7
    b = bufs()
    b["Sf"] = b["v"]                # final state written over an input
    assert chunk(lib, shape(), b) == 7
    b = bufs()
    b["o"] = b["S0"]                # decode: o overlapping S is rejected too
    assert decode(lib, shape(L=1), b) == 7


def test_empty_problem_is_ok_without_buffers(lib):
    # B*H == 0: nothing to do, no pointer needed, no HIP call made
    none = {n: None for n in bufs()}
    assert chunk(lib, shape(B=0), none) == 0
    assert decode(lib, shape(B=0, L=1), none) == 0


def test_header_mentions_every_status():
    text = open(binding.HEADER).read()
    for name in binding.STATUS.values():
        assert name in text


def test_timing_calls_without_launches(lib):
    n, ms = ctypes.c_int64(-1), ctypes.c_double(-1.0)
    assert lib.kda_timing_read(None, ctypes.byref(n), ctypes.byref(ms)) == 1
    assert lib.kda_timing_read(b"kda_intra_kernel", None, ctypes.byref(ms)) == 1
    assert lib.kda_timing_read(b"no_such_kernel", ctypes.byref(n), ctypes.byref(ms)) == 2
    assert lib.kda_timing_enable(1) == 0
    try:
        # a rejected call launches nothing, so nothing is recorded
        assert chunk(lib, shape(dk=96), bufs()) == 2
        for name in binding.KERNELS:
            assert lib.kda_timing_read(name.encode(), ctypes.byref(n), ctypes.byref(ms)) == 0
            assert n.value == 0 and ms.value == 0.0
    finally:
        assert lib.kda_timing_enable(0) == 0
        assert lib.kda_timing_reset() == 0


def decode_slots(lib, s, b, n_slots=4, slots=None):
    return lib.kda_decode_step_slots(ctypes.byref(s) if s is not None else None, b["q"], b["k"],
                                     b["v"], b["la"], b["beta"], b["S0"], n_slots,
                                     b["ws"] if slots is None else slots, b["o"], None)


def test_decode_slots_host_checks(lib):
    s = shape(L=1)
    b = bufs()
    assert lib.kda_decode_step_slots(ctypes.byref(s), b["q"], b["k"], b["v"], b["la"], b["beta"],
                                     b["S0"], 4, None, b["o"], None) == 1
    assert decode_slots(lib, s, b, n_slots=-1) == 2
    assert decode_slots(lib, shape(L=2), b) == 2
    assert decode_slots(lib, s, b, slots=b["ws"] + 2) == 5
    assert decode_slots(lib, s, b, slots=b["o"]) == 7            # slots overlap o
    assert decode_slots(lib, s, dict(b, o=b["S0"] + 64)) == 7    # o inside the pool
    assert decode_slots(lib, shape(B=0, L=1), b) == 0           # empty: nothing to do


def test_input_flags_host_checks(lib):
    """Unknown kda_input_flags bits are rejected before any other work; known
    bits pass the flag check and reach the ordinary argument checks."""
    b = bufs()
    s = shape()
    args = (b["q"], b["k"], b["v"], b["la"], b["beta"], b["S0"], b["o"], b["Sf"], b["ws"],
            1 << 30, None)
    for bad in (8, 16, 1 << 31, 0xFFFFFFFF):
        assert lib.kda_chunk_fwd_ex(ctypes.byref(s), bad, *args) == 9
        d = shape(L=1)
        assert lib.kda_decode_step_ex(ctypes.byref(d), bad, b["q"], b["k"], b["v"], b["la"],
                                      b["beta"], b["S0"], b["o"], None) == 9
        assert lib.kda_decode_step_slots_ex(ctypes.byref(d), bad, b["q"], b["k"], b["v"],
                                            b["la"], b["beta"], b["S0"], 4, b["ws"], b["o"],
                                            None) == 9
    assert b"flags" in lib.kda_strerror(9)
    all_bits = binding.NORM_QK | binding.BETA_LOGIT | binding.GATE_RAW
    # a valid flag set with a bad shape fails on the shape, as the plain call does
    assert lib.kda_chunk_fwd_ex(ctypes.byref(shape(dk=96)), all_bits, *args) == 2
    assert lib.kda_chunk_fwd_ex(ctypes.byref(s), all_bits, b["q"], None, *args[2:]) == 1
    assert lib.kda_decode_step_ex(ctypes.byref(shape(L=2)), all_bits, b["q"], b["k"], b["v"],
                                  b["la"], b["beta"], b["S0"], b["o"], None) == 2
    # empty problems are fine with any valid flag set
    none = {n: None for n in bufs()}
    assert lib.kda_chunk_fwd_ex(ctypes.byref(shape(B=0)), all_bits, none["q"], none["k"],
                                none["v"], none["la"], none["beta"], none["S0"], none["o"],
                                none["Sf"], none["ws"], 0, None) == 0


def test_flag_values_match_header():
    text = open(binding.HEADER).read()
    for name, val in (("KDA_IN_NORM_QK", binding.NORM_QK), ("KDA_IN_BETA_LOGIT",
                      binding.BETA_LOGIT), ("KDA_IN_GATE_RAW", binding.GATE_RAW)):
        assert f"{name} = {val}" in text


def varlen(lib, s, b, max_len, cu=None, flags=0, wsb=1 << 30):
    return lib.kda_chunk_fwd_varlen(ctypes.byref(s) if s is not None else None, flags,
                                    b["cu"] if cu is None else cu, max_len, b["q"], b["k"],
                                    b["v"], b["la"], b["beta"], b["S0"], b["o"], b["Sf"],
                                    b["ws"], wsb, None)


def test_varlen_host_checks(lib):
    """Packed sequences: B = sequences, L = total tokens; the token offsets are
    an input on the device, max_seqlen sizes the plan."""
    b = dict(bufs(), cu=BASE + 20 * 64 * MB)
    s = shape(B=3, H=4, L=1000)
    assert varlen(lib, s, b, -1) == 2
    assert varlen(lib, s, b, 500, cu=0) == 1           # no offsets with N > 0
    assert varlen(lib, s, b, 500, cu=b["cu"] + 2) == 5
    assert varlen(lib, s, b, 500, cu=b["o"]) == 7      # offsets overlap o
    assert varlen(lib, s, b, 500, cu=b["ws"]) == 7     # or the workspace
    assert varlen(lib, s, b, 500, flags=8) == 9
    assert varlen(lib, shape(B=3, H=4, L=1000, dk=96), b, 500) == 2
    assert varlen(lib, s, b, 500, wsb=16) == 6         # workspace too small
    # the workspace follows the longest sequence: that of a dense [N, H, max] call
    for n, T, m in ((3, 1000, 500), (2, 8192, 8192), (5, 4096, 64), (7, 300, 0)):
        for mode in (binding.KDA_ALPHA_CHANNEL, binding.KDA_ALPHA_HEAD):
            sv = shape(B=n, H=32, L=T, mode=mode)
            got = lib.kda_chunk_fwd_varlen_workspace_bytes(ctypes.byref(sv), m)
            want = lib.kda_chunk_fwd_workspace_bytes(ctypes.byref(shape(B=n, H=32, L=m,
                                                                        mode=mode)))
            assert got == want
    # no sequence is longer than T: a larger max_seqlen plans for T
    assert (lib.kda_chunk_fwd_varlen_workspace_bytes(ctypes.byref(s), 10 ** 9)
            == lib.kda_chunk_fwd_varlen_workspace_bytes(ctypes.byref(s), 1000))
    assert lib.kda_chunk_fwd_varlen_workspace_bytes(ctypes.byref(s), -5) == 0
    # no sequences: nothing to do, no pointer needed
    none = {n: None for n in b}
    assert varlen(lib, shape(B=0, H=4, L=0), none, 0) == 0


def test_linear_attn_host_checks(lib):
    b = dict(bufs(), z0=BASE + 21 * 64 * MB, zf=BASE + 22 * 64 * MB)
    s = shape(mode=binding.KDA_ALPHA_NONE)

    def la(s_, wsb=1 << 30, **kw):
        x = dict(b, **kw)
        return lib.kda_linear_attn_fwd(ctypes.byref(s_) if s_ is not None else None, x["q"],
                                       x["k"], x["v"], x["S0"], x["z0"], x["o"], x["Sf"],
                                       x["zf"], x["ws"], wsb, None)
    assert la(None) == 1
    assert la(shape(mode=binding.KDA_ALPHA_CHANNEL)) == 4     # no decay in this op
    assert la(shape(mode=binding.KDA_ALPHA_NONE, dk=96)) == 2
    assert la(s, q=0) == 1
    assert la(s, z0=b["z0"] + 4) == 5
    assert la(s, o=b["q"]) == 7
    assert la(s, zf=b["v"]) == 7
    assert la(s, zf=b["Sf"]) == 7
    assert la(s, zf=b["z0"] + 16) == 7                       # partial overlap with z0
    assert la(s, ws=b["v"]) == 7                             # workspace over an input
    # phi(q) in the input type
    need = lib.kda_linear_attn_fwd_workspace_bytes(ctypes.byref(s))
    assert need == 2 * 3 * 100 * 128 * 2
    assert la(s, wsb=need - 1) == 6
    assert lib.kda_linear_attn_fwd_workspace_bytes(ctypes.byref(shape())) == 0  # has decay
    none = {n: None for n in b}
    assert la(shape(B=0, mode=binding.KDA_ALPHA_NONE), wsb=0, **none) == 0


def test_linear_attn_decode_host_checks(lib):
    b = dict(bufs(), z=BASE + 21 * 64 * MB)

    def st(s_, **kw):
        x = dict(b, **kw)
        return lib.kda_linear_attn_decode_step(ctypes.byref(s_) if s_ is not None else None,
                                               x["q"], x["k"], x["v"], x["S0"], x["z"], x["o"],
                                               None)
    s = shape(L=1, mode=binding.KDA_ALPHA_NONE)
    assert st(None) == 1
    assert st(shape(L=2, mode=binding.KDA_ALPHA_NONE)) == 2
    assert st(shape(L=1, mode=binding.KDA_ALPHA_HEAD)) == 4
    assert st(s, z=0) == 1
    assert st(s, z=b["z"] + 8) == 5
    assert st(s, z=b["S0"] + 64) == 7     # normalizer inside the state
    assert st(s, o=b["k"]) == 7
    none = {n: None for n in b}
    assert st(shape(B=0, L=1, mode=binding.KDA_ALPHA_NONE), **none) == 0


def bwd(lib, s, b, wsb=1 << 30):
    return lib.kda_recurrence_bwd(ctypes.byref(s) if s is not None else None, b["q"], b["k"],
                                  b["v"], b["la"], b["beta"], b["S0"], b["do"], b["dSf"],
                                  b["dq"], b["dk"], b["dv"], b["dla"], b["dbeta"], b["dS0"],
                                  b["ws"], wsb, None)


def bwd_bufs():
    names = ["q", "k", "v", "la", "beta", "S0", "do", "dSf", "dq", "dk", "dv", "dla", "dbeta",
             "dS0", "ws"]
    return {n: BASE + i * 64 * MB for i, n in enumerate(names)}


def test_recurrence_bwd_host_checks(lib):
    s = shape()
    # one fp32 state slice per (head, 8 tokens)
    ws = lib.kda_recurrence_bwd_workspace_bytes(ctypes.byref(s))
    assert ws == 2 * 3 * 13 * 128 * 128 * 4
    assert lib.kda_recurrence_bwd_workspace_bytes(ctypes.byref(shape(L=0))) == 0
    assert lib.kda_recurrence_bwd_workspace_bytes(None) == 0
    assert bwd(lib, None, bwd_bufs()) == 1
    assert bwd(lib, s, bwd_bufs(), wsb=ws - 1) == 6                 # workspace too small
    for name in ["q", "k", "v", "la", "beta", "do", "dq", "dk", "dv", "dla", "dbeta", "ws"]:
        b = bwd_bufs()
        b[name] = None
        assert bwd(lib, s, b) == 1, name                             # required pointer
    b = bwd_bufs()
    b["la"] = b["dla"] = None                                        # no decay: both unused
    assert bwd(lib, shape(mode=binding.KDA_ALPHA_NONE), b, wsb=0) == 6
    for name in bwd_bufs():
        b = bwd_bufs()
        b[name] += 8
        assert bwd(lib, s, b) == 5, name                             # misaligned
    for out, inp in [("dq", "q"), ("dv", "do"), ("dS0", "dSf"), ("dk", "dq"), ("ws", "dla"),
                     ("dbeta", "beta")]:
        b = bwd_bufs()
        b[out] = b[inp] + 1024
        assert bwd(lib, s, b) == 7, (out, inp)                       # overlap
    bad = shape()
    bad.dv = 96
    assert bwd(lib, bad, bwd_bufs()) == 2
    none = {n: None for n in bwd_bufs()}
    assert bwd(lib, shape(B=0), none) == 0                           # empty problem


def cbwd(lib, s, b, wsb=1 << 30):
    return lib.kda_chunk_bwd(ctypes.byref(s) if s is not None else None, b["q"], b["k"], b["v"],
                             b["la"], b["beta"], b["S0"], b["do"], b["dSf"], b["dq"], b["dk"],
                             b["dv"], b["dla"], b["dbeta"], b["dS0"], b["ws"], wsb, None)


def test_chunk_bwd_workspace_size(lib):
    """Per chunk of 64 tokens and head: the forward record, a reverse record
    (the same sections and dO in one more), T^T (fp32 64 x 64), the states S
    and G (fp32 dk x dv) and u, du (bf16 64 x dv); without a decay, zero
    per-channel fp32 ln(alpha) and an fp32 beta per token are added (a head
    gate is read per token by every channel)."""
    up = lambda x: (x + 255) // 256 * 256
    rec = 64 * 128 * 2 * 4 + 64 * 64 * 2 + 1024     # W, U, K^T, Q~ (bf16), P, decays
    rrec = rec + 64 * 128 * 2                        # and dO
    nch = 2 * 3 * 2                                   # B H ceil(100 / 64)
    want = (up(nch * rec) + up(nch * rrec) + up(nch * 64 * 64 * 4) +
            2 * up(nch * 128 * 128 * 4) + 2 * up(nch * 64 * 128 * 2))
    assert lib.kda_chunk_bwd_workspace_bytes(ctypes.byref(shape())) == want
    head = shape(mode=binding.KDA_ALPHA_HEAD)
    assert lib.kda_chunk_bwd_workspace_bytes(ctypes.byref(head)) == want
    none = shape(mode=binding.KDA_ALPHA_NONE)
    assert lib.kda_chunk_bwd_workspace_bytes(ctypes.byref(none)) == \
        want + up(600 * 128 * 4) + up(600 * 4)
    assert lib.kda_chunk_bwd_workspace_bytes(ctypes.byref(shape(qd=binding.KDA_F32))) == 0
    assert lib.kda_chunk_bwd_workspace_bytes(ctypes.byref(shape(L=0))) == 0
    assert lib.kda_chunk_bwd_workspace_bytes(None) == 0


def test_chunk_bwd_host_checks(lib):
    s = shape()
    ws = lib.kda_chunk_bwd_workspace_bytes(ctypes.byref(s))
    assert cbwd(lib, None, bwd_bufs()) == 1
    assert cbwd(lib, shape(qd=binding.KDA_F32), bwd_bufs()) == 3      # bf16 q/k/v/do only
    assert cbwd(lib, s, bwd_bufs(), wsb=ws - 1) == 6
    for name in ["q", "k", "v", "la", "beta", "do", "dq", "dk", "dv", "dla", "dbeta", "ws"]:
        b = bwd_bufs()
        b[name] = None
        assert cbwd(lib, s, b) == 1, name
    for name in bwd_bufs():
        b = bwd_bufs()
        b[name] += 8
        assert cbwd(lib, s, b) == 5, name
    for out, inp in [("dq", "q"), ("dv", "do"), ("dS0", "dSf"), ("dk", "dq"), ("ws", "dla"),
                     ("dbeta", "beta"), ("dS0", "ws")]:
        b = bwd_bufs()
        b[out] = b[inp] + 1024
        assert cbwd(lib, s, b) == 7, (out, inp)
    bad = shape()
    bad.dv = 96
    assert cbwd(lib, bad, bwd_bufs()) == 2
    none = {n: None for n in bwd_bufs()}
    assert cbwd(lib, shape(B=0), none) == 0


def bwd_ex(lib, s, flags, b, wsb=1 << 30):
    return lib.kda_recurrence_bwd_ex(ctypes.byref(s) if s is not None else None, flags, b["q"],
                                     b["k"], b["v"], b["la"], b["beta"], b["S0"], b["do"],
                                     b["dSf"], b["dq"], b["dk"], b["dv"], b["dla"], b["dbeta"],
                                     b["dS0"], b["ws"], wsb, None)


def test_recurrence_bwd_ex_host_checks(lib):
    s = shape()
    plain = lib.kda_recurrence_bwd_workspace_bytes(ctypes.byref(s))
    ws = lib.kda_recurrence_bwd_ex_workspace_bytes(ctypes.byref(s), 7)
    assert ws > plain                                  # plus the fp32 copies and norms
    assert lib.kda_recurrence_bwd_ex_workspace_bytes(ctypes.byref(s), 8) == 0
    assert lib.kda_recurrence_bwd_ex_workspace_bytes(ctypes.byref(shape(L=0)), 7) == 0
    assert bwd_ex(lib, s, 8, bwd_bufs()) == 9          # unknown flag bit
    assert bwd_ex(lib, None, 7, bwd_bufs()) == 1
    assert bwd_ex(lib, s, 7, bwd_bufs(), wsb=ws - 1) == 6
    for name in ["q", "k", "v", "la", "beta", "do", "dq", "dk", "dv", "dla", "dbeta", "ws"]:
        b = bwd_bufs()
        b[name] = None
        assert bwd_ex(lib, s, 7, b) == 1, name
    for name in bwd_bufs():
        b = bwd_bufs()
        b[name] += 8
        assert bwd_ex(lib, s, 7, b) == 5, name
    for out, inp in [("dq", "q"), ("ws", "k"), ("dbeta", "beta"), ("dS0", "S0")]:
        b = bwd_bufs()
        b[out] = b[inp] + 1024
        assert bwd_ex(lib, s, 7, b) == 7, (out, inp)
    none = {n: None for n in bwd_bufs()}
    assert bwd_ex(lib, shape(B=0), 7, none) == 0


def test_recurrence_bwd_ex_outputs_against_workspace_and_each_other(lib):
    """Every output is checked against the whole raw-input workspace (its fp32
    copies and row norms) and against the other outputs before anything is
    enqueued."""
    s = shape()
    ws = lib.kda_recurrence_bwd_ex_workspace_bytes(ctypes.byref(s), 7)
    plain = lib.kda_recurrence_bwd_workspace_bytes(ctypes.byref(s))
    for out in ["dq", "dk", "dv", "dla", "dbeta", "dS0"]:
        # inside the workspace, past the gradient kernel's own area (the
        # fp32 copies and the norms at its end)
        for off in (plain + 4096, ws - 4096):
            b = bwd_bufs()
            b[out] = b["ws"] + (off // 256) * 256
            assert bwd_ex(lib, s, 7, b) == 7, (out, off)
    for a, c in [("dq", "dk"), ("dv", "dbeta"), ("dla", "dS0"), ("dk", "dv")]:
        b = bwd_bufs()
        b[a] = b[c] + 1024
        assert bwd_ex(lib, s, 7, b) == 7, (a, c)


def test_recurrence_bwd_ex_row_limit(lib):
    """The prep and post kernels take one 64-lane workgroup per token row:
    more rows than 2^32 / 64 are rejected on the host."""
    # 17 x 4,000,000 rows: a valid shape otherwise (L within the per-head
    # limit), just above 2^26 rows
    s = shape(B=17, H=1, L=4_000_000, dk=64, dv=64)
    assert lib.kda_recurrence_bwd_workspace_bytes(ctypes.byref(s)) > 0
    b = {n: BASE + i * (1 << 40) for i, n in enumerate(bwd_bufs())}
    assert bwd_ex(lib, s, 7, b, wsb=1 << 62) == 2


def noalloc(lib, s, flags, b):
    return lib.kda_chunk_fwd_noalloc(ctypes.byref(s) if s is not None else None, flags, b["q"],
                                     b["k"], b["v"], b["la"], b["beta"], b["S0"], b["o"], b["Sf"],
                                     None)


def test_noalloc_host_checks(lib):
    """kda_chunk_fwd_noalloc makes kda_chunk_fwd_ex's host checks, and rejects
    a problem whose one-chunk span does not fit its static buffer, all before
    any HIP call (no device here)."""
    s = shape()
    assert noalloc(lib, None, 0, bufs()) == 1
    assert noalloc(lib, s, 8, bufs()) == 9                         # unknown flag bit
    for name in ["q", "k", "v", "la", "beta", "o"]:
        b = bufs()
        b[name] = None
        assert noalloc(lib, s, 0, b) == 1, name
    for name in ["q", "k", "v", "la", "beta", "S0", "o", "Sf"]:
        b = bufs()
        b[name] += 8
        assert noalloc(lib, s, 0, b) == 5, name
    b = bufs()
    b["o"] = b["q"] + 1024
    assert noalloc(lib, s, 0, b) == 7
    bad = shape()
    bad.dk = 96
    assert noalloc(lib, bad, 0, bufs()) == 2
    # per-channel decay, d = 128, bf16: 73 KiB of records per (head, chunk),
    # so 1,024 heads need 75 MB for one chunk each: more than the 64 MiB buffer
    big = shape(B=8, H=128, L=64)
    b = {n: BASE + i * (1 << 36) for i, n in enumerate(bufs())}
    assert noalloc(lib, big, 0, b) == 10                           # KDA_ERR_SCRATCH
    assert lib.kda_strerror(10).startswith(b"the problem needs more work memory")
    # the same heads with one decay per head fit (9 KiB records)
    none = {n: None for n in bufs()}
    assert noalloc(lib, shape(B=0), 0, none) == 0                  # empty problem


# ---- host diagnostics (KDA_LOG) ---------------------------------------------
_LOG_PROG = r"""
import ctypes, sys
sys.path.insert(0, {root!r})
from linear_attention_sequence_kda_amd import binding
lib = binding.library()
B = 0x7F0000000000
s = binding.KdaShape(1, 2, 8, 96, 128, binding.KDA_BF16, binding.KDA_F32, binding.KDA_ALPHA_CHANNEL)
rc = lib.kda_chunk_fwd(ctypes.byref(s), B, B + (1 << 26), B + (2 << 26), B + (3 << 26), B + (4 << 26),
                       None, B + (5 << 26), None, None, 0, None)
rc2 = lib.kda_decode_step(None, B, B, B, B, B, B, B, None)
print("rc", rc, rc2)
"""


def _run_log_prog(env_value):
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ)
    env.pop("KDA_LOG", None)
    if env_value is not None:
        env["KDA_LOG"] = env_value
    return subprocess.run([sys.executable, "-c", _LOG_PROG.format(root=root)], env=env,
                          capture_output=True, text=True, timeout=120)


def test_log_reports_shape_and_status_of_rejected_calls():
    """KDA_LOG=1: each call's shape and its status when it is not KDA_OK go to
    stderr (checked on calls the host rejects, so no GPU is needed)."""
    p = _run_log_prog("1")
    assert p.returncode == 0, p.stderr
    assert "rc 2 1" in p.stdout  # KDA_ERR_SHAPE, KDA_ERR_NULL
    lines = [x for x in p.stderr.splitlines() if x.startswith("[kda] ")]
    assert any("kda_chunk_fwd: B=1 H=2 L=8 dk=96 dv=128 qkv=bf16 gate=f32 alpha=channel" in x for x in lines), lines
    assert any("kda_chunk_fwd: status 2: unsupported or inconsistent shape" in x
               for x in lines), lines
    assert any("kda_decode_step: no shape" in x for x in lines), lines
    assert any("kda_decode_step: status 1: a required pointer is NULL" in x
               for x in lines), lines


@pytest.mark.parametrize("value", [None, "0", ""])
def test_log_is_silent_unless_enabled(value):
    p = _run_log_prog(value)
    assert p.returncode == 0, p.stderr
    assert "[kda]" not in p.stderr


def test_library_links_profiler_ranges():
    """Every ABI call is one roctx range (rocprofiler-sdk's roctx library)."""
    import subprocess
    out = subprocess.run(["ldd", binding.LIB_PATH], capture_output=True, text=True).stdout
    assert "librocprofiler-sdk-roctx" in out


def test_longest_sequence_accepted_one_more_rejected(lib):
    """Kernels address one head's [L, d] rows with 32-bit byte offsets, so L is
    capped at INT_MAX / 512 (4,194,303 tokens: fp32 rows of 128 values): that L
    gets a plan, one more token is rejected as a shape error, before any HIP
    call (the calls below are host checks or return before launching)."""
    L_MAX = (2 ** 31 - 1) // 512
    for qd in (binding.KDA_BF16, binding.KDA_F32):
        ok = shape(B=1, H=1, L=L_MAX, qd=qd)
        assert lib.kda_chunk_fwd_workspace_bytes(ctypes.byref(ok)) > 0
        bad = shape(B=1, H=1, L=L_MAX + 1, qd=qd)
        assert lib.kda_chunk_fwd_workspace_bytes(ctypes.byref(bad)) == 0
        assert chunk(lib, bad, bufs()) == 2  # KDA_ERR_SHAPE
