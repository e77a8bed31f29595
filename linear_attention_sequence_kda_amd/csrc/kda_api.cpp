// kda_api.cpp -- the C ABI of libkda: argument checks, then kernel launches.
//
// Every check runs on the host before any HIP call, so rejected calls touch
// neither the device nor any buffer (and can be exercised without a GPU).
#include <limits.h>
#include <stdint.h>
#include <string.h>

#include <string>

#include "kda.h"
#include "kda_internal.h"

namespace {

thread_local std::string g_last_error;

struct Span {
    uintptr_t lo = 0, hi = 0;  // [lo, hi); empty when lo == hi
};

Span span_of(const void* p, int64_t bytes) {
    Span s;
    if (p && bytes > 0) {
        s.lo = (uintptr_t)p;
        s.hi = s.lo + (uintptr_t)bytes;
    }
    return s;
}

bool overlaps(const Span& a, const Span& b) {
    return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int elem_size(int32_t dtype) { return dtype == KDA_BF16 ? 2 : 4; }

// a * b with an overflow check against INT64_MAX / 8 (room for byte counts)
bool mul_ok(int64_t a, int64_t b, int64_t* out) {
    const int64_t lim = INT64_MAX / 8;
    if (a < 0 || b < 0) return false;
    if (a != 0 && b > lim / a) return false;
    *out = a * b;
    return true;
}

int check_shape(const kda_shape* s, bool decode) {
    if (!s) return KDA_ERR_NULL;
    if ((s->qkv_dtype != KDA_F32 && s->qkv_dtype != KDA_BF16) ||
        (s->gate_dtype != KDA_F32 && s->gate_dtype != KDA_BF16))
        return KDA_ERR_DTYPE;
    if (s->alpha_mode != KDA_ALPHA_NONE && s->alpha_mode != KDA_ALPHA_HEAD &&
        s->alpha_mode != KDA_ALPHA_CHANNEL)
        return KDA_ERR_ALPHA_MODE;
    if (s->B < 0 || s->H < 0 || s->L < 0) return KDA_ERR_SHAPE;
    if ((s->dk != 64 && s->dk != 128) || (s->dv != 64 && s->dv != 128)) return KDA_ERR_SHAPE;
    if (decode && s->L != 1) return KDA_ERR_SHAPE;
    int64_t bh, tok, x;
    if (!mul_ok(s->B, s->H, &bh)) return KDA_ERR_SHAPE;
    // one workgroup per (head, 16-column slice) at most: keep the grid in int
    if (bh > (int64_t)(INT_MAX / 8)) return KDA_ERR_SHAPE;
    if (!mul_ok(bh, s->L, &tok)) return KDA_ERR_SHAPE;
    if (!mul_ok(tok, 128, &x)) return KDA_ERR_SHAPE;
    return KDA_OK;
}

}  // namespace

extern "C" {

int kda_abi_version(void) { return KDA_ABI_VERSION; }

const char* kda_strerror(int status) {
    switch (status) {
        case KDA_OK: return "ok";
        case KDA_ERR_NULL: return "a required pointer is NULL";
        case KDA_ERR_SHAPE: return "unsupported or inconsistent shape (dk, dv must be 64 or 128; sizes >= 0; L == 1 for decode)";
        case KDA_ERR_DTYPE: return "unsupported dtype (KDA_F32 or KDA_BF16)";
        case KDA_ERR_ALPHA_MODE: return "unsupported alpha_mode";
        case KDA_ERR_ALIGN: return "a pointer is not 16-byte aligned";
        case KDA_ERR_WORKSPACE: return "workspace smaller than kda_chunk_fwd_workspace_bytes()";
        case KDA_ERR_ALIAS: return "an output buffer overlaps an input (or S_final partly overlaps S0)";
        case KDA_ERR_HIP: return "HIP launch failed";
        default: return "unknown kda status";
    }
}

const char* kda_last_error(void) { return g_last_error.c_str(); }

size_t kda_chunk_fwd_workspace_bytes(const kda_shape* shape) {
    (void)check_shape(shape, false);
    return 0;  // the fused kernel keeps every intermediate on chip
}

int kda_chunk_fwd(const kda_shape* s, const void* q, const void* k, const void* v,
                  const void* log_alpha, const void* beta, const float* S0, void* o,
                  float* S_final, void* workspace, size_t workspace_bytes,
                  void* hip_stream) {
    int rc = check_shape(s, false);
    if (rc != KDA_OK) return rc;
    const int64_t bh = s->B * s->H;
    const int64_t tok = bh * s->L;
    const int eq = elem_size(s->qkv_dtype), eg = elem_size(s->gate_dtype);
    const bool has_alpha = s->alpha_mode != KDA_ALPHA_NONE;

    if (tok > 0) {
        if (!q || !k || !v || !beta || !o) return KDA_ERR_NULL;
        if (has_alpha && !log_alpha) return KDA_ERR_NULL;
    }
    const void* ptrs[] = {q, k, v, has_alpha ? log_alpha : nullptr, beta, S0, o, S_final, workspace};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return KDA_ERR_ALIGN;
    if (workspace_bytes < kda_chunk_fwd_workspace_bytes(s)) return KDA_ERR_WORKSPACE;

    const int64_t la_elems = s->alpha_mode == KDA_ALPHA_CHANNEL ? tok * s->dk : tok;
    const Span sq = span_of(q, tok * s->dk * eq), sk = span_of(k, tok * s->dk * eq),
               sv = span_of(v, tok * s->dv * eq),
               sla = span_of(has_alpha ? log_alpha : nullptr, la_elems * eg),
               sb = span_of(beta, tok * eg), s0 = span_of(S0, bh * s->dk * s->dv * 4),
               so = span_of(o, tok * s->dv * eq), sf = span_of(S_final, bh * s->dk * s->dv * 4);
    const Span inputs[] = {sq, sk, sv, sla, sb};
    for (const Span& in : inputs)
        if (overlaps(so, in) || overlaps(sf, in)) return KDA_ERR_ALIAS;
    if (overlaps(so, s0) || overlaps(so, sf)) return KDA_ERR_ALIAS;
    if (overlaps(sf, s0) && (const void*)S_final != (const void*)S0) return KDA_ERR_ALIAS;

    if (bh == 0) return KDA_OK;
    kda::ChunkParams prm;
    prm.q = q;
    prm.k = k;
    prm.v = v;
    prm.log_alpha = has_alpha ? log_alpha : nullptr;
    prm.beta = beta;
    prm.S0 = S0;
    prm.o = o;
    prm.S_final = S_final;
    prm.L = s->L;
    prm.BH = (int)bh;
    prm.DV = (int)s->dv;
    prm.n_slices = 0;
    prm.gate_bf16 = s->gate_dtype == KDA_BF16;
    prm.alpha_mode = s->alpha_mode;
    const int qbf = s->qkv_dtype == KDA_BF16;
    const int nv = kda::chunk_slice_width((int)s->dk, (int)s->dv, qbf, bh);
    hipError_t err = kda::launch_chunk(prm, (int)s->dk, qbf, nv, (hipStream_t)hip_stream);
    if (err != hipSuccess) {
        g_last_error = std::string("kda_chunk_fwd: ") + hipGetErrorString(err);
        return KDA_ERR_HIP;
    }
    return KDA_OK;
}

int kda_decode_step(const kda_shape* s, const void* q, const void* k, const void* v,
                    const void* log_alpha, const void* beta, float* S, void* o,
                    void* hip_stream) {
    int rc = check_shape(s, true);
    if (rc != KDA_OK) return rc;
    const int64_t bh = s->B * s->H;
    const int eq = elem_size(s->qkv_dtype), eg = elem_size(s->gate_dtype);
    const bool has_alpha = s->alpha_mode != KDA_ALPHA_NONE;
    if (bh > 0) {
        if (!q || !k || !v || !beta || !S || !o) return KDA_ERR_NULL;
        if (has_alpha && !log_alpha) return KDA_ERR_NULL;
    }
    const void* ptrs[] = {q, k, v, has_alpha ? log_alpha : nullptr, beta, S, o};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return KDA_ERR_ALIGN;

    const int64_t la_elems = s->alpha_mode == KDA_ALPHA_CHANNEL ? bh * s->dk : bh;
    const Span sq = span_of(q, bh * s->dk * eq), sk = span_of(k, bh * s->dk * eq),
               sv = span_of(v, bh * s->dv * eq),
               sla = span_of(has_alpha ? log_alpha : nullptr, la_elems * eg),
               sb = span_of(beta, bh * eg), ss = span_of(S, bh * s->dk * s->dv * 4),
               so = span_of(o, bh * s->dv * eq);
    const Span inputs[] = {sq, sk, sv, sla, sb};
    for (const Span& in : inputs)
        if (overlaps(so, in) || overlaps(ss, in)) return KDA_ERR_ALIAS;
    if (overlaps(so, ss)) return KDA_ERR_ALIAS;

    if (bh == 0) return KDA_OK;
    kda::DecodeParams prm;
    prm.q = q;
    prm.k = k;
    prm.v = v;
    prm.log_alpha = has_alpha ? log_alpha : nullptr;
    prm.beta = beta;
    prm.S = S;
    prm.o = o;
    prm.BH = (int)bh;
    prm.gate_bf16 = s->gate_dtype == KDA_BF16;
    prm.alpha_mode = s->alpha_mode;
    hipError_t err = kda::launch_decode(prm, (int)s->dk, (int)s->dv,
                                        s->qkv_dtype == KDA_BF16, (hipStream_t)hip_stream);
    if (err != hipSuccess) {
        g_last_error = std::string("kda_decode_step: ") + hipGetErrorString(err);
        return KDA_ERR_HIP;
    }
    return KDA_OK;
}

}  // extern "C"
