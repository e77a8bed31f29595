// kda_api.cpp -- the C ABI of libkda: argument checks, then kernel launches.
//
// Every check runs on the host before any HIP call, so rejected calls touch
// neither the device nor any buffer (and can be exercised without a GPU).
#include <limits.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <rocprofiler-sdk-roctx/roctx.h>

#include <mutex>
#include <string>
#include <vector>

#include "kda.h"
#include "kda_internal.h"

namespace {

thread_local std::string g_last_error;

// ---- host diagnostics (KDA_LOG) and profiler ranges --------------------------
// KDA_LOG set to anything but "" or "0": every call writes its shape, the
// prefill plan and any status other than KDA_OK to stderr, one line each.
// Every call is also one roctx range named after the entry point, which
// rocprofv3 --marker-trace records beside the kernels it launched.
bool log_on() {
    static const bool on = [] {
        const char* e = getenv("KDA_LOG");
        return e && *e && strcmp(e, "0") != 0;
    }();
    return on;
}
void klog(const char* fmt, ...) {
    if (!log_on()) return;
    char line[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(line, sizeof line, fmt, ap);
    va_end(ap);
    fprintf(stderr, "[kda] %s\n", line);
    fflush(stderr);
}
const char* dtype_name(int32_t d) { return d == KDA_BF16 ? "bf16" : d == KDA_F32 ? "f32" : "?"; }
const char* alpha_name(int32_t a) {
    return a == KDA_ALPHA_NONE ? "none" : a == KDA_ALPHA_HEAD ? "head" : a == KDA_ALPHA_CHANNEL ? "channel" : "?";
}
struct CallScope {
    const char* who;
    CallScope(const char* w, const kda_shape* s, uint32_t flags) : who(w) {
        roctxRangePushA(w);
        if (!log_on()) return;
        if (s)
            klog("%s: B=%lld H=%lld L=%lld dk=%lld dv=%lld qkv=%s gate=%s alpha=%s flags=0x%x", w,
                 (long long)s->B, (long long)s->H, (long long)s->L, (long long)s->dk, (long long)s->dv,
                 dtype_name(s->qkv_dtype), dtype_name(s->gate_dtype), alpha_name(s->alpha_mode), flags);
        else
            klog("%s: no shape", w);
    }
    ~CallScope() { roctxRangePop(); }
    int done(int rc) const;
};

// ---- kernel timing (kda_timing_*) --------------------------------------------
// While enabled, each kernel launch is bracketed by two events recorded on the
// launch's stream; the pairs are kept until read or reset.
enum KernelId { K_INTRA = 0, K_INTER, K_INTER_SCALAR, K_DECODE, K_FEATURE, K_BWD, K_INTER_WIDE,
                K_INTER_QUAD, K_WIDE_SCAN, K_CHUNK_GRAD, K_GATE_WIDEN, K_COUNT };
// (kda_inter_wide_scan is kda_inter_wide_kernel in its scan form)
const char* const kKernelNames[K_COUNT] = {"kda_intra_kernel", "kda_inter_kernel",
                                           "kda_inter_scalar_kernel", "kda_decode_kernel",
                                           "kda_feature_map_kernel", "kda_bwd_kernel",
                                           "kda_inter_wide_kernel", "kda_inter_quad_kernel",
                                           "kda_inter_wide_scan", "kda_chunk_grad_kernel",
                                           "kda_gate_widen_kernel"};
struct TimedLaunch {
    int kernel;
    hipEvent_t start, stop;
};
std::mutex g_timing_mu;
bool g_timing_on = false;
std::vector<TimedLaunch> g_timed;

template <class Launch>
hipError_t timed_launch(int kernel, hipStream_t stream, Launch&& launch) {
    {
        std::lock_guard<std::mutex> lock(g_timing_mu);
        if (!g_timing_on) return launch();
    }
    TimedLaunch t{kernel, nullptr, nullptr};
    hipError_t err = hipEventCreate(&t.start);
    if (err == hipSuccess) err = hipEventCreate(&t.stop);
    if (err == hipSuccess) err = hipEventRecord(t.start, stream);
    if (err == hipSuccess) err = launch();
    if (err == hipSuccess) err = hipEventRecord(t.stop, stream);
    if (err != hipSuccess) {
        if (t.start) (void)hipEventDestroy(t.start);
        if (t.stop) (void)hipEventDestroy(t.stop);
        return err;
    }
    std::lock_guard<std::mutex> lock(g_timing_mu);
    g_timed.push_back(t);
    return hipSuccess;
}

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

constexpr uint32_t kAllFlags = KDA_IN_NORM_QK | KDA_IN_BETA_LOGIT | KDA_IN_GATE_RAW;

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
    // kernels address one head's [L, d] tensors with 32-bit byte offsets
    if (s->L > (int64_t)(INT_MAX / (128 * 4))) return KDA_ERR_SHAPE;
    return KDA_OK;
}

// ---- prefill plan: chunk spans and workspace ----------------------------------
// The intra-chunk kernel writes one record per (head, chunk) of a span of
// chunks, the inter-chunk kernel consumes them; long inputs run as several
// spans, so the records of one span stay within a bounded workspace (and, at
// the target size, within the 256 MiB memory-side cache of an MI355X).  Between
// spans the state goes through S_final, or through the workspace's state area
// when no final state is wanted.  When the state pass has a workgroup for
// every CU, longer spans are used: the intra-chunk grid then runs more rounds
// of workgroups per launch, which lets their input loads overlap other
// workgroups' work (measured on MI355X: the intra-chunk kernel 20% faster per
// chunk, the state pass unchanged); a state pass with fewer workgroups reads
// its records more slowly once they leave that cache, so it keeps spans whose
// records fit there beside the rest of the traffic.  The intra-chunk kernel
// reads its inputs with the non-temporal hint, which leaves that cache to the
// records: on the 16-head long-context shape 160 MiB (128-chunk) spans then
// measured 4% faster per call than 128 MiB (96 chunks, the best length with
// ordinary loads) and 160 and 192 chunks slower again; on 2 x 32 heads x 8192
// tokens (full chip) 48-chunk spans (229 MB of records) beat 32, 64, 80 and
// 128 chunks by 1-4%.
#ifndef KDA_SPAN_TARGET_BYTES
#define KDA_SPAN_TARGET_BYTES (160ll << 20)
#endif
constexpr int64_t kSpanTargetBytes = KDA_SPAN_TARGET_BYTES;
constexpr int64_t kFullChipSpanBytes = 240ll << 20;
constexpr int64_t kChipCUs = 256;

struct Plan {
    int C = 0;
    int64_t nchunks = 0, span = 0, nspans = 0;
    int64_t rec_bytes = 0, rec_area = 0, state_area = 0;
    int64_t ws_bytes = 0;
    bool fits = true;  // false: no plan fits the byte cap make_plan was given
};

// The plan above, shortened so that its workspace fits in cap bytes when cap
// >= 0 (kda_chunk_fwd_noalloc's static buffer): one span of every chunk if
// the records alone fit, else the longest spans that fit beside the state
// area; fits = false when not even one chunk per span does.
Plan make_plan(const kda_shape* s, int64_t cap = -1);

Plan make_plan_uncapped(const kda_shape* s) {
    Plan p;
    const int bf = s->qkv_dtype == KDA_BF16;
    const int64_t bh = s->B * s->H;
    p.C = kda::chunk_len(bf);
    p.nchunks = (s->L + p.C - 1) / p.C;
    if (bh == 0 || p.nchunks == 0) return p;
    p.rec_bytes = s->alpha_mode == KDA_ALPHA_CHANNEL
                      ? kda::rec_layout((int)s->dk, (int)s->dv, p.C, bf ? 2 : 4, true).bytes
                      : kda::rec_layout_thin(p.C, bf ? 2 : 4).bytes;
    int64_t per_chunk = bh * p.rec_bytes;
    const int wv = kda::wide_slice_width((int)s->dk, (int)s->dv, bf, s->alpha_mode, bh);
    const int nv = wv ? wv : kda::chunk_slice_width((int)s->dk, (int)s->dv, bf, bh);
    const bool full_chip = bh * (s->dv / nv) >= kChipCUs;
    p.span = (full_chip ? kFullChipSpanBytes : kSpanTargetBytes) / per_chunk;
    if (p.span < 1) p.span = 1;
    if (p.span < p.nchunks) {
        // Round the span down so one span's intra-chunk grid (B*H*span
        // workgroups) fills whole rounds of an MI355X's resident workgroups
        // (256 CUs x 2 for KDA records, x 4 otherwise): a partial last round
        // would leave most CUs idle.
        const int64_t slots = 256 * (s->alpha_mode == KDA_ALPHA_CHANNEL ? 2 : 4);
        int64_t a = bh, b = slots;
        while (b) {
            const int64_t t = a % b;
            a = b;
            b = t;
        }
        const int64_t unit = slots / a;  // smallest span with bh * span a multiple of slots
        if (unit <= p.span) p.span -= p.span % unit;
    }
    if (p.span > p.nchunks) p.span = p.nchunks;
    p.nspans = (p.nchunks + p.span - 1) / p.span;
    p.rec_area = p.span * per_chunk;
    p.state_area = p.nspans > 1 ? bh * s->dk * s->dv * 4 : 0;
    p.ws_bytes = p.rec_area + p.state_area;
    return p;
}

Plan make_plan(const kda_shape* s, int64_t cap) {
    Plan p = make_plan_uncapped(s);
    if (cap < 0 || p.ws_bytes <= cap) return p;
    const int64_t per_chunk = s->B * s->H * p.rec_bytes;
    if (p.nchunks * per_chunk <= cap) {
        p.span = p.nchunks;
    } else {
        const int64_t st = s->B * s->H * s->dk * s->dv * 4;
        p.span = cap > st ? (cap - st) / per_chunk : 0;
        if (p.span < 1) {
            p.fits = false;
            return p;
        }
    }
    p.nspans = (p.nchunks + p.span - 1) / p.span;
    p.rec_area = p.span * per_chunk;
    p.state_area = p.nspans > 1 ? s->B * s->H * s->dk * s->dv * 4 : 0;
    p.ws_bytes = p.rec_area + p.state_area;
    return p;
}

}  // namespace

namespace {
// Shared body of kda_decode_step (slots == nullptr: S is [B,H,dk,dv]) and
// kda_decode_step_slots (S is a pool of n_slots states).
int decode_body(const char* who, const kda_shape* s, uint32_t flags, const void* q,
                const void* k, const void* v, const void* log_alpha, const void* beta,
                float* S, int64_t n_slots, const int32_t* slots, void* o, void* hip_stream) {
    int rc = check_shape(s, true);
    if (rc != KDA_OK) return rc;
    if (flags & ~kAllFlags) return KDA_ERR_FLAGS;
    const int64_t bh = s->B * s->H;
    const int eq = elem_size(s->qkv_dtype), eg = elem_size(s->gate_dtype);
    const bool has_alpha = s->alpha_mode != KDA_ALPHA_NONE;
    if (slots && n_slots < 0) return KDA_ERR_SHAPE;
    int64_t state_elems = 0;
    if (!mul_ok(slots ? n_slots : s->B, s->H * s->dk * s->dv, &state_elems)) return KDA_ERR_SHAPE;
    if (bh > 0) {
        if (!q || !k || !v || !beta || !S || !o) return KDA_ERR_NULL;
        if (has_alpha && !log_alpha) return KDA_ERR_NULL;
    }
    const void* ptrs[] = {q, k, v, has_alpha ? log_alpha : nullptr, beta, S, o};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return KDA_ERR_ALIGN;
    if (slots && ((uintptr_t)slots & 3u)) return KDA_ERR_ALIGN;

    const int64_t la_elems = s->alpha_mode == KDA_ALPHA_CHANNEL ? bh * s->dk : bh;
    const Span sq = span_of(q, bh * s->dk * eq), sk = span_of(k, bh * s->dk * eq),
               sv = span_of(v, bh * s->dv * eq),
               sla = span_of(has_alpha ? log_alpha : nullptr, la_elems * eg),
               sb = span_of(beta, bh * eg), ss = span_of(S, state_elems * 4),
               so = span_of(o, bh * s->dv * eq),
               si = span_of(slots, slots ? s->B * 4 : 0);
    const Span inputs[] = {sq, sk, sv, sla, sb, si};
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
    prm.slots = slots;
    prm.n_slots = n_slots;
    prm.H = (int)s->H;
    prm.flags = flags;
    const hipStream_t stream = (hipStream_t)hip_stream;
    hipError_t err = timed_launch(K_DECODE, stream, [&] {
        return kda::launch_decode(prm, (int)s->dk, (int)s->dv, s->qkv_dtype == KDA_BF16, stream);
    });
    if (err != hipSuccess) {
        g_last_error = std::string(who) + ": " + hipGetErrorString(err);
        return KDA_ERR_HIP;
    }
    return KDA_OK;
}
int decode_common(const char* who, const kda_shape* s, uint32_t flags, const void* q,
                  const void* k, const void* v, const void* log_alpha, const void* beta,
                  float* S, int64_t n_slots, const int32_t* slots, void* o, void* hip_stream) {
    const CallScope sc(who, s, flags);
    return sc.done(decode_body(who, s, flags, q, k, v, log_alpha, beta, S, n_slots, slots, o, hip_stream));
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
        case KDA_ERR_FLAGS: return "unknown kda_input_flags bit";
        case KDA_ERR_SCRATCH: return "the problem needs more work memory than kda_chunk_fwd_noalloc's static buffer (KDA_NOALLOC_SCRATCH_BYTES) holds";
        default: return "unknown kda status";
    }
}

const char* kda_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"

namespace {
int CallScope::done(int rc) const {
    if (rc != KDA_OK)
        klog("%s: status %d: %s%s%s", who, rc, kda_strerror(rc), rc == KDA_ERR_HIP ? ": " : "",
             rc == KDA_ERR_HIP ? g_last_error.c_str() : "");
    return rc;
}
}  // namespace

extern "C" {

size_t kda_chunk_fwd_workspace_bytes(const kda_shape* shape) {
    if (check_shape(shape, false) != KDA_OK) return 0;
    return (size_t)make_plan(shape).ws_bytes;
}

int kda_chunk_fwd(const kda_shape* s, const void* q, const void* k, const void* v,
                  const void* log_alpha, const void* beta, const float* S0, void* o,
                  float* S_final, void* workspace, size_t workspace_bytes,
                  void* hip_stream) {
    return kda_chunk_fwd_ex(s, 0u, q, k, v, log_alpha, beta, S0, o, S_final, workspace,
                            workspace_bytes, hip_stream);
}

}  // extern "C"

namespace {
// Shared body of kda_chunk_fwd_ex (cu == nullptr: dense [B,H,L,*] tensors) and
// kda_chunk_fwd_varlen (B packed sequences in [H, L = T, *] tensors, token
// offsets cu on the device, the longest sequence max_len tokens).
// noalloc: kda_chunk_fwd_noalloc -- the plan is capped to the static buffer,
// whose address replaces workspace once every host check has passed, and no
// timing event is created.
int chunk_body(const char* who, const kda_shape* s, uint32_t flags, const int32_t* cu,
               int64_t max_len, const void* q, const void* k, const void* v,
               const void* log_alpha, const void* beta, const float* S0, void* o,
               float* S_final, void* workspace, size_t workspace_bytes, void* hip_stream,
               bool noalloc) {
    int rc = check_shape(s, false);
    if (rc != KDA_OK) return rc;
    if (flags & ~kAllFlags) return KDA_ERR_FLAGS;
    const bool packed = cu != nullptr || max_len >= 0;
    if (packed && max_len < 0) return KDA_ERR_SHAPE;
    const int64_t bh = s->B * s->H;
    // token rows of every [*, d] tensor: B H L dense, H T packed
    const int64_t tok = packed ? s->H * s->L : bh * s->L;
    const int eq = elem_size(s->qkv_dtype), eg = elem_size(s->gate_dtype);
    const bool has_alpha = s->alpha_mode != KDA_ALPHA_NONE;
    // the plan (spans, records) follows the longest sequence, which no
    // sequence of T tokens can exceed
    kda_shape ps = *s;
    if (packed) ps.L = max_len < s->L ? max_len : s->L;

    if (tok > 0) {
        if (!q || !k || !v || !beta || !o) return KDA_ERR_NULL;
        if (has_alpha && !log_alpha) return KDA_ERR_NULL;
    }
    if (packed && s->B > 0 && !cu) return KDA_ERR_NULL;
    const void* ptrs[] = {q, k, v, has_alpha ? log_alpha : nullptr, beta, S0, o, S_final, workspace};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return KDA_ERR_ALIGN;
    if (cu && ((uintptr_t)cu & 3u)) return KDA_ERR_ALIGN;
    const Plan plan = make_plan(&ps, noalloc ? (int64_t)KDA_NOALLOC_SCRATCH_BYTES : -1);
    if (!plan.fits) return KDA_ERR_SCRATCH;
    if (!noalloc && plan.ws_bytes > 0 && (!workspace || workspace_bytes < (size_t)plan.ws_bytes))
        return KDA_ERR_WORKSPACE;

    const int64_t la_elems = s->alpha_mode == KDA_ALPHA_CHANNEL ? tok * s->dk : tok;
    const Span sq = span_of(q, tok * s->dk * eq), sk = span_of(k, tok * s->dk * eq),
               sv = span_of(v, tok * s->dv * eq),
               sla = span_of(has_alpha ? log_alpha : nullptr, la_elems * eg),
               sb = span_of(beta, tok * eg), s0 = span_of(S0, bh * s->dk * s->dv * 4),
               so = span_of(o, tok * s->dv * eq), sf = span_of(S_final, bh * s->dk * s->dv * 4),
               sc = span_of(cu, packed ? (s->B + 1) * 4 : 0);
    const Span inputs[] = {sq, sk, sv, sla, sb, sc};
    for (const Span& in : inputs)
        if (overlaps(so, in) || overlaps(sf, in)) return KDA_ERR_ALIAS;
    if (overlaps(so, s0) || overlaps(so, sf)) return KDA_ERR_ALIAS;
    if (overlaps(sf, s0) && (const void*)S_final != (const void*)S0) return KDA_ERR_ALIAS;
    const Span sw = span_of(noalloc ? nullptr : workspace, plan.ws_bytes);
    const Span all[] = {sq, sk, sv, sla, sb, s0, so, sf, sc};
    for (const Span& x : all)
        if (overlaps(sw, x)) return KDA_ERR_ALIAS;

    if (bh == 0) return KDA_OK;
    const int qbf = s->qkv_dtype == KDA_BF16;
    const hipStream_t stream = (hipStream_t)hip_stream;
    if (noalloc) {
        hipError_t e = kda::scratch_address(&workspace);
        if (e != hipSuccess) {
            g_last_error = std::string(who) + ": " + hipGetErrorString(e);
            return KDA_ERR_HIP;
        }
    }
    // the allocation-free call records no timing events
    auto launch = [&](int kernel, auto&& fn) -> hipError_t {
        return noalloc ? fn() : timed_launch(kernel, stream, fn);
    };
    const int nv = kda::chunk_slice_width((int)s->dk, (int)s->dv, qbf, bh);
    // per-channel decay in bf16: the wide state pass (and the record order it reads)
    const int wv = kda::wide_slice_width((int)s->dk, (int)s->dv, qbf, s->alpha_mode, bh);
    float* s_mid = S_final ? S_final : (float*)((char*)workspace + plan.rec_area);
    if (log_on())
        klog("%s: %lld chunks of %d in %lld span(s) of %lld; record %lld B per chunk and head; "
             "workspace %lld B%s; state pass %s, %d-column slices", who, (long long)plan.nchunks, plan.C,
             (long long)plan.nspans, (long long)plan.span, (long long)plan.rec_bytes,
             (long long)plan.ws_bytes, noalloc ? " (static buffer)" : "",
             wv ? (wv == 16 ? "kda_inter_quad_kernel" : "kda_inter_wide_kernel")
                : (s->alpha_mode == KDA_ALPHA_CHANNEL ? "kda_inter_kernel" : "kda_inter_scalar_kernel"),
             wv ? wv : nv);

    kda::IntraParams ip;
    ip.q = q;
    ip.k = k;
    ip.v = v;
    ip.log_alpha = has_alpha ? log_alpha : nullptr;
    ip.beta = beta;
    ip.ws = workspace;
    ip.L = s->L;
    ip.BH = (int)bh;
    ip.gate_bf16 = s->gate_dtype == KDA_BF16;
    ip.flags = flags;
    ip.cu = cu;
    ip.H = (int)s->H;
    ip.wide = wv != 0;
    kda::InterParams xp;
    xp.q = q;
    xp.k = k;
    xp.v = v;
    xp.ws = workspace;
    xp.o = o;
    xp.L = s->L;
    xp.BH = (int)bh;
    xp.DV = (int)s->dv;
    xp.n_slices = 0;
    xp.flags = flags;
    xp.cu = cu;
    xp.H = (int)s->H;
    // per-channel decay: records hold every operand (inter-chunk kernel);
    // one decay per token: records hold T diag(beta) and the decay scalars
    auto launch_state = [&](const kda::InterParams& x) {
        // 16-column slices run kda_inter_quad_kernel, wider ones kda_inter_wide_kernel
        if (wv)
            return launch(wv == 16 ? K_INTER_QUAD : K_INTER_WIDE,
                          [&] { return kda::launch_inter_wide(x, (int)s->dk, wv, stream); });
        return s->alpha_mode == KDA_ALPHA_CHANNEL
                   ? launch(K_INTER, [&] {
                         return kda::launch_inter(x, (int)s->dk, qbf, s->alpha_mode, nv, stream);
                     })
                   : launch(K_INTER_SCALAR, [&] {
                         return kda::launch_inter_scalar(x, (int)s->dk, qbf, nv, stream);
                     });
    };
    hipError_t err = hipSuccess;
    if (plan.nchunks == 0) {
        // L == 0: the final state is the initial one
        xp.S_in = S0;
        xp.S_out = S_final;
        xp.c0 = 0;
        xp.ncs = 0;
        err = launch_state(xp);
    }
    for (int64_t sp = 0; sp < plan.nspans && err == hipSuccess; ++sp) {
        const int64_t c0 = sp * plan.span;
        const int64_t ncs = plan.nchunks - c0 < plan.span ? plan.nchunks - c0 : plan.span;
        ip.c0 = c0;
        ip.ncs = (int)ncs;
        err = launch(K_INTRA, [&] {
            return kda::launch_intra(ip, (int)s->dk, (int)s->dv, qbf, s->alpha_mode, stream);
        });
        if (err != hipSuccess) break;
        xp.S_in = sp == 0 ? S0 : s_mid;
        xp.S_out = sp == plan.nspans - 1 ? S_final : s_mid;
        xp.c0 = c0;
        xp.ncs = (int)ncs;
        err = launch_state(xp);
    }
    if (err != hipSuccess) {
        g_last_error = std::string(who) + ": " + hipGetErrorString(err);
        return KDA_ERR_HIP;
    }
    return KDA_OK;
}
int chunk_common(const char* who, const kda_shape* s, uint32_t flags, const int32_t* cu,
                 int64_t max_len, const void* q, const void* k, const void* v,
                 const void* log_alpha, const void* beta, const float* S0, void* o,
                 float* S_final, void* workspace, size_t workspace_bytes, void* hip_stream,
                 bool noalloc = false) {
    const CallScope sc(who, s, flags);
    return sc.done(chunk_body(who, s, flags, cu, max_len, q, k, v, log_alpha, beta, S0, o, S_final,
                              workspace, workspace_bytes, hip_stream, noalloc));
}
}  // namespace

extern "C" {

int kda_chunk_fwd_ex(const kda_shape* s, uint32_t flags, const void* q, const void* k,
                     const void* v, const void* log_alpha, const void* beta, const float* S0,
                     void* o, float* S_final, void* workspace, size_t workspace_bytes,
                     void* hip_stream) {
    return chunk_common("kda_chunk_fwd", s, flags, nullptr, -1, q, k, v, log_alpha, beta, S0, o,
                        S_final, workspace, workspace_bytes, hip_stream);
}

int kda_chunk_fwd_noalloc(const kda_shape* s, uint32_t flags, const void* q, const void* k,
                          const void* v, const void* log_alpha, const void* beta,
                          const float* S0, void* o, float* S_final, void* hip_stream) {
    return chunk_common("kda_chunk_fwd_noalloc", s, flags, nullptr, -1, q, k, v, log_alpha, beta,
                        S0, o, S_final, nullptr, 0, hip_stream, true);
}

size_t kda_chunk_fwd_varlen_workspace_bytes(const kda_shape* shape, int64_t max_seqlen) {
    if (check_shape(shape, false) != KDA_OK) return 0;
    if (max_seqlen < 0) return 0;
    kda_shape ps = *shape;
    ps.L = max_seqlen < shape->L ? max_seqlen : shape->L;
    return (size_t)make_plan(&ps).ws_bytes;
}

int kda_chunk_fwd_varlen(const kda_shape* s, uint32_t flags, const int32_t* cu_seqlens,
                         int64_t max_seqlen, const void* q, const void* k, const void* v,
                         const void* log_alpha, const void* beta, const float* S0, void* o,
                         float* S_final, void* workspace, size_t workspace_bytes,
                         void* hip_stream) {
    if (max_seqlen < 0) return KDA_ERR_SHAPE;
    return chunk_common("kda_chunk_fwd_varlen", s, flags, cu_seqlens, max_seqlen, q, k, v,
                        log_alpha, beta, S0, o, S_final, workspace, workspace_bytes, hip_stream);
}


size_t kda_linear_attn_fwd_workspace_bytes(const kda_shape* s) {
    if (check_shape(s, false) != KDA_OK || s->alpha_mode != KDA_ALPHA_NONE) return 0;
    return (size_t)(s->B * s->H * s->L * s->dk * elem_size(s->qkv_dtype));
}

static int kda_linear_attn_fwd_body(const kda_shape* s, const void* q, const void* k, const void* v,
                        const float* S0, const float* z0, void* o, float* S_final,
                        float* z_final, void* workspace, size_t workspace_bytes,
                        void* hip_stream) {
    int rc = check_shape(s, false);
    if (rc != KDA_OK) return rc;
    if (s->alpha_mode != KDA_ALPHA_NONE) return KDA_ERR_ALPHA_MODE;
    const int64_t bh = s->B * s->H;
    const int64_t tok = bh * s->L;
    const int eq = elem_size(s->qkv_dtype);
    if (tok > 0 && (!q || !k || !v || !o)) return KDA_ERR_NULL;
    const void* ptrs[] = {q, k, v, S0, z0, o, S_final, z_final, workspace};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return KDA_ERR_ALIGN;
    const int64_t one = tok * s->dk * eq;
    const int64_t wsb = (int64_t)kda_linear_attn_fwd_workspace_bytes(s);
    if (wsb > 0 && (!workspace || workspace_bytes < (size_t)wsb)) return KDA_ERR_WORKSPACE;
    const Span sq = span_of(q, one), sk = span_of(k, one),
               sv = span_of(v, tok * s->dv * eq), so = span_of(o, tok * s->dv * eq),
               s0 = span_of(S0, bh * s->dk * s->dv * 4), sf = span_of(S_final, bh * s->dk * s->dv * 4),
               z0s = span_of(z0, bh * s->dk * 4), zfs = span_of(z_final, bh * s->dk * 4),
               sw = span_of(workspace, wsb);
    // outputs overlap no input (S_final may be S0 and z_final may be z0 exactly)
    const Span ins[] = {sq, sk, sv};
    const Span outs[] = {so, sf, zfs};
    for (const Span& x : outs)
        for (const Span& y : ins)
            if (overlaps(x, y)) return KDA_ERR_ALIAS;
    if (overlaps(so, s0) || overlaps(so, z0s) || overlaps(so, sf) || overlaps(so, zfs) ||
        overlaps(sf, zfs) || overlaps(sf, z0s) || overlaps(zfs, s0))
        return KDA_ERR_ALIAS;
    if (overlaps(sf, s0) && (const void*)S_final != (const void*)S0) return KDA_ERR_ALIAS;
    if (overlaps(zfs, z0s) && (const void*)z_final != (const void*)z0) return KDA_ERR_ALIAS;
    const Span all[] = {sq, sk, sv, so, s0, sf, z0s, zfs};
    for (const Span& x : all)
        if (overlaps(sw, x)) return KDA_ERR_ALIAS;
    if (bh == 0) return KDA_OK;

    const int qbf = s->qkv_dtype == KDA_BF16;
    const int C = kda::chunk_len(qbf);
    const hipStream_t stream = (hipStream_t)hip_stream;
    void* fq = workspace;
    hipError_t err = hipSuccess;
    if (tok > 0) {
        kda::FeatureParams fp{q, fq, one / 16};
        err = timed_launch(K_FEATURE, stream, [&] { return kda::launch_feature_map(fp, qbf, stream); });
    }
    kda::InterParams xp;
    xp.q = fq;
    xp.k = k;
    xp.v = v;
    xp.ws = nullptr;
    xp.S_in = S0;
    xp.S_out = S_final;
    xp.o = o;
    xp.L = s->L;
    xp.c0 = 0;
    xp.ncs = (int)((s->L + C - 1) / C);
    xp.BH = (int)bh;
    xp.DV = (int)s->dv;
    xp.n_slices = 0;
    xp.linear_attn = 1;
    xp.z_in = z0;
    xp.z_out = z_final;
    const int nv = kda::chunk_slice_width((int)s->dk, (int)s->dv, qbf, bh);
    if (err == hipSuccess)
        err = timed_launch(K_INTER_SCALAR, stream, [&] {
            return kda::launch_inter_scalar(xp, (int)s->dk, qbf, nv, stream);
        });
    if (err != hipSuccess) {
        g_last_error = std::string("kda_linear_attn_fwd: ") + hipGetErrorString(err);
        return KDA_ERR_HIP;
    }
    return KDA_OK;
}

int kda_linear_attn_fwd(const kda_shape* s, const void* q, const void* k, const void* v,
                        const float* S0, const float* z0, void* o, float* S_final,
                        float* z_final, void* workspace, size_t workspace_bytes,
                        void* hip_stream) {
    const CallScope sc("kda_linear_attn_fwd", s, 0u);
    return sc.done(kda_linear_attn_fwd_body(s, q, k, v, S0, z0, o, S_final, z_final, workspace, workspace_bytes, hip_stream));
}

static int kda_linear_attn_decode_step_body(const kda_shape* s, const void* q, const void* k,
                                const void* v, float* S, float* z, void* o,
                                void* hip_stream) {
    int rc = check_shape(s, true);
    if (rc != KDA_OK) return rc;
    if (s->alpha_mode != KDA_ALPHA_NONE) return KDA_ERR_ALPHA_MODE;
    const int64_t bh = s->B * s->H;
    const int eq = elem_size(s->qkv_dtype);
    if (bh > 0 && (!q || !k || !v || !S || !z || !o)) return KDA_ERR_NULL;
    const void* ptrs[] = {q, k, v, S, z, o};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return KDA_ERR_ALIGN;
    const Span sq = span_of(q, bh * s->dk * eq), sk = span_of(k, bh * s->dk * eq),
               sv = span_of(v, bh * s->dv * eq), ss = span_of(S, bh * s->dk * s->dv * 4),
               sz = span_of(z, bh * s->dk * 4), so = span_of(o, bh * s->dv * eq);
    const Span ins[] = {sq, sk, sv};
    const Span outs[] = {ss, sz, so};
    for (const Span& x : outs)
        for (const Span& y : ins)
            if (overlaps(x, y)) return KDA_ERR_ALIAS;
    if (overlaps(ss, sz) || overlaps(ss, so) || overlaps(sz, so)) return KDA_ERR_ALIAS;
    if (bh == 0) return KDA_OK;
    kda::DecodeParams prm;
    prm.q = q;
    prm.k = k;
    prm.v = v;
    prm.log_alpha = nullptr;
    prm.beta = nullptr;
    prm.S = S;
    prm.o = o;
    prm.BH = (int)bh;
    prm.gate_bf16 = 0;
    prm.alpha_mode = KDA_ALPHA_NONE;
    prm.H = (int)s->H;
    prm.linear_attn = 1;
    prm.z = z;
    const hipStream_t stream = (hipStream_t)hip_stream;
    hipError_t err = timed_launch(K_DECODE, stream, [&] {
        return kda::launch_decode(prm, (int)s->dk, (int)s->dv, s->qkv_dtype == KDA_BF16, stream);
    });
    if (err != hipSuccess) {
        g_last_error = std::string("kda_linear_attn_decode_step: ") + hipGetErrorString(err);
        return KDA_ERR_HIP;
    }
    return KDA_OK;
}

int kda_linear_attn_decode_step(const kda_shape* s, const void* q, const void* k,
                                const void* v, float* S, float* z, void* o,
                                void* hip_stream) {
    const CallScope sc("kda_linear_attn_decode_step", s, 0u);
    return sc.done(kda_linear_attn_decode_step_body(s, q, k, v, S, z, o, hip_stream));
}

size_t kda_recurrence_bwd_workspace_bytes(const kda_shape* s) {
    if (check_shape(s, false) != KDA_OK) return 0;
    return (size_t)kda::bwd_workspace_bytes(s->B * s->H, s->L, (int)s->dk, (int)s->dv);
}

}  // extern "C"

namespace {
// Every host check of kda_recurrence_bwd (no HIP call); KDA_OK when a launch
// may follow.
// (ws: the workspace bytes the call needs; the shape has passed check_shape)
int bwd_checks(const kda_shape* s, const void* q, const void* k, const void* v,
               const void* log_alpha, const void* beta, const float* S0, const void* dout,
               const float* dS_final, float* dq, float* dk, float* dv, float* dlog_alpha,
               float* dbeta, float* dS0, void* workspace, size_t workspace_bytes, int64_t ws) {
    const int64_t bh = s->B * s->H, tok = bh * s->L;
    const int eq = elem_size(s->qkv_dtype), eg = elem_size(s->gate_dtype);
    const bool has_alpha = s->alpha_mode != KDA_ALPHA_NONE;
    const int64_t la_elems = s->alpha_mode == KDA_ALPHA_CHANNEL ? tok * s->dk : tok;
    if (bh > 0) {
        if (tok > 0) {
            if (!q || !k || !v || !beta || !dout || !dq || !dk || !dv || !dbeta)
                return KDA_ERR_NULL;
            if (has_alpha && (!log_alpha || !dlog_alpha)) return KDA_ERR_NULL;
        }
        if (ws > 0 && !workspace) return KDA_ERR_NULL;
    }
    if ((int64_t)workspace_bytes < ws) return KDA_ERR_WORKSPACE;
    const void* ptrs[] = {q, k, v, has_alpha ? log_alpha : nullptr, beta, S0, dout, dS_final,
                          dq, dk, dv, has_alpha ? dlog_alpha : nullptr, dbeta, dS0, workspace};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return KDA_ERR_ALIGN;

    const int64_t st = bh * s->dk * s->dv * 4;
    const Span in[] = {span_of(q, tok * s->dk * eq), span_of(k, tok * s->dk * eq),
                       span_of(v, tok * s->dv * eq),
                       span_of(has_alpha ? log_alpha : nullptr, la_elems * eg),
                       span_of(beta, tok * eg), span_of(S0, st),
                       span_of(dout, tok * s->dv * eq), span_of(dS_final, st)};
    const Span out[] = {span_of(dq, tok * s->dk * 4), span_of(dk, tok * s->dk * 4),
                        span_of(dv, tok * s->dv * 4),
                        span_of(has_alpha ? dlog_alpha : nullptr, la_elems * 4),
                        span_of(dbeta, tok * 4), span_of(dS0, st),
                        span_of(workspace, ws)};
    const int nout = sizeof(out) / sizeof(out[0]);
    for (int i = 0; i < nout; ++i) {
        for (const Span& x : in)
            if (overlaps(out[i], x)) return KDA_ERR_ALIAS;
        for (int j = i + 1; j < nout; ++j)
            if (overlaps(out[i], out[j])) return KDA_ERR_ALIAS;
    }
    return KDA_OK;
}
}  // namespace

extern "C" {

static int kda_recurrence_bwd_body(const kda_shape* s, const void* q, const void* k, const void* v,
                       const void* log_alpha, const void* beta, const float* S0,
                       const void* dout, const float* dS_final, float* dq, float* dk,
                       float* dv, float* dlog_alpha, float* dbeta, float* dS0, void* workspace,
                       size_t workspace_bytes, void* hip_stream) {
    int rc = check_shape(s, false);
    if (rc != KDA_OK) return rc;
    // one 64-lane workgroup per (head, 8 state columns): keep the grid in int
    if (s->B * s->H > (int64_t)(INT_MAX / 64 / (s->dv / 8))) return KDA_ERR_SHAPE;
    rc = bwd_checks(s, q, k, v, log_alpha, beta, S0, dout, dS_final, dq, dk, dv, dlog_alpha,
                    dbeta, dS0, workspace, workspace_bytes,
                    kda::bwd_workspace_bytes(s->B * s->H, s->L, (int)s->dk, (int)s->dv));
    if (rc != KDA_OK) return rc;
    const int64_t bh = s->B * s->H;
    const bool has_alpha = s->alpha_mode != KDA_ALPHA_NONE;
    if (bh == 0) return KDA_OK;

    kda::BwdParams prm;
    prm.q = q;
    prm.k = k;
    prm.v = v;
    prm.log_alpha = has_alpha ? log_alpha : nullptr;
    prm.beta = beta;
    prm.dout = dout;
    prm.S0 = S0;
    prm.dS_final = dS_final;
    prm.dq = dq;
    prm.dk = dk;
    prm.dv_out = dv;
    prm.dlog_alpha = has_alpha ? dlog_alpha : nullptr;
    prm.dbeta = dbeta;
    prm.dS0 = dS0;
    prm.ckpt = (float*)workspace;
    prm.BH = bh;
    prm.L = s->L;
    prm.dv = (int)s->dv;
    prm.gate_bf16 = s->gate_dtype == KDA_BF16;
    prm.alpha_mode = s->alpha_mode;
    const hipStream_t stream = (hipStream_t)hip_stream;
    hipError_t err = kda::zero_bwd_outputs(prm, (int)s->dk, stream);
    if (err == hipSuccess)
        err = timed_launch(K_BWD, stream, [&] {
            return kda::launch_bwd(prm, (int)s->dk, s->qkv_dtype == KDA_BF16, stream);
        });
    if (err != hipSuccess) {
        g_last_error = std::string("kda_recurrence_bwd: ") + hipGetErrorString(err);
        return KDA_ERR_HIP;
    }
    return KDA_OK;
}

int kda_recurrence_bwd(const kda_shape* s, const void* q, const void* k, const void* v,
                       const void* log_alpha, const void* beta, const float* S0,
                       const void* dout, const float* dS_final, float* dq, float* dk,
                       float* dv, float* dlog_alpha, float* dbeta, float* dS0, void* workspace,
                       size_t workspace_bytes, void* hip_stream) {
    const CallScope sc("kda_recurrence_bwd", s, 0u);
    return sc.done(kda_recurrence_bwd_body(s, q, k, v, log_alpha, beta, S0, dout, dS_final, dq, dk, dv, dlog_alpha, dbeta, dS0, workspace, workspace_bytes, hip_stream));
}

namespace {
// Layout of kda_recurrence_bwd_ex's workspace: the gradient kernel's own
// area, then the fp32 preprocessed inputs and the row norms, each piece
// rounded up to 256 bytes.
struct BwdExPlan {
    int64_t ckpt = 0, qn = 0, kn = 0, v32 = 0, do32 = 0, la32 = 0, b32 = 0, nq = 0, nk = 0;
    int64_t total = 0;
};
BwdExPlan bwd_ex_plan(const kda_shape* s) {
    auto up = [](int64_t x) { return (x + 255) / 256 * 256; };
    const int64_t rows = s->B * s->H * s->L;
    BwdExPlan p;
    int64_t off = up(kda::bwd_workspace_bytes(s->B * s->H, s->L, (int)s->dk, (int)s->dv));
    p.ckpt = 0;
    p.qn = off; off += up(rows * s->dk * 4);
    p.kn = off; off += up(rows * s->dk * 4);
    p.v32 = off; off += up(rows * s->dv * 4);
    p.do32 = off; off += up(rows * s->dv * 4);
    p.la32 = off; off += up(s->alpha_mode == KDA_ALPHA_CHANNEL ? rows * s->dk * 4 : rows * 4);
    p.b32 = off; off += up(rows * 4);
    p.nq = off; off += up(rows * 4);
    p.nk = off; off += up(rows * 4);
    p.total = off;
    return p;
}
}  // namespace

size_t kda_recurrence_bwd_ex_workspace_bytes(const kda_shape* s, uint32_t flags) {
    if (check_shape(s, false) != KDA_OK || (flags & ~kAllFlags)) return 0;
    if (s->B * s->H * s->L == 0) return 0;
    return (size_t)bwd_ex_plan(s).total;
}

static int kda_recurrence_bwd_ex_body(const kda_shape* s, uint32_t flags, const void* q, const void* k,
                          const void* v, const void* log_alpha, const void* beta,
                          const float* S0, const void* dout, const float* dS_final, float* dq,
                          float* dk, float* dv, float* dlog_alpha, float* dbeta, float* dS0,
                          void* workspace, size_t workspace_bytes, void* hip_stream) {
    int rc = check_shape(s, false);
    if (rc != KDA_OK) return rc;
    if (flags & ~kAllFlags) return KDA_ERR_FLAGS;
    const int64_t bh = s->B * s->H, rows = bh * s->L;
    if (rows == 0)  // nothing to preprocess: the plain call (dS0 = dS_final)
        return kda_recurrence_bwd(s, q, k, v, log_alpha, beta, S0, dout, dS_final, dq, dk, dv,
                                  dlog_alpha, dbeta, dS0, workspace, workspace_bytes, hip_stream);
    const bool has_alpha = s->alpha_mode != KDA_ALPHA_NONE;
    if (!q || !k || !v || !beta || !dout || !dq || !dk || !dv || !dbeta) return KDA_ERR_NULL;
    if (has_alpha && (!log_alpha || !dlog_alpha)) return KDA_ERR_NULL;
    if (!workspace) return KDA_ERR_NULL;
    const BwdExPlan pl = bwd_ex_plan(s);
    if ((int64_t)workspace_bytes < pl.total) return KDA_ERR_WORKSPACE;
    const void* ptrs[] = {q, k, v, has_alpha ? log_alpha : nullptr, beta, S0, dout, dS_final,
                          dq, dk, dv, has_alpha ? dlog_alpha : nullptr, dbeta, dS0, workspace};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return KDA_ERR_ALIGN;
    // the raw inputs against the outputs and the workspace (the plain call
    // below checks the outputs against each other and the fp32 copies)
    const int eq = elem_size(s->qkv_dtype), eg = elem_size(s->gate_dtype);
    const int64_t la_elems = s->alpha_mode == KDA_ALPHA_CHANNEL ? rows * s->dk : rows;
    const int64_t st = bh * s->dk * s->dv * 4;
    const Span in[] = {span_of(q, rows * s->dk * eq), span_of(k, rows * s->dk * eq),
                       span_of(v, rows * s->dv * eq),
                       span_of(has_alpha ? log_alpha : nullptr, la_elems * eg),
                       span_of(beta, rows * eg), span_of(S0, st),
                       span_of(dout, rows * s->dv * eq), span_of(dS_final, st)};
    const Span out[] = {span_of(dq, rows * s->dk * 4), span_of(dk, rows * s->dk * 4),
                        span_of(dv, rows * s->dv * 4),
                        span_of(has_alpha ? dlog_alpha : nullptr, la_elems * 4),
                        span_of(dbeta, rows * 4), span_of(dS0, st),
                        span_of(workspace, pl.total)};
    const int nout = sizeof(out) / sizeof(out[0]);
    for (int i = 0; i < nout; ++i) {
        for (const Span& x : in)
            if (overlaps(out[i], x)) return KDA_ERR_ALIAS;
        // the outputs against each other and against the whole workspace
        // (which holds the fp32 copies and the row norms the chain rule reads)
        for (int j = i + 1; j < nout; ++j)
            if (overlaps(out[i], out[j])) return KDA_ERR_ALIAS;
    }
    // the prep and post kernels run one 64-lane workgroup per token row
    if (rows > (int64_t)(UINT32_MAX / 64)) return KDA_ERR_SHAPE;

    char* ws = (char*)workspace;
    kda::BwdPrep pp;
    pp.q = q;
    pp.k = k;
    pp.v = v;
    pp.dout = dout;
    pp.log_alpha = has_alpha ? log_alpha : nullptr;
    pp.beta = beta;
    pp.qn = (float*)(ws + pl.qn);
    pp.kn = (float*)(ws + pl.kn);
    pp.v32 = (float*)(ws + pl.v32);
    pp.do32 = (float*)(ws + pl.do32);
    pp.la32 = (float*)(ws + pl.la32);
    pp.b32 = (float*)(ws + pl.b32);
    pp.nq = (float*)(ws + pl.nq);
    pp.nk = (float*)(ws + pl.nk);
    pp.dq = dq;
    pp.dk = dk;
    pp.dlog_alpha = has_alpha ? dlog_alpha : nullptr;
    pp.dbeta = dbeta;
    pp.rows = rows;
    pp.DK = (int)s->dk;
    pp.DV = (int)s->dv;
    pp.alpha_mode = s->alpha_mode;
    pp.flags = flags;
    kda_shape s32 = *s;
    s32.qkv_dtype = KDA_F32;
    s32.gate_dtype = KDA_F32;
    // the inner call's own checks, before anything is enqueued
    if (bh > (int64_t)(INT_MAX / 64 / (s->dv / 8))) return KDA_ERR_SHAPE;
    rc = bwd_checks(&s32, pp.qn, pp.kn, pp.v32, has_alpha ? pp.la32 : nullptr, pp.b32, S0,
                    pp.do32, dS_final, dq, dk, dv, dlog_alpha, dbeta, dS0, ws + pl.ckpt,
                    (size_t)pl.qn, kda::bwd_workspace_bytes(bh, s->L, (int)s->dk, (int)s->dv));
    if (rc != KDA_OK) return rc;
    const hipStream_t stream = (hipStream_t)hip_stream;
    hipError_t err = kda::launch_bwd_prep(pp, s->qkv_dtype == KDA_BF16,
                                          s->gate_dtype == KDA_BF16, stream);
    if (err != hipSuccess) {
        g_last_error = std::string("kda_recurrence_bwd_ex: ") + hipGetErrorString(err);
        return KDA_ERR_HIP;
    }
    rc = kda_recurrence_bwd(&s32, pp.qn, pp.kn, pp.v32, has_alpha ? pp.la32 : nullptr, pp.b32,
                            S0, pp.do32, dS_final, dq, dk, dv, dlog_alpha, dbeta, dS0,
                            ws + pl.ckpt, (size_t)pl.qn, hip_stream);
    if (rc != KDA_OK) return rc;
    err = kda::launch_bwd_post(pp, stream);
    if (err != hipSuccess) {
        g_last_error = std::string("kda_recurrence_bwd_ex: ") + hipGetErrorString(err);
        return KDA_ERR_HIP;
    }
    return KDA_OK;
}

int kda_recurrence_bwd_ex(const kda_shape* s, uint32_t flags, const void* q, const void* k,
                          const void* v, const void* log_alpha, const void* beta,
                          const float* S0, const void* dout, const float* dS_final, float* dq,
                          float* dk, float* dv, float* dlog_alpha, float* dbeta, float* dS0,
                          void* workspace, size_t workspace_bytes, void* hip_stream) {
    const CallScope sc("kda_recurrence_bwd_ex", s, flags);
    return sc.done(kda_recurrence_bwd_ex_body(s, flags, q, k, v, log_alpha, beta, S0, dout, dS_final, dq, dk, dv, dlog_alpha, dbeta, dS0, workspace, workspace_bytes, hip_stream));
}

}  // extern "C"

namespace {
// Layout of kda_chunk_bwd's workspace (each piece rounded up to 256 bytes):
// the forward records of every chunk, the reverse records (one per chunk),
// T^T, the forward scan's S and u and the reverse scan's G and du per chunk,
// and, without a decay, zero per-channel fp32 ln(alpha) and an fp32 beta.
struct ChunkBwdPlan {
    int64_t recs = 0, rrecs = 0, tt = 0, S = 0, G = 0, u = 0, du = 0, la = 0, b = 0, total = 0;
    int64_t nc = 0;
    bool ok = false;
};
ChunkBwdPlan chunk_bwd_plan(const kda_shape* s) {
    ChunkBwdPlan p;
    const int64_t bh = s->B * s->H, C = 64;
    p.nc = (s->L + C - 1) / C;
    const int64_t rb = kda::rec_layout((int)s->dk, (int)s->dv, (int)C, 2, true).bytes;
    // sizes in doubles first: a shape whose workspace passes 2^60 bytes is refused
    const double chunks = (double)bh * (double)p.nc;
    const int64_t rrb = kda::rev_rec_bytes((int)s->dk, (int)s->dv);
    const double est = chunks * (rb + rrb + C * C * 4.0 + 2.0 * s->dk * s->dv * 4 + 2.0 * C * s->dv * 2) +
                       (double)bh * s->L * (s->dk + 1) * 4.0;
    if (est > 1.0e18 || chunks > (double)INT_MAX) return p;
    auto up = [](int64_t x) { return (x + 255) / 256 * 256; };
    const int64_t nch = bh * p.nc;
    int64_t off = 0;
    p.recs = off; off += up(nch * rb);
    p.rrecs = off; off += up(nch * rrb);
    p.tt = off; off += up(nch * C * C * 4);
    p.S = off; off += up(nch * s->dk * s->dv * 4);
    p.G = off; off += up(nch * s->dk * s->dv * 4);
    p.u = off; off += up(nch * C * s->dv * 2);
    p.du = off; off += up(nch * C * s->dv * 2);
    if (s->alpha_mode == KDA_ALPHA_NONE) {
        p.la = off; off += up(bh * s->L * s->dk * 4);
        p.b = off; off += up(bh * s->L * 4);
    }
    p.total = nch > 0 ? off : 0;
    p.ok = true;
    return p;
}
// kda_chunk_bwd's shape check: kda_chunk_fwd's, bf16 q/k/v/do, and a plan
int chunk_bwd_shape(const kda_shape* s, ChunkBwdPlan* plan) {
    int rc = check_shape(s, false);
    if (rc != KDA_OK) return rc;
    if (s->qkv_dtype != KDA_BF16) return KDA_ERR_DTYPE;
    *plan = chunk_bwd_plan(s);
    return plan->ok ? KDA_OK : KDA_ERR_SHAPE;
}
}  // namespace

extern "C" {

size_t kda_chunk_bwd_workspace_bytes(const kda_shape* s) {
    ChunkBwdPlan p;
    if (chunk_bwd_shape(s, &p) != KDA_OK) return 0;
    return (size_t)p.total;
}

static int kda_chunk_bwd_body(const kda_shape* s, const void* q, const void* k, const void* v,
                              const void* log_alpha, const void* beta, const float* S0,
                              const void* dout, const float* dS_final, float* dq, float* dk,
                              float* dv, float* dlog_alpha, float* dbeta, float* dS0,
                              void* workspace, size_t workspace_bytes, void* hip_stream) {
    ChunkBwdPlan pl;
    int rc = chunk_bwd_shape(s, &pl);
    if (rc != KDA_OK) return rc;
    rc = bwd_checks(s, q, k, v, log_alpha, beta, S0, dout, dS_final, dq, dk, dv, dlog_alpha,
                    dbeta, dS0, workspace, workspace_bytes, pl.total);
    if (rc != KDA_OK) return rc;
    const int64_t bh = s->B * s->H;
    if (bh == 0) return KDA_OK;
    const hipStream_t stream = (hipStream_t)hip_stream;
    const int dkk = (int)s->dk, dvv = (int)s->dv;
    const int nc = (int)pl.nc;
    char* ws = (char*)workspace;
    auto fail = [&](hipError_t e) {
        g_last_error = std::string("kda_chunk_bwd: ") + hipGetErrorString(e);
        return KDA_ERR_HIP;
    };
    hipError_t err = hipSuccess;
    if (nc == 0) {
        // L = 0: dJ/dS0 is dJ/dS_final
        if (dS0) {
            const size_t st = (size_t)bh * dkk * dvv * 4;
            err = dS_final ? hipMemcpyAsync(dS0, dS_final, st, hipMemcpyDeviceToDevice, stream)
                           : hipMemsetAsync(dS0, 0, st, stream);
        }
        return err == hipSuccess ? KDA_OK : fail(err);
    }
    if (log_on())
        klog("kda_chunk_bwd: %d chunks of 64; workspace %lld B", nc, (long long)pl.total);
    // per-channel gates: read as given per channel, read per token by every
    // channel for a head gate, widened (zeros) without a decay
    const void* la = log_alpha;
    const void* bt = beta;
    int gate_bf16 = s->gate_dtype == KDA_BF16;
    if (s->alpha_mode == KDA_ALPHA_NONE) {
        kda::GateWiden gw{};
        gw.log_alpha = nullptr;
        gw.beta = beta;
        gw.la = (float*)(ws + pl.la);
        gw.b = (float*)(ws + pl.b);
        gw.rows = bh * s->L;
        gw.DK = dkk;
        gw.gate_bf16 = gate_bf16;
        err = timed_launch(K_GATE_WIDEN, stream, [&] { return kda::launch_gate_widen(gw, stream); });
        if (err != hipSuccess) return fail(err);
        la = gw.la;
        bt = gw.b;
        gate_bf16 = 0;
    }
    // forward records of every chunk, with T^T
    kda::IntraParams ip{};
    ip.q = q;
    ip.k = k;
    ip.v = v;
    ip.log_alpha = la;
    ip.beta = bt;
    ip.ws = ws + pl.recs;
    ip.L = s->L;
    ip.c0 = 0;
    ip.ncs = nc;
    ip.BH = (int)bh;
    ip.gate_bf16 = gate_bf16;
    ip.wide = 1;
    ip.tt = (float*)(ws + pl.tt);
    ip.la_head = s->alpha_mode == KDA_ALPHA_HEAD;
    // and, from each record just written, the chunk's reverse record
    ip.rrecs = ws + pl.rrecs;
    ip.dout = dout;
    err = timed_launch(K_INTRA, stream, [&] {
        return kda::launch_intra(ip, dkk, dvv, 1, KDA_ALPHA_CHANNEL, stream);
    });
    if (err != hipSuccess) return fail(err);
    // forward scan: the state entering every chunk, and its u
    const int nv = 32;
    kda::InterParams xp{};
    xp.ws = ws + pl.recs;
    xp.S_in = S0;
    xp.S_out = nullptr;
    xp.o = nullptr;
    xp.L = s->L;
    xp.c0 = 0;
    xp.ncs = nc;
    xp.BH = (int)bh;
    xp.DV = dvv;
    xp.S_all = (float*)(ws + pl.S);
    xp.u_all = ws + pl.u;
    xp.scan_shift = 0;
    xp.n_store = nc;
    err = timed_launch(K_WIDE_SCAN, stream, [&] { return kda::launch_inter_wide_scan(xp, dkk, nv, stream); });
    if (err != hipSuccess) return fail(err);
    // the reverse scan over the reverse records: dJ/dS leaving every chunk
    // and dJ/du, and dJ/dS0 at its end
    kda::InterParams rx = xp;
    rx.ws = ws + pl.rrecs;
    rx.S_in = dS_final;
    rx.S_out = dS0;
    rx.L = (int64_t)nc * 64;
    rx.ncs = nc;
    rx.S_all = (float*)(ws + pl.G);
    rx.u_all = ws + pl.du;
    rx.scan_shift = 0;
    rx.n_store = nc;
    rx.rev = 1;
    err = timed_launch(K_WIDE_SCAN, stream, [&] { return kda::launch_inter_wide_scan(rx, dkk, nv, stream); });
    if (err != hipSuccess) return fail(err);
    // every chunk's gradients
    kda::ChunkGradParams gp{};
    gp.q = q;
    gp.k = k;
    gp.v = v;
    gp.dout = dout;
    gp.la = la;
    gp.beta = bt;
    gp.tt = (const float*)(ws + pl.tt);
    gp.S_all = (const float*)(ws + pl.S);
    gp.u_all = ws + pl.u;
    gp.G_all = (const float*)(ws + pl.G);
    gp.du_all = ws + pl.du;
    gp.dq = dq;
    gp.dk = dk;
    gp.dv_out = dv;
    gp.dbeta = dbeta;
    gp.dla = s->alpha_mode == KDA_ALPHA_NONE ? nullptr : dlog_alpha;
    gp.L = s->L;
    gp.nc = nc;
    gp.BH = (int)bh;
    gp.gate_bf16 = gate_bf16;
    gp.dla_mode = s->alpha_mode == KDA_ALPHA_CHANNEL ? 2 : (s->alpha_mode == KDA_ALPHA_HEAD ? 1 : 0);
    gp.la_rs = s->alpha_mode == KDA_ALPHA_HEAD ? 1 : dkk;
    err = timed_launch(K_CHUNK_GRAD, stream, [&] { return kda::launch_chunk_grad(gp, dkk, dvv, stream); });
    if (err != hipSuccess) return fail(err);
    return KDA_OK;
}

int kda_chunk_bwd(const kda_shape* s, const void* q, const void* k, const void* v,
                  const void* log_alpha, const void* beta, const float* S0, const void* dout,
                  const float* dS_final, float* dq, float* dk, float* dv, float* dlog_alpha,
                  float* dbeta, float* dS0, void* workspace, size_t workspace_bytes,
                  void* hip_stream) {
    const CallScope sc("kda_chunk_bwd", s, 0u);
    return sc.done(kda_chunk_bwd_body(s, q, k, v, log_alpha, beta, S0, dout, dS_final, dq, dk, dv,
                                      dlog_alpha, dbeta, dS0, workspace, workspace_bytes,
                                      hip_stream));
}

int kda_decode_step(const kda_shape* s, const void* q, const void* k, const void* v,
                    const void* log_alpha, const void* beta, float* S, void* o,
                    void* hip_stream) {
    return decode_common("kda_decode_step", s, 0u, q, k, v, log_alpha, beta, S, 0, nullptr, o,
                         hip_stream);
}

int kda_decode_step_ex(const kda_shape* s, uint32_t flags, const void* q, const void* k,
                       const void* v, const void* log_alpha, const void* beta, float* S, void* o,
                       void* hip_stream) {
    return decode_common("kda_decode_step_ex", s, flags, q, k, v, log_alpha, beta, S, 0,
                         nullptr, o, hip_stream);
}

int kda_decode_step_slots(const kda_shape* s, const void* q, const void* k, const void* v,
                          const void* log_alpha, const void* beta, float* S_pool,
                          int64_t n_slots, const int32_t* slots, void* o, void* hip_stream) {
    return kda_decode_step_slots_ex(s, 0u, q, k, v, log_alpha, beta, S_pool, n_slots, slots, o,
                                    hip_stream);
}

int kda_decode_step_slots_ex(const kda_shape* s, uint32_t flags, const void* q,
                             const void* k, const void* v, const void* log_alpha,
                             const void* beta, float* S_pool, int64_t n_slots,
                             const int32_t* slots, void* o, void* hip_stream) {
    if (s && !slots && s->B * s->H > 0) return KDA_ERR_NULL;
    return decode_common("kda_decode_step_slots", s, flags, q, k, v, log_alpha, beta, S_pool,
                         n_slots, slots, o, hip_stream);
}

int kda_timing_enable(int on) {
    std::lock_guard<std::mutex> lock(g_timing_mu);
    g_timing_on = on != 0;
    return KDA_OK;
}

int kda_timing_reset(void) {
    std::vector<TimedLaunch> old;
    {
        std::lock_guard<std::mutex> lock(g_timing_mu);
        old.swap(g_timed);
    }
    hipError_t err = hipSuccess;
    for (const TimedLaunch& t : old) {
        hipError_t e1 = hipEventDestroy(t.start), e2 = hipEventDestroy(t.stop);
        if (err == hipSuccess) err = e1 != hipSuccess ? e1 : e2;
    }
    if (err != hipSuccess) {
        g_last_error = std::string("kda_timing_reset: ") + hipGetErrorString(err);
        return KDA_ERR_HIP;
    }
    return KDA_OK;
}

int kda_timing_read(const char* kernel, int64_t* launches, double* total_ms) {
    if (!kernel || !launches || !total_ms) return KDA_ERR_NULL;
    int id = -1;
    for (int i = 0; i < K_COUNT; ++i)
        if (strcmp(kernel, kKernelNames[i]) == 0) id = i;
    if (id < 0) return KDA_ERR_SHAPE;
    std::lock_guard<std::mutex> lock(g_timing_mu);
    int64_t n = 0;
    double sum = 0.0;
    for (const TimedLaunch& t : g_timed) {
        if (t.kernel != id) continue;
        float ms = 0.f;
        hipError_t err = hipEventSynchronize(t.stop);
        if (err == hipSuccess) err = hipEventElapsedTime(&ms, t.start, t.stop);
        if (err != hipSuccess) {
            g_last_error = std::string("kda_timing_read: ") + hipGetErrorString(err);
            return KDA_ERR_HIP;
        }
        ++n;
        sum += ms;
    }
    *launches = n;
    *total_ms = sum;
    return KDA_OK;
}

}  // extern "C"
