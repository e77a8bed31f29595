// kda_bwd.hip -- gradients of the KDA / gated delta rule recurrence on gfx950.
//
// The forward step is the one of the prefill and decode kernels ("22,580:
// From GPT-2 to Kimi K3" (yichencityu.github.io) section 5.2 with section 08's
// decay; "22580: From GPT-2 to Kimi K3, Explained" (lukebest.github.io), "Key
// code and formulas"):
//     S~_t = diag(alpha_t) S_{t-1};  e_t = v_t - k_t S~_t;  u_t = beta_t e_t
//     S_t  = S~_t + k_t^T u_t;        o_t = q_t S_t
// The pages give no backward pass; its gradients follow from the step by the
// chain rule, walking the tokens from last to first with G = dJ/dS_t (G starts
// at dS_final):
//     G     += q_t^T do_t                 dq_t   = S_t do_t^T
//     gu     = k_t G                      dbeta_t = gu . e_t
//     ge     = beta_t gu                  dv_t   = ge
//     dk_t   = G u_t^T - S~_t ge^T        gS~    = G - k_t^T ge
//     dln(alpha_t)_i = sum_j gS~_ij S~_ij (summed over i too for one decay per
//     head)                                G      = diag(alpha_t) gS~
// and dS0 = G after the first token.
//
// Columns of the state evolve independently in both directions, so the grid
// is one single-wave workgroup per (head, slice of W = 8 state columns).  Lane
// l holds rows l and l + 64 (d_k = 128) of its slice in registers; sums over
// the slice's columns (dq, dk, d ln alpha) are per lane and reach the outputs
// through float atomics (one add per slice, so the order of the adds, and the
// last bits of those outputs, vary from run to run); sums over rows (k S~,
// k G) are wave reductions whose totals are wave-uniform.
//
// Pass 1 runs the forward recurrence and stores the slice's state before
// every CK = 8th token (the workspace holds ceil(L / 8) states per head).
// Pass 2 walks the checkpoints backwards: it recomputes the decayed states
// S~_t of an interval from its checkpoint into LDS (with e_t), then runs the
// reverse step above over them.  Row and column reductions go through the
// gfx950 lane-swap instructions (v_permlane32_swap / v_permlane16_swap) and
// DPP, not through LDS.  Each pass loads the next interval's inputs before working
// on the current one.
//
// The step is a chain of dependent wave reductions (three per token over the
// two passes), so the kernel is bound by their latency, not by memory.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int W = 8;    // state columns per workgroup
constexpr int CK = 8;   // tokens per checkpoint interval

template <int C>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), C, 0xf, 0xf, false));
}

// x + y after swapping the upper 32 lanes of x with the lower 32 lanes of y:
// lanes 0-31 get x_l + x_{l+32}, lanes 32-63 get y_{l-32} + y_l.
__device__ __forceinline__ float swap32_add(float x, float y) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y),
                                                    false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The same over rows of 16 lanes: odd rows of x swapped with even rows of y,
// so lanes with bit 4 clear get x_l + x_{l+16}, the others y_{l-16} + y_l.
__device__ __forceinline__ float swap16_add(float x, float y) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y),
                                                    false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Totals over the 64 lanes of the W per-lane partials x[0..W-1]:
// reduce-scatter over lane bits 5, 4 (and 3 for W = 8), so that lane l keeps
// one column, sums inside each group of 64 / W lanes, then the total of
// column c is read from lane (64 / W) c into a wave-uniform value.
__device__ __forceinline__ void column_totals(const float (&x)[W], float (&tot)[W]) {
    static_assert(W == 4 || W == 8, "column_totals: W is 4 or 8");
    float y[W / 2], z[W / 4];
#pragma unroll
    for (int c = 0; c < W / 2; ++c) y[c] = swap32_add(x[c], x[c + W / 2]);
#pragma unroll
    for (int c = 0; c < W / 4; ++c) z[c] = swap16_add(y[c], y[c + W / 4]);
    // row_mirror pairs lane i of a row of 16 with lane 15 - i (opposite bit 3,
    // same bits 5 and 4): for W = 8 it completes the scatter over bit 3
    float w;
    if constexpr (W == 8) {
        const bool b3 = lane_id() & 8;
        w = (b3 ? z[1] : z[0]) + dpp<0x140>(b3 ? z[0] : z[1]);
    } else {
        w = z[0] + dpp<0x140>(z[0]);
    }
    w += dpp<0x141>(w);   // row_half_mirror: i <-> 7 - i inside eight lanes
    w += dpp<0xB1>(w);    // quad_perm [1,0,3,2]
    w += dpp<0x4E>(w);    // quad_perm [2,3,0,1]
#pragma unroll
    for (int c = 0; c < W; ++c) tot[c] = read_lane(w, (64 / W) * c);
}

// W consecutive floats <-> registers, in 16-byte pieces
__device__ __forceinline__ void ld_row(const float* r, float (&x)[W]) {
#pragma unroll
    for (int h = 0; h < W / 4; ++h) {
        const floatx4 v = *(const floatx4*)(r + 4 * h);
#pragma unroll
        for (int i = 0; i < 4; ++i) x[4 * h + i] = v[i];
    }
}
__device__ __forceinline__ void st_row(float* r, const float (&x)[W]) {
#pragma unroll
    for (int h = 0; h < W / 4; ++h)
        *(floatx4*)(r + 4 * h) = floatx4{x[4 * h], x[4 * h + 1], x[4 * h + 2], x[4 * h + 3]};
}

template <typename T>
__device__ __forceinline__ float f32(T x) { return (float)x; }

// Inputs of one interval of CK tokens t0 .. t0 + CK - 1 (positions past the
// end are clamped to the last token and never used).  Per-row values are kept
// in their stored type until used, so the loads stay in flight across the
// previous interval's work.  Column values are spread over the lanes: lane l
// holds token t0 + l / W, column l % W; per-token scalars sit in lanes < CK.
template <int RPL, typename E>
struct Interval {
    E k[RPL][CK], q[RPL][CK];
    uint32_t a[RPL][CK];   // channel gate as loaded: bf16 bits (zero-extended) or fp32
    E vcol, docol;
    uint32_t bcol, hcol;   // beta, head gate, as loaded
    float ck[RPL][W];      // reverse pass: the interval's checkpoint rows
};

template <bool B>
struct Flag {
    static constexpr bool value = B;
};

// REV: the reverse pass's loads (q, dJ/do and the checkpoint at ckp as well)
template <int DK, typename E, int MODE, bool REV>
__device__ __forceinline__ void load_interval(const BwdParams& p, int64_t bh, int slice,
                                              int64_t t0, const float* ckp,
                                              Interval<DK / 64, E>& in) {
    constexpr int RPL = DK / 64;
    const int l = lane_id();
    const int64_t last = p.L - 1;
    const bool gbf = p.gate_bf16 != 0;
#pragma unroll
    for (int tau = 0; tau < CK; ++tau) {
        const int64_t t = t0 + tau < last ? t0 + tau : last;
#pragma unroll
        for (int m = 0; m < RPL; ++m) {
            const int64_t off = (bh * p.L + t) * DK + l + 64 * m;
            in.k[m][tau] = ((const E*)p.k)[off];
            if constexpr (REV) in.q[m][tau] = ((const E*)p.q)[off];
            if constexpr (MODE == KDA_ALPHA_CHANNEL)
                in.a[m][tau] = gbf ? (uint32_t)((const uint16_t*)p.log_alpha)[off]
                                   : ((const uint32_t*)p.log_alpha)[off];
        }
    }
    {
        const int64_t tl = t0 + l / W < last ? t0 + l / W : last;
        const int64_t off = (bh * p.L + tl) * p.dv + slice * W + l % W;
        in.vcol = ((const E*)p.v)[off];
        if constexpr (REV) in.docol = ((const E*)p.dout)[off];
    }
    if constexpr (REV) {
#pragma unroll
        for (int m = 0; m < RPL; ++m) {
            ld_row(ckp + (l + 64 * m) * W, in.ck[m]);
        }
    }
    {
        const int64_t tl = t0 + (l & (CK - 1)) < last ? t0 + (l & (CK - 1)) : last;
        const int64_t off = bh * p.L + tl;
        in.bcol = gbf ? (uint32_t)((const uint16_t*)p.beta)[off]
                      : ((const uint32_t*)p.beta)[off];
        if constexpr (MODE == KDA_ALPHA_HEAD)
            in.hcol = gbf ? (uint32_t)((const uint16_t*)p.log_alpha)[off]
                          : ((const uint32_t*)p.log_alpha)[off];
    }
}

// A gate value as loaded (bf16 bits zero-extended, or fp32 bits) -> float.  The
// widening happens here, at the use, so that it does not wait for the load in
// the interval that issues it.
__device__ __forceinline__ float gate(uint32_t b, bool gbf) {
    return __uint_as_float(gbf ? b << 16 : b);
}

template <int DK, typename E, int MODE>
__global__ void __launch_bounds__(64) kda_bwd_kernel(BwdParams p) {
    constexpr int RPL = DK / 64;
    __shared__ __attribute__((aligned(16))) float sSt[CK][RPL][64][W];  // S~ of each token
    __shared__ __attribute__((aligned(16))) float sE[CK][W];
    __shared__ __attribute__((aligned(16))) float sDV[CK * W];   // dv of an interval
    __shared__ float sDB[CK], sDH[CK];                           // dbeta, head d ln alpha

    const int l = lane_id();
    const int ns = p.dv / W;
    const int64_t bh = blockIdx.x / ns;
    const int slice = blockIdx.x - (int)(bh * ns);
    const int j0 = slice * W;
    const int64_t L = p.L;
    const int64_t nck = (L + CK - 1) / CK;
    const bool gbf = p.gate_bf16 != 0;
    float* ck = p.ckpt + (int64_t)blockIdx.x * nck * DK * W;

    // decay of row m at token tau of an interval
    auto decay = [&](const Interval<RPL, E>& in, int m, int tau) -> float {
        if constexpr (MODE == KDA_ALPHA_CHANNEL) return __expf(gate(in.a[m][tau], gbf));
        else if constexpr (MODE == KDA_ALPHA_HEAD) return __expf(read_lane(gate(in.hcol, gbf), tau));
        else return 1.f;
    };

    // ---- pass 1: forward recurrence, checkpoint before every CK-th token --------
    float S[RPL][W];
#pragma unroll
    for (int m = 0; m < RPL; ++m) {
        if (p.S0) {
            ld_row(p.S0 + (bh * DK + l + 64 * m) * p.dv + j0, S[m]);
        } else {
#pragma unroll
            for (int j = 0; j < W; ++j) S[m][j] = 0.f;
        }
    }
    Interval<RPL, E> nxt;
    if (nck > 0) load_interval<DK, E, MODE, false>(p, bh, slice, 0, nullptr, nxt);
    for (int64_t c = 0; c < nck; ++c) {
        const Interval<RPL, E> cur = nxt;
        if (c + 1 < nck)
            load_interval<DK, E, MODE, false>(p, bh, slice, (c + 1) * CK, nullptr, nxt);
#pragma unroll
        for (int m = 0; m < RPL; ++m) {
            st_row(ck + (c * DK + l + 64 * m) * W, S[m]);
        }
        const int n = L - c * CK < CK ? (int)(L - c * CK) : CK;
        // full intervals run without per-token guards (the tail one with them),
        // so the compiler sees every token's loads and waits consumed in order
        auto forward = [&](auto full) {
#pragma unroll
        for (int tau = 0; tau < CK; ++tau) {
            if (decltype(full)::value || tau < n) {
                float part[W] = {};
#pragma unroll
                for (int m = 0; m < RPL; ++m) {
                    const float a = decay(cur, m, tau), km = f32(cur.k[m][tau]);
#pragma unroll
                    for (int j = 0; j < W; ++j) {
                        S[m][j] *= a;
                        part[j] += km * S[m][j];
                    }
                }
                float tot[W];
                column_totals(part, tot);
                const float beta = read_lane(gate(cur.bcol, gbf), tau);
                const float vv = f32(cur.vcol);
#pragma unroll
                for (int j = 0; j < W; ++j) {
                    const float u = beta * (read_lane(vv, tau * W + j) - tot[j]);
#pragma unroll
                    for (int m = 0; m < RPL; ++m) S[m][j] += f32(cur.k[m][tau]) * u;
                }
            }
        }
        };
        if (n == CK)
            forward(Flag<true>{});
        else
            forward(Flag<false>{});
    }

    // ---- pass 2: reverse sweep over the intervals ----------------------------------
    float G[RPL][W];
#pragma unroll
    for (int m = 0; m < RPL; ++m) {
        if (p.dS_final) {
            ld_row(p.dS_final + (bh * DK + l + 64 * m) * p.dv + j0, G[m]);
        } else {
#pragma unroll
            for (int j = 0; j < W; ++j) G[m][j] = 0.f;
        }
    }
    if (nck > 0)
        load_interval<DK, E, MODE, true>(p, bh, slice, (nck - 1) * CK, ck + (nck - 1) * DK * W,
                                         nxt);
    for (int64_t c = nck - 1; c >= 0; --c) {
        const Interval<RPL, E> cur = nxt;
        if (c > 0)
            load_interval<DK, E, MODE, true>(p, bh, slice, (c - 1) * CK, ck + (c - 1) * DK * W,
                                             nxt);
        const int64_t t0 = c * CK;
        const int n = L - t0 < CK ? (int)(L - t0) : CK;
        auto reverse = [&](auto full) {
#pragma unroll
        for (int m = 0; m < RPL; ++m) {
#pragma unroll
            for (int j = 0; j < W; ++j) S[m][j] = cur.ck[m][j];
        }
        // recompute the interval's states S_{t-1} and residuals e_t
        const float vv = f32(cur.vcol);
#pragma unroll
        for (int tau = 0; tau < CK; ++tau) {
            if (decltype(full)::value || tau < n) {
                float part[W] = {};
#pragma unroll
                for (int m = 0; m < RPL; ++m) {
                    const float a = decay(cur, m, tau), km = f32(cur.k[m][tau]);
#pragma unroll
                    for (int j = 0; j < W; ++j) {
                        S[m][j] *= a;
                        part[j] += km * S[m][j];
                    }
                    st_row(&sSt[tau][m][l][0], S[m]);
                }
                float tot[W];
                column_totals(part, tot);
                const float beta = read_lane(gate(cur.bcol, gbf), tau);
                float e[W];
#pragma unroll
                for (int j = 0; j < W; ++j) {
                    e[j] = read_lane(vv, tau * W + j) - tot[j];
                    const float u = beta * e[j];
#pragma unroll
                    for (int m = 0; m < RPL; ++m) S[m][j] += f32(cur.k[m][tau]) * u;
                }
                if (l == 0) st_row(&sE[tau][0], e);
            }
        }
        __syncthreads();
        // reverse step over the interval's tokens
        const float dov = f32(cur.docol);
#pragma unroll
        for (int tau = CK - 1; tau >= 0; --tau) {
            if (decltype(full)::value || tau < n) {
                const int64_t t = t0 + tau;
                const float beta = read_lane(gate(cur.bcol, gbf), tau);
                float e[W], u[W], dd[W];
                ld_row(&sE[tau][0], e);
#pragma unroll
                for (int j = 0; j < W; ++j) {
                    u[j] = beta * e[j];
                    dd[j] = read_lane(dov, tau * W + j);
                }
                // dq = S_t do^T with S_t = S~ + k^T u: the k part is k (u . do)
                float ud = 0.f;
#pragma unroll
                for (int j = 0; j < W; ++j) ud += u[j] * dd[j];
                float St[RPL][W], a[RPL], part[W] = {};
#pragma unroll
                for (int m = 0; m < RPL; ++m) {
                    ld_row(&sSt[tau][m][l][0], St[m]);
                    a[m] = decay(cur, m, tau);
                    const float km = f32(cur.k[m][tau]), qm = f32(cur.q[m][tau]);
                    float dq = km * ud;
#pragma unroll
                    for (int j = 0; j < W; ++j) {
                        dq += St[m][j] * dd[j];
                        G[m][j] += qm * dd[j];
                        part[j] += km * G[m][j];
                    }
                    // S~ of this row and token is in registers now: its LDS slot
                    // keeps the row's dq, dk and d ln alpha until the interval's
                    // atomics
                    sSt[tau][m][l][0] = dq;
                }
                float gu[W];
                column_totals(part, gu);
                float db = 0.f;
#pragma unroll
                for (int j = 0; j < W; ++j) db += gu[j] * e[j];
                float ge[W];
#pragma unroll
                for (int j = 0; j < W; ++j) ge[j] = beta * gu[j];
                // dv and dbeta (and a head gate's d ln alpha below) are staged
                // in LDS and written once per interval by all lanes
                if (l == 0) {
                    st_row(&sDV[tau * W], ge);
                    sDB[tau] = db;
                }
                // with gS~ = G - k^T ge:  dk = G u^T - S~ ge^T,
                // d ln alpha = sum_j gS~ S~ = G.S~ - k (S~ ge^T),  G <- diag(alpha) gS~
                float dla_head = 0.f;
#pragma unroll
                for (int m = 0; m < RPL; ++m) {
                    const float km = f32(cur.k[m][tau]);
                    float gu_m = 0.f, sge = 0.f, gs = 0.f;
#pragma unroll
                    for (int j = 0; j < W; ++j) {
                        gu_m += G[m][j] * u[j];
                        sge += St[m][j] * ge[j];
                        gs += G[m][j] * St[m][j];
                    }
                    const float ak = a[m] * km;
#pragma unroll
                    for (int j = 0; j < W; ++j) G[m][j] = a[m] * G[m][j] - ak * ge[j];
                    sSt[tau][m][l][1] = gu_m - sge;
                    const float dla = gs - km * sge;
                    if constexpr (MODE == KDA_ALPHA_CHANNEL)
                        sSt[tau][m][l][2] = dla;
                    dla_head += dla;
                }
                if constexpr (MODE == KDA_ALPHA_HEAD) {
                    dla_head = group_sum<64>(dla_head);
                    if (l == 0) sDH[tau] = dla_head;
                }
            }
        }
        __syncthreads();
        // lane l: dv of token t0 + l / W, column j0 + l % W; lanes < CK: dbeta
        // (and d ln alpha of a head gate) of token t0 + l
        if (l < CK * W && (decltype(full)::value || (l / W) < n))
            p.dv_out[(bh * L + t0 + l / W) * p.dv + j0 + l % W] = sDV[l];
        // this slice's share of dq, dk (and a channel gate's d ln alpha) for
        // the interval's tokens, added with one atomic per row and token
#pragma unroll
        for (int tau = 0; tau < CK; ++tau) {
            if (decltype(full)::value || tau < n) {
                const int64_t row0 = (bh * L + t0 + tau) * DK + l;
#pragma unroll
                for (int m = 0; m < RPL; ++m) {
                    unsafeAtomicAdd(p.dq + row0 + 64 * m, sSt[tau][m][l][0]);
                    unsafeAtomicAdd(p.dk + row0 + 64 * m, sSt[tau][m][l][1]);
                    if constexpr (MODE == KDA_ALPHA_CHANNEL)
                        unsafeAtomicAdd(p.dlog_alpha + row0 + 64 * m, sSt[tau][m][l][2]);
                }
            }
        }
        if (l < CK && (decltype(full)::value || l < n)) {
            unsafeAtomicAdd(p.dbeta + bh * L + t0 + l, sDB[l]);
            if constexpr (MODE == KDA_ALPHA_HEAD)
                unsafeAtomicAdd(p.dlog_alpha + bh * L + t0 + l, sDH[l]);
        }
        __syncthreads();
        };
        if (n == CK)
            reverse(Flag<true>{});
        else
            reverse(Flag<false>{});
    }
    if (p.dS0) {
#pragma unroll
        for (int m = 0; m < RPL; ++m) {
            st_row(p.dS0 + (bh * DK + l + 64 * m) * p.dv + j0, G[m]);
        }
    }
}

__global__ void __launch_bounds__(256) kda_zero_kernel(float* a, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        a[i] = 0.f;
}

hipError_t zero(float* a, int64_t n, hipStream_t stream) {
    if (!a || n == 0) return hipSuccess;
    const int64_t blocks = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
    hipLaunchKernelGGL(kda_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a, n);
    return hipGetLastError();
}

// ---- raw inputs: preprocessing before, chain rule after --------------------
// One wave per (head, token) row.  Prep: q and k (normalized when asked) and
// v, dJ/do as fp32; beta (through the sigmoid when asked) and ln alpha (-exp
// of the raw gate when asked) as fp32; |q| and |k|.  Post: dq and dk through
// the normalization, dbeta through the sigmoid, d ln alpha through -exp.
template <typename E, typename G>
__global__ void __launch_bounds__(64) kda_bwd_prep_kernel(BwdPrep p) {
    const int l = lane_id();
    const int64_t row = blockIdx.x;  // bh * L + t
    const E* q = (const E*)p.q + row * p.DK;
    const E* k = (const E*)p.k + row * p.DK;
    float sq = 0.f, sk = 0.f;
    for (int i = l; i < p.DK; i += 64) {
        const float a = to_f32(q[i]), b = to_f32(k[i]);
        sq += a * a;
        sk += b * b;
    }
    sq = group_sum<64>(sq);
    sk = group_sum<64>(sk);
    const bool norm = p.flags & KDA_IN_NORM_QK;
    const float iq = norm ? inv_norm(sq) : 1.f, ik = norm ? inv_norm(sk) : 1.f;
    for (int i = l; i < p.DK; i += 64) {
        p.qn[row * p.DK + i] = to_f32(q[i]) * iq;
        p.kn[row * p.DK + i] = to_f32(k[i]) * ik;
    }
    for (int i = l; i < p.DV; i += 64) {
        p.v32[row * p.DV + i] = to_f32(((const E*)p.v)[row * p.DV + i]);
        p.do32[row * p.DV + i] = to_f32(((const E*)p.dout)[row * p.DV + i]);
    }
    const bool raw_gate = p.flags & KDA_IN_GATE_RAW;
    if (p.alpha_mode == KDA_ALPHA_CHANNEL) {
        for (int i = l; i < p.DK; i += 64) {
            const float g = to_f32(((const G*)p.log_alpha)[row * p.DK + i]);
            p.la32[row * p.DK + i] = raw_gate ? log_alpha_of_raw(g) : g;
        }
    }
    if (l == 0) {
        const float b = to_f32(((const G*)p.beta)[row]);
        p.b32[row] = (p.flags & KDA_IN_BETA_LOGIT) ? sigmoid(b) : b;
        if (p.alpha_mode == KDA_ALPHA_HEAD) {
            const float g = to_f32(((const G*)p.log_alpha)[row]);
            p.la32[row] = raw_gate ? log_alpha_of_raw(g) : g;
        }
        p.nq[row] = sqrtf(sq);
        p.nk[row] = sqrtf(sk);
    }
}

__global__ void __launch_bounds__(64) kda_bwd_post_kernel(BwdPrep p) {
    const int l = lane_id();
    const int64_t row = blockIdx.x;
    if (p.flags & KDA_IN_NORM_QK) {
        // d raw = (dn - n (n . dn)) / |x| above the 1e-12 floor, dn / 1e-12 at it
#pragma unroll
        for (int w = 0; w < 2; ++w) {
            float* d = (w ? p.dk : p.dq) + row * p.DK;
            const float* xn = (w ? p.kn : p.qn) + row * p.DK;
            const float nrm = (w ? p.nk : p.nq)[row];
            float dot = 0.f;
            for (int i = l; i < p.DK; i += 64) dot += xn[i] * d[i];
            dot = group_sum<64>(dot);
            for (int i = l; i < p.DK; i += 64)
                d[i] = nrm > 1e-12f ? (d[i] - xn[i] * dot) / nrm : d[i] / 1e-12f;
        }
    }
    if ((p.flags & KDA_IN_GATE_RAW) && p.alpha_mode == KDA_ALPHA_CHANNEL)
        for (int i = l; i < p.DK; i += 64) p.dlog_alpha[row * p.DK + i] *= p.la32[row * p.DK + i];
    if (l == 0) {
        if (p.flags & KDA_IN_BETA_LOGIT) {
            const float b = p.b32[row];
            p.dbeta[row] *= b * (1.f - b);
        }
        if ((p.flags & KDA_IN_GATE_RAW) && p.alpha_mode == KDA_ALPHA_HEAD)
            p.dlog_alpha[row] *= p.la32[row];
    }
}

}  // namespace

int64_t bwd_workspace_bytes(int64_t bh, int64_t L, int dk, int dv) {
    return bh * ((L + CK - 1) / CK) * dk * dv * 4;
}

hipError_t zero_bwd_outputs(const BwdParams& prm, int dk, hipStream_t stream) {
    const int64_t tok = prm.BH * prm.L;
    hipError_t err = zero(prm.dq, tok * dk, stream);
    if (err == hipSuccess) err = zero(prm.dk, tok * dk, stream);
    if (err == hipSuccess && prm.alpha_mode != KDA_ALPHA_NONE)
        err = zero(prm.dlog_alpha, prm.alpha_mode == KDA_ALPHA_CHANNEL ? tok * dk : tok, stream);
    if (err == hipSuccess) err = zero(prm.dbeta, tok, stream);
    return err;
}

hipError_t launch_bwd(const BwdParams& prm, int dk, int qkv_bf16, hipStream_t stream) {
    if (prm.BH == 0) return hipSuccess;
    const dim3 grid((unsigned)(prm.BH * (prm.dv / W)));
#define KDA_MODES(DK_, E_)                                                                 \
    if (dk == DK_ && (qkv_bf16 != 0) == (sizeof(E_) == 2)) {                              \
        if (prm.alpha_mode == KDA_ALPHA_CHANNEL)                                           \
            hipLaunchKernelGGL((kda_bwd_kernel<DK_, E_, KDA_ALPHA_CHANNEL>), grid, dim3(64), 0, \
                               stream, prm);                                               \
        else if (prm.alpha_mode == KDA_ALPHA_HEAD)                                         \
            hipLaunchKernelGGL((kda_bwd_kernel<DK_, E_, KDA_ALPHA_HEAD>), grid, dim3(64), 0,    \
                               stream, prm);                                               \
        else                                                                               \
            hipLaunchKernelGGL((kda_bwd_kernel<DK_, E_, KDA_ALPHA_NONE>), grid, dim3(64), 0,    \
                               stream, prm);                                               \
        return hipGetLastError();                                                          \
    }
    KDA_MODES(128, bf16)
    KDA_MODES(64, bf16)
    KDA_MODES(128, float)
    KDA_MODES(64, float)
#undef KDA_MODES
    return hipErrorInvalidValue;
}

hipError_t launch_bwd_prep(const BwdPrep& prm, int qkv_bf16, int gate_bf16, hipStream_t stream) {
    if (prm.rows == 0) return hipSuccess;
    const dim3 grid((unsigned)prm.rows);
    if (qkv_bf16 && gate_bf16)
        hipLaunchKernelGGL((kda_bwd_prep_kernel<bf16, bf16>), grid, dim3(64), 0, stream, prm);
    else if (qkv_bf16)
        hipLaunchKernelGGL((kda_bwd_prep_kernel<bf16, float>), grid, dim3(64), 0, stream, prm);
    else if (gate_bf16)
        hipLaunchKernelGGL((kda_bwd_prep_kernel<float, bf16>), grid, dim3(64), 0, stream, prm);
    else
        hipLaunchKernelGGL((kda_bwd_prep_kernel<float, float>), grid, dim3(64), 0, stream, prm);
    return hipGetLastError();
}

hipError_t launch_bwd_post(const BwdPrep& prm, hipStream_t stream) {
    if (prm.rows == 0) return hipSuccess;
    hipLaunchKernelGGL(kda_bwd_post_kernel, dim3((unsigned)prm.rows), dim3(64), 0, stream, prm);
    return hipGetLastError();
}

}  // namespace kda
