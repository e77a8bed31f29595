// kda_chunk.hip -- fused chunkwise-parallel prefill of the KDA / gated delta rule
// for gfx950 (MI355X).
//
// Math: "22,580: From GPT-2 to Kimi K3" (yichencityu.github.io) section 6.3 gives
// the alpha = 1 chunk form; the gated and per-channel forms below follow from
// unrolling the recurrence inside a chunk (the pages stop before printing them,
// sections 08 and 9.1).  For a chunk of C tokens entering with state S, with
// g_r = sum_{s<=r} ln(alpha_s) (chunk-relative, inclusive; per key channel in
// KDA, per token otherwise):
//
//   A_rj = beta_r sum_c k_rc k_jc e^{g_rc - g_jc}   (j < r)       strictly lower
//   T    = (I + A)^-1                                             forward substitution
//   u    = T diag(beta) (V - (K * e^g) S)                         corrected values
//   P_rj = sum_c q_rc k_jc e^{g_rc - g_jc}           (j <= r)
//   O    = (Q * e^g) S + P u
//   S   <- diag(e^{g_n}) S + (K * e^{g_n - g})^T u                 g_n: last token
//
// (The pages' alpha = 1 form writes u = U - W S with W = T diag(beta) K and
// U = T diag(beta) V; merging the two products into T diag(beta)(V - K S) keeps
// W off chip and out of the per-chunk work.)
//
// One workgroup (8 waves, two per SIMD) owns one (b, h) head and one slice of NV state
// columns; columns of S evolve independently, so slices never talk.  It walks
// the chunks in order with its fp32 state slice resident in registers, and
// fetches chunk i+1's inputs into registers while chunk i computes.  Per chunk:
//   G  inputs to LDS (and decay factors)
//   AP A and P in 16x16 blocks on MFMA (k = key channels)
//   T  diagonal 16x16 blocks of T by forward substitution (one lane per column),
//      off-diagonal blocks by T_RJ = -T_RR sum_M A_RM T_MJ on fp32 MFMA; each
//      block is also written as T diag(beta) in operand precision
//   S  X = V - K~ S;  u = T' X;  o = Q~ S + P u;  S = e^{g_n} S + K^^T u
//
// Scalar decay (one alpha per token: Gated DeltaNet, or alpha = 1): e^{g_r - g_j}
// leaves every channel sum, so A, P, K S and Q S take the stored bf16 inputs as
// MFMA operands unchanged and the decay is applied to the fp32 results.
//
// Per-channel decay (KDA): e^{g_rc - g_jc} stays inside the sums and is split
// at the end of r's 16-token sub-block R (cumulative G_{R+1}): the row operand
// carries e^{g_r - G_{R+1}} (>= 1, at most e^{16 |ln alpha|}), the column
// operand e^{G_{J+1} - g_j} (<= 1) and, for J < R, a per-channel pair scale
// e^{G_{R+1} - G_{J+1}} (<= 1).  A diagonal pair therefore uses both stored
// operands unscaled.  The bound on the row factor is why the KDA path asks for
// ln(alpha) >= -5 per token and channel.
#include <type_traits>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

template <int DK_, int NV_, int C_, typename E_, int AMODE_>
struct ChunkCfg {
    typedef E_ E;
    static constexpr int DK = DK_, NV = NV_, C = C_, AMODE = AMODE_;
    static constexpr bool KDA = AMODE == KDA_ALPHA_CHANNEL;  // per-channel decay
    static constexpr int NB = C / 16;                  // 16-token sub-blocks per chunk
    static constexpr int NPAIR = NB * (NB + 1) / 2;    // (R, J <= R) block pairs
    static constexpr int ESZ = sizeof(E);
    // Row pitches: operand tiles are read 16 bytes per lane as (row l%16,
    // 16-byte column l/16); on gfx950 those reads are free of bank conflicts
    // when the pitch is 32 (mod 64) bytes, so rows carry 32 bytes of padding.
    static constexpr int PADE = 32 / ESZ;
    static constexpr int PK = DK + PADE;               // pitch of [*][DK] tiles
    static constexpr int PC = C + PADE;                // pitch of [*][C] tiles
    static constexpr int PV = NV + PADE;               // pitch of [C][NV] tiles
    static constexpr int PA = C + 4;                   // pitch of the fp32 A/T tile
    static constexpr int PKH = PK;                     // pitch of the KDA K^ tile (read transposed)
    static constexpr int NCB = DK / 16, NVB = NV / 16; // 16x16 blocks of the state slice
    static constexpr int NW = 8;                       // waves per workgroup (2 per SIMD)
    static constexpr int NTHREADS = 64 * NW;
    static constexpr int SBW = (NCB * NVB + NW - 1) / NW;  // state blocks per wave

    // LDS byte offsets.  Tiles: K row operand (KDA: k e^{g-G_{R+1}}; scalar: k,
    // also read transposed for the state update), Q row operand, KDA only: the
    // column operand k e^{G_{J+1}-g} and K^ = k e^{g_n-g} (read transposed);
    // T', P, v slice, S^T (double buffered), X^T (then o), u^T, scalar only:
    // (e^{g_n-g} u)^T.
    static constexpr int O_KR = 0;
    static constexpr int O_QR = O_KR + C * PK * ESZ;
    static constexpr int O_KC = O_QR + C * PK * ESZ;
    static constexpr int SZ_KC = KDA ? C * PK * ESZ : 0;
    static constexpr int O_KT = O_KC + SZ_KC;
    static constexpr int SZ_KT = KDA ? C * PKH * ESZ : 0;
    static constexpr int O_TB = O_KT + SZ_KT;
    static constexpr int O_P = O_TB + C * PC * ESZ;
    static constexpr int O_V = O_P + C * PC * ESZ;
    static constexpr int O_ST0 = O_V + C * PV * ESZ;
    static constexpr int O_ST1 = O_ST0 + NV * PK * ESZ;
    static constexpr int SZ_XT = (NV * PC > C * PV ? NV * PC : C * PV) * ESZ;  // X^T, then o
    static constexpr int O_XT = O_ST1 + NV * PK * ESZ;
    static constexpr int O_UT = O_XT + SZ_XT;
    static constexpr int O_UHT = O_UT + NV * PC * ESZ;
    static constexpr int SZ_UHT = KDA ? 0 : NV * PC * ESZ;
    static constexpr int O_A = O_UHT + SZ_UHT;
    static constexpr int O_GATE = O_A + C * PA * 4;
    // KDA gate area: Z[NB][DK], E'[NB][DK], Y'[NPAIR][DK], e^{g_n}[DK]
    // scalar gate area: g[C], e^g[C], e^{g_n-g}[C], e^{g_n} (one float, padded)
    static constexpr int SZ_GATE = KDA ? (2 * NB + NPAIR + 1) * DK * 4 : (3 * C + 4) * 4;
    static constexpr int O_BETA = O_GATE + SZ_GATE;
    static constexpr int LDS_BYTES = O_BETA + C * 4;

    static_assert(DK % 32 == 0 && NV % 16 == 0 && (C == 32 || C == 64), "tile shape");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget of one gfx950 CU");
};

template <typename E>
__device__ __forceinline__ void st2(E* p, float a, float b) {
    if constexpr (sizeof(E) == 2) {
        bf16x2 v;
        v[0] = (bf16)a;
        v[1] = (bf16)b;
        *(bf16x2*)p = v;
    } else {
        floatx2 v;
        v[0] = a;
        v[1] = b;
        *(floatx2*)p = v;
    }
}

template <typename E>
__device__ __forceinline__ void st4(E* p, floatx4 v) {
    if constexpr (sizeof(E) == 2) {
        bf16x4 t;
        t[0] = (bf16)v[0];
        t[1] = (bf16)v[1];
        t[2] = (bf16)v[2];
        t[3] = (bf16)v[3];
        *(bf16x4*)p = t;
    } else {
        *(floatx4*)p = v;
    }
}

__device__ __forceinline__ void pair_of(int p, int& R, int& J) {
    R = 0;
    while (p >= R + 1) {
        p -= R + 1;
        ++R;
    }
    J = p;
}

// v if keep, else zero (an explicit mask: a select of 16-byte values can be
// lowered into a select of stack addresses)
__device__ __forceinline__ uint4 keep_or_zero(uint4 v, bool keep) {
    const uint32_t m = keep ? 0xffffffffu : 0u;
    return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m);
}

// Load through a uniform base pointer plus a 32-bit byte offset (saddr form).
template <typename T>
__device__ __forceinline__ T ldg(const void* base, uint32_t byte_off) {
    return *(const T*)((const char*)base + byte_off);
}

template <class Cfg, bool GBF>
__global__ void __launch_bounds__(Cfg::NTHREADS)
kda_chunk_kernel(ChunkParams prm) {
    typedef typename Cfg::E E;
    typedef Frag<E> F;
    constexpr int DK = Cfg::DK, NV = Cfg::NV, C = Cfg::C, NB = Cfg::NB, AMODE = Cfg::AMODE;
    constexpr bool KDA = Cfg::KDA;
    constexpr int PK = Cfg::PK, PC = Cfg::PC, PV = Cfg::PV, PA = Cfg::PA;
    constexpr int PKH = Cfg::PKH;
    constexpr int NCB = Cfg::NCB, NVB = Cfg::NVB, NW = Cfg::NW, NT = Cfg::NTHREADS;
    constexpr int SBW = Cfg::SBW;
    constexpr int ESZ = Cfg::ESZ;

    __shared__ __attribute__((aligned(16))) char smem[Cfg::LDS_BYTES];
    E* sKr = (E*)(smem + Cfg::O_KR);
    E* sQr = (E*)(smem + Cfg::O_QR);
    E* sKc = (E*)(smem + Cfg::O_KC);
    E* sKh = (E*)(smem + Cfg::O_KT);
    E* sTb = (E*)(smem + Cfg::O_TB);
    E* sP = (E*)(smem + Cfg::O_P);
    E* sV = (E*)(smem + Cfg::O_V);
    E* sST0 = (E*)(smem + Cfg::O_ST0);
    E* sST1 = (E*)(smem + Cfg::O_ST1);
    E* sXT = (E*)(smem + Cfg::O_XT);
    E* sO = (E*)(smem + Cfg::O_XT);  // o tile reuses the X^T area after u is formed
    E* sUT = (E*)(smem + Cfg::O_UT);
    E* sUhT = (E*)(smem + Cfg::O_UHT);
    float* sA = (float*)(smem + Cfg::O_A);
    float* sGate = (float*)(smem + Cfg::O_GATE);
    float* sBeta = (float*)(smem + Cfg::O_BETA);
    // KDA gate views
    float* sZ = sGate;
    float* sE = sGate + NB * DK;
    float* sY = sGate + 2 * NB * DK;
    float* sGnv = sGate + (2 * NB + Cfg::NPAIR) * DK;
    // scalar gate views
    float* sG = sGate;
    float* sEg = sGate + C;
    float* sEgn = sGate + 2 * C;
    float* sGn1 = sGate + 3 * C;

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
    const int l = tid & 63;
    const int lr = l & 15, lq = l >> 4;

    // ---- which (head, column slice) this workgroup owns --------------------
    // Dispatch places workgroup i on XCD i % 8; give all slices of a head the
    // same XCD so their shared q/k/gate reads hit one L2.
    const int total = prm.BH * prm.n_slices;
    int pidx = blockIdx.x;
    if ((total & 7) == 0) pidx = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
    const int bh = pidx / prm.n_slices;
    const int slice = pidx % prm.n_slices;
    const int v0 = slice * NV;
    const int64_t L = prm.L;
    const int DV = prm.DV;

    // per-head base pointers (64-bit, uniform); all offsets below are 32-bit
    const char* gq = (const char*)prm.q + (int64_t)bh * L * DK * ESZ;
    const char* gk = (const char*)prm.k + (int64_t)bh * L * DK * ESZ;
    const char* gv = (const char*)prm.v + (int64_t)bh * L * DV * ESZ + v0 * ESZ;
    char* go = (char*)prm.o + (int64_t)bh * L * DV * ESZ + v0 * ESZ;
    constexpr int GSZ = GBF ? 2 : 4;
    const char* gla = (const char*)prm.log_alpha +
                      (int64_t)bh * L * (KDA ? DK : 1) * GSZ;
    const char* gbeta = (const char*)prm.beta + (int64_t)bh * L * GSZ;

    // ---- zero the triangular operand tiles once (upper blocks stay zero) ---
    for (int i = tid; i < C * PC; i += NT) {
        sTb[i] = from_f32<E>(0.f);
        sP[i] = from_f32<E>(0.f);
    }

    // ---- initial state slice into registers, and its operand copy ----------
    // Wave w holds the 16x16 state blocks item = w + NW i (cb = item % NCB,
    // vb = item / NCB); lane element e is S[16cb + 4lq + e][16vb + lr].
    floatx4 Sreg[SBW];
#pragma unroll
    for (int i = 0; i < SBW; ++i) Sreg[i] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (prm.S0) {  // uniform branch: all loads issue before the first use
        const float* s0 = prm.S0 + (int64_t)bh * DK * DV + v0;
#pragma unroll
        for (int i = 0; i < SBW; ++i) {
            const int item = w + NW * i;
            if (item < NCB * NVB) {
                const int cb = item % NCB, vb = item / NCB;
#pragma unroll
                for (int e = 0; e < 4; ++e) Sreg[i][e] = s0[(16 * cb + 4 * lq + e) * DV + 16 * vb + lr];
            }
        }
    }
#pragma unroll
    for (int i = 0; i < SBW; ++i) {
        const int item = w + NW * i;
        if (item < NCB * NVB) {
            const int cb = item % NCB, vb = item / NCB;
            store_acc_transposed<E>(sST0 + (16 * vb) * PK + 16 * cb, PK, Sreg[i]);
        }
    }

    // ---- raw registers of the next chunk's inputs ---------------------------
    // Every load reads a clamped, in-bounds token (the last valid one of a
    // ragged tail) and is masked when used, so the loads carry no branches and
    // all stay in flight together while the previous chunk computes.
    constexpr int VPIECE = 16 / ESZ;              // elements per 16-byte piece
    constexpr int VPPR = NV / VPIECE;             // pieces per row of the v slice
    constexpr int VPT = (C * VPPR + NT - 1) / NT; // pieces per thread
    uint4 rv[VPT];
    uint32_t rb = 0, rla = 0;

    // KDA: thread (c, R) owns key channel c of 16-token sub-block R
    const int kc = tid % DK, kR = tid / DK;
    const bool kact = KDA && kR < NB;
    uint32_t rq[KDA ? 16 : 1], rk[KDA ? 16 : 1], rg[KDA ? 16 : 1];  // raw element bits

    // scalar decay: q and k rows as 16-byte pieces
    constexpr int TW = VPIECE;
    constexpr int PPR = DK / TW;                  // pieces per q/k row
    constexpr int QPT = (C * PPR) / NT;           // pieces per thread and tensor
    static_assert(KDA || (C * PPR) % NT == 0, "scalar-decay copy split");
    uint4 rqp[KDA ? 1 : QPT], rkp[KDA ? 1 : QPT];

    auto load_chunk = [&](int64_t ch) {
        const int64_t t0 = ch * C;
        const int n = (int)((L - t0) < C ? (L - t0) : C);
        const uint32_t tb = (uint32_t)t0;  // chunk's first token (fits: checked on the host)
        if constexpr (KDA) {
            if (kact) {
#pragma unroll
                for (int s = 0; s < 16; ++s) {
                    const uint32_t r = (uint32_t)((16 * kR + s) < n ? (16 * kR + s) : (n - 1));
                    const uint32_t el = (tb + r) * DK + kc;
                    if constexpr (ESZ == 2) {
                        rq[s] = ldg<uint16_t>(gq, el * 2);
                        rk[s] = ldg<uint16_t>(gk, el * 2);
                    } else {
                        rq[s] = ldg<uint32_t>(gq, el * 4);
                        rk[s] = ldg<uint32_t>(gk, el * 4);
                    }
                    if constexpr (GBF) rg[s] = ldg<uint16_t>(gla, el * 2);
                    else rg[s] = ldg<uint32_t>(gla, el * 4);
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < QPT; ++i) {
                const int idx = tid + NT * i;
                const int r0 = idx / PPR, cc = (idx % PPR) * TW;
                const uint32_t r = r0 < n ? r0 : n - 1;
                rqp[i] = ldg<uint4>(gq, ((tb + r) * DK + cc) * ESZ);
                rkp[i] = ldg<uint4>(gk, ((tb + r) * DK + cc) * ESZ);
            }
            if constexpr (AMODE == KDA_ALPHA_HEAD) {
                if (tid < C) {
                    const uint32_t r = tid < n ? tid : n - 1;
                    if constexpr (GBF) rla = ldg<uint16_t>(gla, (tb + r) * 2);
                    else rla = ldg<uint32_t>(gla, (tb + r) * 4);
                }
            }
        }
        if (tid < C) {
            const uint32_t r = tid < n ? tid : n - 1;
            if constexpr (GBF) rb = ldg<uint16_t>(gbeta, (tb + r) * 2);
            else rb = ldg<uint32_t>(gbeta, (tb + r) * 4);
        }
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            int idx = tid + NT * i;
            idx = idx < C * VPPR ? idx : C * VPPR - 1;
            const int r = idx / VPPR, cc = (idx % VPPR) * VPIECE;
            const int rr = r < n ? r : n - 1;
            rv[i] = ldg<uint4>(gv, ((tb + rr) * DV + cc) * ESZ);
        }
    };
    // raw element bits -> fp32
    auto bits_f32 = [](uint32_t u, bool half) -> float {
        return half ? __uint_as_float(u << 16) : __uint_as_float(u);
    };

    const int64_t nchunks = (L + C - 1) / C;
    if (nchunks > 0) load_chunk(0);
    for (int64_t ch = 0; ch < nchunks; ++ch) {
        const int64_t t0 = ch * C;
        const int n = (int)((L - t0) < C ? (L - t0) : C);  // valid tokens in this chunk
        E* sSTc = (ch & 1) ? sST1 : sST0;
        E* sSTn = (ch & 1) ? sST0 : sST1;

        // ================= G: inputs into LDS =================================
        float ky[KDA ? 16 : 1];  // KDA: k * y for the K^ tile, kept across the barrier
        if constexpr (KDA) {
            if (kact) {
                const int R = kR;
                float a[16], qv[16], kv[16];
#pragma unroll
                for (int s = 0; s < 16; ++s) {
                    const bool valid = (16 * R + s) < n;
                    const float qq = bits_f32(rq[s], ESZ == 2);
                    const float kk2 = bits_f32(rk[s], ESZ == 2);
                    const float la = bits_f32(rg[s], GBF);
                    qv[s] = valid ? qq : 0.f;
                    kv[s] = valid ? kk2 : 0.f;
                    a[s] = valid ? la : 0.f;
                }
                // alpha = exp(ln alpha); x_s = prod_{s'<=s} alpha (within block)
                float x[16];
                float run = 1.f;
#pragma unroll
                for (int s = 0; s < 16; ++s) {
                    a[s] = exp_neg(a[s]);
                    run *= a[s];
                    x[s] = run;
                }
                // y_s = prod_{s' > s} alpha = e^{G_{R+1} - g_s} (<= 1)
                float yrun = 1.f;
#pragma unroll
                for (int s = 15; s >= 0; --s) {
                    ky[s] = kv[s] * yrun;
                    yrun *= a[s];
                }
                // x'_s = x_s / Z_R = e^{g_s - G_{R+1}} (>= 1)
                const float rz = 1.f / x[15];
#pragma unroll
                for (int s = 0; s < 16; ++s) {
                    const int r = 16 * R + s;
                    const float xp = x[s] * rz;
                    sKr[r * PK + kc] = from_f32<E>(kv[s] * xp);
                    sQr[r * PK + kc] = from_f32<E>(qv[s] * xp);
                    sKc[r * PK + kc] = from_f32<E>(ky[s]);
                }
                sZ[R * DK + kc] = x[15];
            }
        } else {
            // q, k rows; invalid rows become zero
#pragma unroll
            for (int i = 0; i < QPT; ++i) {
                const int idx = tid + NT * i;
                const int r0 = idx / PPR, cc = (idx % PPR) * TW;
                *(uint4*)(sQr + r0 * PK + cc) = keep_or_zero(rqp[i], r0 < n);
                *(uint4*)(sKr + r0 * PK + cc) = keep_or_zero(rkp[i], r0 < n);
            }
            // per-token decay: g = inclusive prefix sum of ln(alpha) over the chunk
            if (w == 0) {
                float g = 0.f;
                if constexpr (AMODE == KDA_ALPHA_HEAD)
                    g = wave_inclusive_sum((l < n) ? bits_f32(rla, GBF) : 0.f);
                const float gn = read_lane(g, C - 1);
                if (l < C) {
                    sG[l] = g;
                    sEg[l] = exp_neg(g);
                    sEgn[l] = exp_neg(gn - g);
                }
                if (l == 0) sGn1[0] = exp_neg(gn);
            }
        }
        if (tid < C) sBeta[tid] = (tid < n) ? bits_f32(rb, GBF) : 0.f;
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int idx = tid + NT * i;
            if (idx < C * VPPR) {
                const int r = idx / VPPR, cc = (idx % VPPR) * VPIECE;
                *(uint4*)(sV + r * PV + cc) = keep_or_zero(rv[i], r < n);
            }
        }
        // the registers are free again: start fetching the next chunk now, so
        // its HBM latency hides behind this chunk's work
        if (ch + 1 < nchunks) load_chunk(ch + 1);
        __syncthreads();

        // ================= G2 (KDA): cross-block factors, K^ tile =============
        if constexpr (KDA) {
            if (kact) {
                const int R = kR;
                float Zb[NB];
#pragma unroll
                for (int b = 0; b < NB; ++b) Zb[b] = sZ[b * DK + kc];
                float Fr = 1.f;  // e^{g_n - G_{R+1}} = prod of later blocks
#pragma unroll
                for (int b = 0; b < NB; ++b)
                    if (b > R) Fr *= Zb[b];
                // K^ = k y F, row-major [token][channel]
#pragma unroll
                for (int s = 0; s < 16; ++s) sKh[(16 * R + s) * PKH + kc] = from_f32<E>(ky[s] * Fr);
                if (R == 0) {
                    // block-end factors E'_R = e^{G_{R+1}}, pair scales
                    // Y'_RJ = e^{G_{R+1} - G_{J+1}} (1 on the diagonal), e^{g_n}
                    float run = 1.f;
#pragma unroll
                    for (int b = 0; b < NB; ++b) {
                        run *= Zb[b];
                        sE[b * DK + kc] = run;
                    }
                    sGnv[kc] = run;
                    int p = 0;
#pragma unroll
                    for (int rb2 = 0; rb2 < NB; ++rb2) {
#pragma unroll
                        for (int jb = 0; jb <= rb2; ++jb, ++p) {
                            float y = 1.f;
#pragma unroll
                            for (int m = 0; m < NB; ++m)
                                if (m > jb && m <= rb2) y *= Zb[m];
                            sY[p * DK + kc] = y;
                        }
                    }
                }
            }
            __syncthreads();
        }

        // ================= AP: A (fp32) and P (operand type) =================
        for (int p = w; p < Cfg::NPAIR; p += NW) {
            int R, J;
            pair_of(p, R, J);
            constexpr int NKS = DK / F::KS;
            const E* pa = (KDA ? sKc : sKr) + (16 * J + lr) * PK + F::W * lq;
            const E* pk = sKr + (16 * R + lr) * PK + F::W * lq;
            const E* pq = sQr + (16 * R + lr) * PK + F::W * lq;
            typename F::T fa[NKS], fk[NKS], fq[NKS];
            if (!KDA || J == R) {
#pragma unroll
                for (int i = 0; i < NKS; ++i) fa[i] = F::load(pa + F::KS * i);
            } else {
                const float* ps = sY + p * DK + F::W * lq;
#pragma unroll
                for (int i = 0; i < NKS; ++i) fa[i] = F::load_scaled(pa + F::KS * i, ps + F::KS * i);
            }
#pragma unroll
            for (int i = 0; i < NKS; ++i) {
                fk[i] = F::load(pk + F::KS * i);
                fq[i] = F::load(pq + F::KS * i);
            }
            floatx4 accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < NKS; ++i) {
                accA = F::mma(accA, fa[i], fk[i]);
                accP = F::mma(accP, fa[i], fq[i]);
            }
            // lane holds [m = j = 16J + 4lq + e][n = r = 16R + lr]
            const int rr = 16 * R + lr;
            const float br = sBeta[rr];
            float gr = 0.f;
            floatx4 gj = {0.f, 0.f, 0.f, 0.f};
            if constexpr (AMODE == KDA_ALPHA_HEAD) {
                gr = sG[rr];
                gj = *(const floatx4*)(sG + 16 * J + 4 * lq);
            }
            floatx4 va, vp;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int jj = 16 * J + 4 * lq + e;
                float f = 1.f;  // scalar decay e^{g_r - g_j}, applied to the result
                if constexpr (AMODE == KDA_ALPHA_HEAD) f = exp_neg(gr - gj[e]);
                va[e] = (J < R || jj < rr) ? br * accA[e] * f : 0.f;
                vp[e] = (J < R || jj <= rr) ? accP[e] * f : 0.f;
            }
            *(floatx4*)(sA + rr * PA + 16 * J + 4 * lq) = va;
            st4<E>(sP + rr * PC + 16 * J + 4 * lq, vp);
        }
        __syncthreads();

        // ================= T1: diagonal blocks by forward substitution =======
        // Wave R < NB solves block R.  Lane (j, s) = (l/4, l%4) owns rows
        // 4s..4s+3 of column j of T_RR, with those rows of A_RR in registers.
        // Right-looking sweep: once t_m is final, its owner lane hands it to
        // the other three lanes of the quad (DPP broadcast) and every row takes
        // its A_RR[i][m] t_m term; the dependent chain is 15 VALU steps long.
        // (A_RR[i][m] is zero for m >= i, so no row needs masking.)
        // Results: T_RR^T (fp32) in the diagonal block of sA, and
        // T_RR diag(beta) in operand precision in sTb.
        if (w < NB) {
            const int R = w, j = l >> 2, s4 = l & 3;
            floatx4 arow[4][4];  // arow[ii][q4] = A_RR[4 s4 + ii][4 q4 .. 4 q4 + 3]
#pragma unroll
            for (int ii = 0; ii < 4; ++ii)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4)
                    arow[ii][q4] = *(const floatx4*)(sA + (16 * R + 4 * s4 + ii) * PA + 16 * R + 4 * q4);
            float acc[4];
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) acc[ii] = (4 * s4 + ii == j) ? 1.f : 0.f;
#pragma unroll
            for (int m = 0; m < 15; ++m) {
                const float tm = quad_bcast(acc[m & 3], m >> 2);
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) acc[ii] -= arow[ii][m >> 2][m & 3] * tm;
            }
            floatx4 v4 = {acc[0], acc[1], acc[2], acc[3]};
            *(floatx4*)(sA + (16 * R + j) * PA + 16 * R + 4 * s4) = v4;
            const float bj = sBeta[16 * R + j];
#pragma unroll
            for (int ii = 0; ii < 4; ++ii)
                sTb[(16 * R + 4 * s4 + ii) * PC + 16 * R + j] = from_f32<E>(acc[ii] * bj);
        } else if constexpr (KDA) {
            // the other waves: rescale the row operands in place, K~ = k e^{g},
            // Q~ = q e^{g} (row operand x E'_R), for the state products
            constexpr int PER_ROW = DK / VPIECE;
            for (int i = tid - 64 * NB; i < 2 * C * PER_ROW; i += NT - 64 * NB) {
                const int which = i / (C * PER_ROW);
                const int rem = i % (C * PER_ROW);
                const int r = rem / PER_ROW, cc = (rem % PER_ROW) * VPIECE;
                E* p = (which ? sQr : sKr) + r * PK + cc;
                const float* sc = sE + (r >> 4) * DK + cc;
                if constexpr (sizeof(E) == 2) {
                    *(bf16x8*)p = Frag<bf16>::load_scaled((const bf16*)p, sc);
                } else {
                    *(floatx4*)p = Frag<float>::load_scaled((const float*)p, sc);
                }
            }
        }
        __syncthreads();

        // ================= T2: off-diagonal blocks, by distance ===============
        // T_RJ = -T_RR sum_{M=J}^{R-1} A_RM T_MJ; T_RJ^T is stored at block (J, R)
        // of sA, and T_RJ diag(beta) in sTb.
#pragma unroll
        for (int d = 1; d < NB; ++d) {
            const int R = d + w, J = w;
            if (R < NB) {
                floatx4 acc = {0.f, 0.f, 0.f, 0.f};
                for (int M = J; M < R; ++M) {
                    floatx4 af = *(const floatx4*)(sA + (16 * R + lr) * PA + 16 * M + 4 * lq);
                    floatx4 bf = *(const floatx4*)(sA + (16 * J + lr) * PA + 16 * M + 4 * lq);
                    acc = Frag<float>::mma(acc, af, bf);
                }
                // A operand T_RR[m][k] with m = lr, k = 4lq + s: stored transposed
                floatx4 tf;
#pragma unroll
                for (int s = 0; s < 4; ++s) tf[s] = sA[(16 * R + 4 * lq + s) * PA + 16 * R + lr];
                floatx4 z = {0.f, 0.f, 0.f, 0.f};
                floatx4 res = -Frag<float>::mma(z, tf, acc);
                *(floatx4*)(sA + (16 * J + lr) * PA + 16 * R + 4 * lq) = res;
                const float bj = sBeta[16 * J + lr];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sTb[(16 * R + 4 * lq + e) * PC + 16 * J + lr] = from_f32<E>(res[e] * bj);
            }
            __syncthreads();
        }

        // ================= S1: X = V - K~ S ===================================
        for (int item = w; item < NB * NVB; item += NW) {
            const int R = item % NB, vb = item / NB;
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = mma_block<E>(acc, sKr + (16 * R) * PK, PK, sSTc + (16 * vb) * PK, PK, DK);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * R + 4 * lq + e;
                float ks = acc[e];
                if constexpr (AMODE == KDA_ALPHA_HEAD) ks *= sEg[r];
                acc[e] = to_f32(sV[r * PV + 16 * vb + lr]) - ks;
            }
            store_acc_transposed<E>(sXT + (16 * vb) * PC + 16 * R, PC, acc);
        }
        __syncthreads();

        // ================= S2: u = T' X =======================================
        for (int item = w; item < NB * NVB; item += NW) {
            const int R = item % NB, vb = item / NB;
            constexpr int KS = Frag<E>::KS;
            const int K = ((16 * (R + 1) + KS - 1) / KS) * KS;
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = mma_block<E>(acc, sTb + (16 * R) * PC, PC, sXT + (16 * vb) * PC, PC, K);
            store_acc_transposed<E>(sUT + (16 * vb) * PC + 16 * R, PC, acc);
            if constexpr (!KDA) {
                // u scaled by e^{g_n - g} for the state update
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] *= sEgn[16 * R + 4 * lq + e];
                store_acc_transposed<E>(sUhT + (16 * vb) * PC + 16 * R, PC, acc);
            }
        }
        __syncthreads();

        // ================= S3: o = (Q e^g) S + P u ============================
        for (int item = w; item < NB * NVB; item += NW) {
            const int R = item % NB, vb = item / NB;
            constexpr int KS = Frag<E>::KS;
            const int K = ((16 * (R + 1) + KS - 1) / KS) * KS;
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = mma_block<E>(acc, sQr + (16 * R) * PK, PK, sSTc + (16 * vb) * PK, PK, DK);
            if constexpr (AMODE == KDA_ALPHA_HEAD) {
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] *= sEg[16 * R + 4 * lq + e];
            }
            acc = mma_block<E>(acc, sP + (16 * R) * PC, PC, sUT + (16 * vb) * PC, PC, K);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                sO[(16 * R + 4 * lq + e) * PV + 16 * vb + lr] = from_f32<E>(acc[e]);
        }

        // ================= S4: S = e^{g_n} S + K^^T u =========================
        // The K^ operand is read transposed out of its row-major tile.
        {
            const E* ub = KDA ? sUT : sUhT;
            const E* kt = KDA ? sKh : sKr;
            constexpr int LDK = KDA ? PKH : PK;
#pragma unroll
            for (int i = 0; i < SBW; ++i) {
                const int item = w + NW * i;
                if (item < NCB * NVB) {
                    const int cb = item % NCB, vb = item / NCB;
                    floatx4 acc = Sreg[i];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        if constexpr (KDA) acc[e] *= sGnv[16 * cb + 4 * lq + e];
                        else if constexpr (AMODE == KDA_ALPHA_HEAD) acc[e] *= sGn1[0];
                    }
                    acc = mma_block_at<E>(acc, kt, LDK, 16 * cb, ub + (16 * vb) * PC, PC, C);
                    Sreg[i] = acc;
                    store_acc_transposed<E>(sSTn + (16 * vb) * PK + 16 * cb, PK, acc);
                }
            }
        }
        __syncthreads();

        // ================= o tile -> HBM (valid rows only) ====================
        for (int i = tid; i < C * VPPR; i += NT) {
            const int r = i / VPPR, cc = (i % VPPR) * VPIECE;
            if (r < n)
                *(uint4*)(go + (((uint32_t)t0 + r) * DV + cc) * ESZ) = *(const uint4*)(sO + r * PV + cc);
        }
    }

    // ---- final state --------------------------------------------------------
    if (prm.S_final) {
        float* sf = prm.S_final + (int64_t)bh * DK * DV + v0;
#pragma unroll
        for (int i = 0; i < SBW; ++i) {
            const int item = w + NW * i;
            if (item < NCB * NVB) {
                const int cb = item % NCB, vb = item / NCB;
#pragma unroll
                for (int e = 0; e < 4; ++e) sf[(16 * cb + 4 * lq + e) * DV + 16 * vb + lr] = Sreg[i][e];
            }
        }
    }
}

// ---- host-side dispatch -----------------------------------------------------

template <int DK, int NV, int C, typename E, int AMODE>
static hipError_t launch_cfg(const ChunkParams& prm, hipStream_t stream) {
    typedef ChunkCfg<DK, NV, C, E, AMODE> Cfg;
    const int total = prm.BH * prm.n_slices;
    if (prm.gate_bf16)
        hipLaunchKernelGGL((kda_chunk_kernel<Cfg, true>), dim3(total), dim3(Cfg::NTHREADS), 0,
                           stream, prm);
    else
        hipLaunchKernelGGL((kda_chunk_kernel<Cfg, false>), dim3(total), dim3(Cfg::NTHREADS), 0,
                           stream, prm);
    return hipGetLastError();
}

template <int DK, int NV, int C, typename E>
static hipError_t launch_mode(const ChunkParams& prm, hipStream_t stream) {
    switch (prm.alpha_mode) {
        case KDA_ALPHA_NONE: return launch_cfg<DK, NV, C, E, KDA_ALPHA_NONE>(prm, stream);
        case KDA_ALPHA_HEAD: return launch_cfg<DK, NV, C, E, KDA_ALPHA_HEAD>(prm, stream);
        case KDA_ALPHA_CHANNEL: return launch_cfg<DK, NV, C, E, KDA_ALPHA_CHANNEL>(prm, stream);
        default: return hipErrorInvalidValue;
    }
}

int chunk_slice_width(int dk, int dv, int qkv_bf16, int64_t BH) {
    // Prefer wide slices while that still gives >= 256 workgroups; else 16.
    if (dk == 64 && qkv_bf16 && BH * (dv / 64) >= 256) return 64;
    if (BH * (dv / 32) >= 256) return 32;
    return 16;
}

hipError_t launch_chunk(ChunkParams prm, int dk, int qkv_bf16, int nv, hipStream_t stream) {
    if (prm.BH == 0) return hipSuccess;
    prm.n_slices = prm.DV / nv;
#define KDA_CASE(DK_, NV_, C_, E_)                                             \
    if (dk == DK_ && nv == NV_ && (qkv_bf16 != 0) == (sizeof(E_) == 2))        \
        return launch_mode<DK_, NV_, C_, E_>(prm, stream);
    KDA_CASE(128, 16, 64, bf16)
    KDA_CASE(128, 32, 64, bf16)
    KDA_CASE(64, 16, 64, bf16)
    KDA_CASE(64, 32, 64, bf16)
    KDA_CASE(64, 64, 64, bf16)
    KDA_CASE(128, 16, 32, float)
    KDA_CASE(128, 32, 32, float)
    KDA_CASE(64, 16, 32, float)
    KDA_CASE(64, 32, 32, float)
#undef KDA_CASE
    return hipErrorInvalidValue;
}

}  // namespace kda
