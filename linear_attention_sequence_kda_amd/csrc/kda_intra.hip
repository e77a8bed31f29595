// kda_intra.hip -- intra-chunk kernel of the two-kernel chunkwise prefill
// (gfx950 / MI355X).
//
// Math: "22,580: From GPT-2 to Kimi K3" (yichencityu.github.io) section 6.3
// gives the alpha = 1 chunk form (A, T = (I + A)^-1 by forward substitution,
// W = T diag(beta) K, U = T diag(beta) V, u = U - W S, O = Q S + P u); the
// gated and per-channel forms follow from unrolling the recurrence inside a
// chunk (the pages stop before printing them, sections 08 and 9.1).  For a
// chunk of C tokens with g_r = sum_{s<=r} ln(alpha_s) (chunk-relative,
// inclusive; per key channel in KDA, per token otherwise):
//
//   A_rj = beta_r sum_c k_rc k_jc e^{g_rc - g_jc}   (j < r)       strictly lower
//   T    = (I + A)^-1
//   W    = T diag(beta) (K * e^g),   U = T diag(beta) V
//   P_rj = sum_c q_rc k_jc e^{g_rc - g_jc}           (j <= r)
//
// and the inter-chunk kernel then runs, chunk after chunk,
//   u = U - W S,  O = (Q * e^g) S + P u,  S <- diag(e^{g_n}) S + (K * e^{g_n-g})^T u.
//
// None of this depends on the state, so one workgroup (8 waves) takes one
// (head, chunk) pair and the whole grid runs at once.  It writes one record
// per chunk (layout in kda_internal.h) with every operand already in the
// register order of the inter-chunk kernel's MFMA loops.
//
// Phases: G inputs to LDS and decay factors; AP A (fp32) and P on MFMA;
// T1 diagonal 16x16 blocks of T by forward substitution (one wave per block,
// pivots broadcast inside lane quads); T2 off-diagonal blocks
// T_RJ = -T_RR sum_M A_RM T_MJ on fp32 MFMA, level by level; WU W and U on
// MFMA.
//
// Scalar decay (one alpha per token: Gated DeltaNet, or alpha = 1): e^{g_r - g_j}
// leaves every channel sum, so A and P take the stored inputs as MFMA operands
// unchanged and the decay is applied to the fp32 results; W takes e^{g_j} on
// the columns of T diag(beta).
//
// Per-channel decay (KDA): e^{g_rc - g_jc} stays inside the sums and is split
// at 16-token sub-block boundaries (G_R = g just before sub-block R, Z_R =
// e^{G_{R+1} - G_R} the sub-block's decay, per channel).  The column operand
// carries e^{G_{J+1} - g_j} (<= 1).  For the row operand each sub-block R
// takes one of two splits:
//  * while Z_R >= 1e-30 in every channel (summed ln(alpha) >= -69): the
//    split at the sub-block's end, row factor e^{g_r - G_{R+1}} (>= 1, at
//    most 1e30), pair scale e^{G_{R+1} - G_{J+1}} = prod_{J<m<=R} Z_m (<= 1)
//    below the diagonal and none on it, so a diagonal pair multiplies the
//    stored operands as they are;
//  * otherwise ("flagged"): the split at its start, row factor e^{g_r - G_R}
//    (<= 1) and pair scale prod_{J<m<R} Z_m (<= 1), so no factor exceeds 1
//    whatever the decay; the diagonal blocks of A and P are then summed
//    directly, channel by channel with running products of alpha (exponents
//    never above 0), reduced across the wave and added into LDS.
#include "kda_device.h"
#include "kda_internal.h"
#include "kda_rev_record.h"

namespace kda {

template <int DK_, int DV_, int C_, typename E_, int AMODE_>
struct IntraCfg {
    typedef E_ E;
    static constexpr int DK = DK_, DV = DV_, C = C_, AMODE = AMODE_;
    static constexpr bool KDA = AMODE == KDA_ALPHA_CHANNEL;   // per-channel decay
    static constexpr bool HEADG = AMODE == KDA_ALPHA_HEAD;    // one decay per token
    static constexpr int NB = C / 16;                         // 16-token sub-blocks
    static constexpr int NPAIR = NB * (NB + 1) / 2;           // (R, J <= R) block pairs
    static constexpr int ESZ = sizeof(E);
    // Row pitches: operand tiles are read 16 bytes per lane as (row l%16,
    // 16-byte column l/16); on gfx950 those reads are free of bank conflicts
    // when the pitch is 32 (mod 64) bytes, so rows carry 32 bytes of padding.
    static constexpr int PADE = 32 / ESZ;
    static constexpr int PK = DK + PADE;                      // [C][DK] tiles
    static constexpr int PVV = DV + PADE;                     // [C][DV] tile
    static constexpr int PC = C + PADE;                       // [C][C] operand tiles
    static constexpr int PA = C + 4;                          // fp32 A / T^T tile
    static constexpr int NCB = DK / 16, NVB = DV / 16;
    static constexpr int NW = 8;
    static constexpr int NT = 64 * NW;

    // Scalar decay ("thin" record): only A and T are built here, the record
    // holds T diag(beta) and the decay scalars.
    static constexpr bool THIN = !KDA;

    // LDS: K row operand (KDA: k e^{g - G_{R+1}}, then K e^g in place),
    // KDA: Q row operand (then V) and column operand k e^{G_{J+1} - g};
    // A / T^T (fp32), T diag(beta), gate factors, beta.
    static constexpr int SZ_K = C * PK * ESZ;
    static constexpr int SZ_QV = THIN ? 0 : (PK > PVV ? PK : PVV) * C * ESZ;
    static constexpr int O_KR = 0;
    static constexpr int O_QV = O_KR + SZ_K;
    static constexpr int O_KC = O_QV + SZ_QV;
    static constexpr int O_A = O_KC + (KDA ? SZ_K : 0);
    // T diag(beta) lives in space whose operand is done once A (and P) are:
    // KDA's column operand (keeps the kernel at two workgroups per CU), the
    // scalar path's K tile (four workgroups per CU)
    static constexpr int O_TB = KDA ? O_KC : O_KR;
    static constexpr int O_GATE = O_A + C * PA * 4;
    // KDA: Z[NB][DK], E'[NB][DK]; scalar: g[C], e^g[C]
    static constexpr int SZ_GATE = KDA ? 2 * NB * DK * 4 : 2 * C * 4;
    static constexpr int O_BETA = O_GATE + SZ_GATE;
    // 1/|q_r| and 1/|k_r| of each token (KDA_IN_NORM_QK)
    static constexpr int O_QN = O_BETA + C * 4;
    static constexpr int O_KN = O_QN + C * 4;
    // KDA: one flag per wave (its sub-block's decay leaves the range of the
    // split), and the diagonal blocks of P summed directly for such
    // sub-blocks: with four sub-blocks they sit in blocks of the A tile above
    // its diagonal (free until T2 writes T^T there), with two in an area of
    // their own
    static constexpr int O_FLAG = O_KN + C * 4;
    static constexpr bool PD_IN_A = NB == 4;
    static constexpr int O_PD = O_FLAG + (KDA ? 64 : 0);
    static constexpr int LDS_BYTES = O_PD + (KDA && !PD_IN_A ? NB * 256 * 4 : 0);
    // a sub-block takes the direct path when some channel's summed ln(alpha)
    // is below this (e^-69 ~ 1e-30, so 1 / Z_R stays below ~1e30)
    static constexpr float UNSAFE_LOG = -69.0f;

    static_assert(DK % 32 == 0 && DV % 16 == 0 && (C == 32 || C == 64), "tile shape");
    static_assert(!KDA || NB * DK <= NT, "one thread per (channel, sub-block)");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget of one gfx950 CU");
    static_assert(C * PC * ESZ <= SZ_K, "T diag(beta) fits the K tile's space");
    // scalar path: registers for eight waves per SIMD (four workgroups per CU)
    static constexpr int MIN_WAVES = THIN ? 8 : 1;
};

template <class Cfg, bool GBF, bool WIDE, bool REV = false>
__global__ void __launch_bounds__(Cfg::NT) __attribute__((amdgpu_waves_per_eu(Cfg::MIN_WAVES)))
kda_intra_kernel(IntraParams prm) {
    typedef typename Cfg::E E;
    typedef Frag<E> F;
    constexpr int DK = Cfg::DK, DV = Cfg::DV, C = Cfg::C, NB = Cfg::NB;
    constexpr bool KDA = Cfg::KDA, HEADG = Cfg::HEADG, THIN = Cfg::THIN;
    constexpr int PK = Cfg::PK, PVV = Cfg::PVV, PC = Cfg::PC, PA = Cfg::PA;
    constexpr int NCB = Cfg::NCB, NVB = Cfg::NVB, NW = Cfg::NW, NT = Cfg::NT;
    constexpr int ESZ = Cfg::ESZ;
    constexpr int W = F::W, KS = F::KS;
    constexpr RecLayout RL = THIN ? rec_layout_thin(C, ESZ) : rec_layout(DK, DV, C, ESZ, KDA);

    __shared__ __attribute__((aligned(16))) char smem[Cfg::LDS_BYTES];
    E* sKr = (E*)(smem + Cfg::O_KR);
    E* sQr = (E*)(smem + Cfg::O_QV);
    E* sV = (E*)(smem + Cfg::O_QV);  // V replaces the Q operand once A and P are done
    E* sKc = (E*)(smem + Cfg::O_KC);
    float* sA = (float*)(smem + Cfg::O_A);
    E* sTb = (E*)(smem + Cfg::O_TB);
    float* sGate = (float*)(smem + Cfg::O_GATE);
    float* sBeta = (float*)(smem + Cfg::O_BETA);
    float* sQn = (float*)(smem + Cfg::O_QN);
    float* sKn = (float*)(smem + Cfg::O_KN);
    int* sFlag = (int*)(smem + Cfg::O_FLAG);
    float* sPd = (float*)(smem + Cfg::O_PD);
    // diagonal block R of P (direct sums) as 16 x 16 floats, pitch pd_ld
    constexpr int pd_ld = Cfg::PD_IN_A ? PA : 16;
    auto pd_block = [&](int R) -> float* {
        if constexpr (Cfg::PD_IN_A) {
            // blocks (0,1), (1,2), (2,3), (0,2) of the A tile (row, column)
            const int rb = R < 3 ? R : 0, cb = R < 3 ? R + 1 : 2;
            return sA + (16 * rb) * PA + 16 * cb;
        } else {
            return sPd + R * 256;
        }
    };
    const bool norm_qk = (prm.flags & KDA_IN_NORM_QK) != 0;
    const bool gate_raw = (prm.flags & KDA_IN_GATE_RAW) != 0;
    const bool beta_logit = (prm.flags & KDA_IN_BETA_LOGIT) != 0;
    float* sZ = sGate;                // KDA views
    float* sE = sGate + NB * DK;
    float* sG = sGate;                // scalar views
    float* sEg = sGate + C;

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63;
    const int lr = l & 15, lq = l >> 4;

    const int bh = blockIdx.x / prm.ncs;
    const int cs = blockIdx.x - bh * prm.ncs;
    const SeqRange sr = seq_range(prm.cu, prm.L, prm.H, bh);
    const int64_t L = sr.len;
    const int64_t t0 = (prm.c0 + cs) * C;
    if (t0 >= L) return;  // packed sequences: past this sequence's last chunk
    const int n = (int)((L - t0) < C ? (L - t0) : C);  // valid tokens, >= 1

    // chunk base pointers (64-bit, uniform); offsets below are 32-bit
    const int64_t row0 = sr.base + t0;
    const char* gq = (const char*)prm.q + row0 * DK * ESZ;
    const char* gk = (const char*)prm.k + row0 * DK * ESZ;
    const char* gv = (const char*)prm.v + row0 * DV * ESZ;
    constexpr int GSZ = GBF ? 2 : 4;
    // ln(alpha): [rows][DK], or one per token read by every channel (la_head)
    const uint32_t la_rs = (KDA && !prm.la_head) ? DK : 1, la_cs = prm.la_head ? 0 : 1;
    const char* gla = (const char*)prm.log_alpha + row0 * la_rs * GSZ;
    const char* gbeta = (const char*)prm.beta + row0 * GSZ;
    char* rec = (char*)prm.ws + ((int64_t)bh * prm.ncs + cs) * RL.bytes;
    E* rW = (E*)(rec + RL.w);
    E* rU = (E*)(rec + RL.ut);
    E* rP = (E*)(rec + RL.p);
    E* rKt = (E*)(rec + RL.kt);
    E* rQt = (E*)(rec + RL.qt);
    float* rGam = (float*)(rec + RL.gam);
    float* rRs = (float*)(rec + RL.rs);
    E* rTb = (E*)(rec + RL.tb);

    // Inputs: with per-channel decay the records carry everything the state
    // pass needs, so the inputs are read once and with the non-temporal hint
    // (they leave the memory-side cache to the records); the scalar-decay
    // state pass reads q, k and v again, so there they are ordinary loads.
    auto ld_in = [](const void* base, uint32_t off, auto tag) __attribute__((always_inline)) {
        typedef decltype(tag) T;
        if constexpr (KDA) return ldg_stream<T>(base, off);
        else return ldg<T>(base, off);
    };
    auto bits_f32 = [](uint32_t u, bool half) -> float {
        return half ? __uint_as_float(u << 16) : __uint_as_float(u);
    };

    // upper blocks of T diag(beta) are zeros (read by the W and U products,
    // or copied out whole); both paths zero them once the operand whose
    // space they share is done

    // ---- v: into registers now, into LDS once the Q tile is free ------------
    constexpr int VPIECE = 16 / ESZ;
    constexpr int VPPR = DV / VPIECE;
    constexpr int VPT = THIN ? 1 : (C * VPPR + NT - 1) / NT;
    uint4 rv[VPT];
#pragma unroll
    for (int i = 0; i < (THIN ? 0 : VPT); ++i) {
        int idx = tid + NT * i;
        idx = idx < C * VPPR ? idx : C * VPPR - 1;
        const int r = idx / VPPR, cc = (idx % VPPR) * VPIECE;
        const int rr = r < n ? r : n - 1;
        rv[i] = ld_in(gv, (rr * DV + cc) * ESZ, uint4{});
    }

    // ================= G: inputs into LDS, decay factors =====================
    const int kc = tid % DK, kR = tid / DK;  // KDA: (key channel, sub-block)
    const bool kact = KDA && kR < NB;
    float ky[KDA ? 16 : 1];                  // KDA: k * y, kept for K^
    // Every global load of the chunk (q and k pieces, ln(alpha), beta) is
    // issued here, before the first of them is waited for, so the inputs
    // arrive in one memory round trip; they are used below in order.  The
    // inputs are read once, with the non-temporal hint, so they leave the
    // memory-side cache to the span's records, which the state pass reads.
    constexpr int PPR = DK / VPIECE;          // 16-byte pieces per q/k row
    constexpr int QPT = (C * PPR + NT - 1) / NT;
    uint4 gqp[KDA ? QPT : 1], gkp[QPT];
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
        const int idx = tid + NT * i;
        if (idx < C * PPR) {
            const int r0 = idx / PPR, cc = (idx % PPR) * VPIECE;
            const int r = r0 < n ? r0 : n - 1;
            if constexpr (KDA) gqp[i] = ld_in(gq, (r * DK + cc) * ESZ, uint4{});
            gkp[i] = ld_in(gk, (r * DK + cc) * ESZ, uint4{});
        }
    }
    // raw bits of ln(alpha): KDA, thread (channel, sub-block) holds its 16
    // tokens; one decay per token, lane l holds token l.  These small loads
    // are made by every thread, at rows clamped into the chunk (the values
    // of inactive threads and rows are never used), so no branch sits
    // between a load and the later loads.
    uint32_t la_bits[KDA ? 16 : 1];
    if constexpr (KDA) {
        const int kRc = kR < NB ? kR : NB - 1;
#pragma unroll
        for (int s = 0; s < 16; ++s) {
            const int r = 16 * kRc + s;
            const int rr = r < n ? r : n - 1;
            const uint32_t el = rr * la_rs + kc * la_cs;
            la_bits[s] = GBF ? (uint32_t)ld_in(gla, el * 2, uint16_t{}) : ld_in(gla, el * 4, uint32_t{});
        }
    } else if constexpr (HEADG) {
        const int rr = l < n ? l : n - 1;
        la_bits[0] = GBF ? (uint32_t)ld_in(gla, rr * 2, uint16_t{}) : ld_in(gla, rr * 4, uint32_t{});
    }
    const int tb = tid < n ? tid : n - 1;
    const uint32_t beta_bits = GBF ? (uint32_t)ld_in(gbeta, tb * 2, uint16_t{}) : ld_in(gbeta, tb * 4, uint32_t{});
    if constexpr (KDA) {
        // q and k rows come in as 16-byte pieces into the tiles they are
        // rescaled in; each thread (channel, sub-block) then reads its 16
        // tokens from LDS.  ln(alpha) is read per thread (one coalesced row
        // segment per wave and token).
#pragma unroll
        for (int i = 0; i < QPT; ++i) {
            const int idx = tid + NT * i;
            if (idx < C * PPR) {
                const int r0 = idx / PPR, cc = (idx % PPR) * VPIECE;
                const uint4 a = keep_or_zero(gqp[i], r0 < n);
                const uint4 b = keep_or_zero(gkp[i], r0 < n);
                *(uint4*)(sQr + r0 * PK + cc) = a;
                *(uint4*)(sKr + r0 * PK + cc) = b;
                if (norm_qk) {
                    // the PPR pieces of a row sit in PPR consecutive lanes
                    const float nq = inv_norm(group_sum<PPR>(sumsq16(a, E{})));
                    const float nk = inv_norm(group_sum<PPR>(sumsq16(b, E{})));
                    if (idx % PPR == 0) {
                        sQn[r0] = nq;
                        sKn[r0] = nk;
                    }
                }
            }
        }
        float a[16];
        float lsum = 0.f;
        if (kact) {
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                const int r = 16 * kR + s;
                float la = bits_f32(la_bits[s], GBF);
                if (gate_raw) la = log_alpha_of_raw(la);
                a[s] = r < n ? la : 0.f;
                lsum += a[s];
            }
        }
        // a wave holds 64 channels of one sub-block: flag it when some
        // channel's decay over the sub-block leaves the split's range
        {
            const bool unsafe = kact && lsum < Cfg::UNSAFE_LOG;
            const uint64_t m = __ballot(unsafe);
            if (l == 0) sFlag[w] = m != 0;
        }
        // the diagonal blocks of A (in sA) and of P (sPd) start at zero for
        // the direct sums; the MFMA path overwrites sA's blocks otherwise
        for (int i = tid; i < NB * 256; i += NT) {
            const int R = i >> 8, e = i & 255;
            sA[(16 * R + (e >> 4)) * PA + 16 * R + (e & 15)] = 0.f;
            pd_block(R)[(e >> 4) * pd_ld + (e & 15)] = 0.f;
        }
        __syncthreads();
        if (kact) {
            const int R = kR;
            float qv[16], kv[16];
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                qv[s] = to_f32(sQr[(16 * R + s) * PK + kc]);
                kv[s] = to_f32(sKr[(16 * R + s) * PK + kc]);
                if (norm_qk) {
                    qv[s] *= sQn[16 * R + s];
                    kv[s] *= sKn[16 * R + s];
                }
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
            bool flagged = false;
#pragma unroll
            for (int u = 0; u < DK / 64; ++u) flagged |= sFlag[R * (DK / 64) + u] != 0;
            // row factor: e^{g_s - G_{R+1}} = x_s / Z_R (<= 1e30), or for a
            // flagged sub-block x_s = e^{g_s - G_R} (<= 1)
            const float rz = flagged ? 1.f : 1.f / x[15];
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
#pragma unroll
        for (int i = 0; i < QPT; ++i) {
            const int idx = tid + NT * i;
            if (idx < C * PPR) {
                const int r0 = idx / PPR, cc = (idx % PPR) * VPIECE;
                const uint4 b = keep_or_zero(gkp[i], r0 < n);
                *(uint4*)(sKr + r0 * PK + cc) = b;
                if (norm_qk) {
                    // the PPR pieces of a row sit in PPR consecutive lanes
                    const float nk = inv_norm(group_sum<PPR>(sumsq16(b, E{})));
                    if (idx % PPR == 0) sKn[r0] = nk;
                }
            }
        }
        // g = inclusive prefix sum of ln(alpha) over the chunk (wave 0)
        if (w == 0) {
            float g = 0.f;
            if constexpr (HEADG) {
                float la = 0.f;
                if (l < n) {
                    la = bits_f32(la_bits[0], GBF);
                    if (gate_raw) la = log_alpha_of_raw(la);
                }
                g = wave_inclusive_sum(la);
            }
            if (l < C) {
                sG[l] = g;
                sEg[l] = exp_neg(g);
            }
        }
    }
    if (tid < C) {
        float b = 0.f;
        if (tid < n) {
            b = bits_f32(beta_bits, GBF);
            if (beta_logit) b = sigmoid(b);
        }
        sBeta[tid] = b;
    }
    // Every load of the chunk has landed before the first record store goes
    // out: loads and stores share one memory counter, so a later wait for a
    // load would also wait for every store issued before it.
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
    __syncthreads();

    // ================= G2 (KDA): cross-block factors, K^ ======================
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
            // K^ = k y F = k e^{g_n - g}, written as the A operand of the state
            // update (rows = key channel, k = token)
#pragma unroll
            for (int pc = 0; pc < 16 / W; ++pc) {
                const int j0 = 16 * R + W * pc;
                if constexpr (ESZ == 2) {
                    bf16x8 v;
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[e] = (bf16)(ky[W * pc + e] * Fr);
                    if constexpr (WIDE) {
                        const bf16x4 lo = {v[0], v[1], v[2], v[3]}, hi = {v[4], v[5], v[6], v[7]};
                        *(bf16x4*)(rKt + wide_elem(kc, j0, C)) = lo;
                        *(bf16x4*)(rKt + wide_elem(kc, j0 + 4, C)) = hi;
                    } else {
                        *(bf16x8*)(rKt + frag_elem<E>(kc, j0, C)) = v;
                    }
                } else {
                    floatx4 v;
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = ky[W * pc + e] * Fr;
                    *(floatx4*)(rKt + frag_elem<E>(kc, j0, C)) = v;
                }
            }
            // direct sums of the diagonal blocks of a flagged sub-block:
            // entry (r, j), j <= r, takes q_r k_j prod_{j<t<=r} alpha_t (and
            // k_r k_j ... for A, beta applied later) from every channel; the
            // wave's 64 channels are reduced and lane 0 adds them to LDS.
            // The thread's 16 tokens are read again from memory, so the
            // registers of the common path are not held for this rare one.
            bool flagged = false;
#pragma unroll
            for (int u = 0; u < DK / 64; ++u) flagged |= sFlag[R * (DK / 64) + u] != 0;
            if (flagged) {
                float qd[16], kd[16], ad[16];
#pragma unroll
                for (int s = 0; s < 16; ++s) {
                    const int r = 16 * R + s;
                    const int rr = r < n ? r : n - 1;
                    const uint32_t el = rr * DK + kc;
                    float qv = ESZ == 2 ? bits_f32(ldg<uint16_t>(gq, el * 2), true)
                                        : bits_f32(ldg<uint32_t>(gq, el * 4), false);
                    float kv = ESZ == 2 ? bits_f32(ldg<uint16_t>(gk, el * 2), true)
                                        : bits_f32(ldg<uint32_t>(gk, el * 4), false);
                    const uint32_t ea = rr * la_rs + kc * la_cs;
                    float la = bits_f32(GBF ? (uint32_t)ldg<uint16_t>(gla, ea * 2) : ldg<uint32_t>(gla, ea * 4), GBF);
                    if (norm_qk) {
                        qv *= sQn[r];
                        kv *= sKn[r];
                    }
                    if (gate_raw) la = log_alpha_of_raw(la);
                    qd[s] = r < n ? qv : 0.f;
                    kd[s] = r < n ? kv : 0.f;
                    ad[s] = exp_neg(r < n ? la : 0.f);
                }
                float* pdb = pd_block(R);
#pragma unroll
                for (int jj = 0; jj < 16; ++jj) {
                    float f = 1.f;
#pragma unroll
                    for (int rr = jj; rr < 16; ++rr) {
                        if (rr > jj) f *= ad[rr];
                        const float tk = group_sum<64>(kd[rr] * kd[jj] * f);
                        const float tq = group_sum<64>(qd[rr] * kd[jj] * f);
                        if (l == 0) {
                            atomicAdd(sA + (16 * R + rr) * PA + 16 * R + jj, tk);
                            atomicAdd(pdb + rr * pd_ld + jj, tq);
                        }
                    }
                }
            }
            if (R == 0) {
                // E_b turns sub-block b's row operand into k e^{g}: e^{G_{b+1}}
                // (e^{G_b} for a flagged sub-block); and e^{g_n}
                float run = 1.f;
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    bool fb = false;
#pragma unroll
                    for (int u = 0; u < DK / 64; ++u) fb |= sFlag[b * (DK / 64) + u] != 0;
                    if (fb) sE[b * DK + kc] = run;
                    run *= Zb[b];
                    if (!fb) sE[b * DK + kc] = run;
                }
                rGam[kc] = run;
            }
        }
        __syncthreads();
    }

    // ================= AP: A (fp32, LDS) and P (record) ======================
    for (int p = w; p < Cfg::NPAIR; p += NW) {
        int R, J;
        pair_of(p, R, J);
        constexpr int NKS = DK / KS;
        const E* pa = (KDA ? sKc : sKr) + (16 * J + lr) * PK + W * lq;
        const E* pk = sKr + (16 * R + lr) * PK + W * lq;
        const E* pq = sQr + (16 * R + lr) * PK + W * lq;
        // lane holds [m = j = 16J + 4lq + e][n = r = 16R + lr]
        const int rr = 16 * R + lr;
        floatx4 accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
        bool flagR = false;  // sub-block R takes the split at its start
        if constexpr (KDA) {
#pragma unroll
            for (int u = 0; u < DK / 64; ++u) flagR |= sFlag[R * (DK / 64) + u] != 0;
        }
        if (flagR && J == R) {
            // summed channel by channel in phase G (A without beta)
            accA = *(const floatx4*)(sA + rr * PA + 16 * J + 4 * lq);
            accP = *(const floatx4*)(pd_block(R) + lr * pd_ld + 4 * lq);
        } else {
            typename F::T fa[NKS], fk[NKS], fq[THIN ? 1 : NKS];
            if (!KDA || J == R) {
#pragma unroll
                for (int i = 0; i < NKS; ++i) fa[i] = F::load(pa + KS * i);
            } else {
                // pair scale per channel: prod_{J < m <= R} Z_m, or up to
                // m < R for a flagged sub-block R
                const int mend = flagR ? R : R + 1;
#pragma unroll
                for (int i = 0; i < NKS; ++i) {
                    const float* pz = sZ + KS * i + W * lq;
                    floatx4 y0 = {1.f, 1.f, 1.f, 1.f}, y1 = {1.f, 1.f, 1.f, 1.f};
                    for (int m = J + 1; m < mend; ++m) {
                        y0 *= *(const floatx4*)(pz + m * DK);
                        if constexpr (W == 8) y1 *= *(const floatx4*)(pz + m * DK + 4);
                    }
                    fa[i] = F::load_scaled_v(pa + KS * i, y0, y1);
                }
            }
#pragma unroll
            for (int i = 0; i < NKS; ++i) {
                fk[i] = F::load(pk + KS * i);
                if constexpr (!THIN) fq[i] = F::load(pq + KS * i);
            }
#pragma unroll
            for (int i = 0; i < NKS; ++i) {
                accA = F::mma(accA, fa[i], fk[i]);
                if constexpr (!THIN) accP = F::mma(accP, fa[i], fq[i]);
            }
        }
        const float br = sBeta[rr];
        float gr = 0.f;
        floatx4 gj = {0.f, 0.f, 0.f, 0.f};
        if constexpr (HEADG) {
            gr = sG[rr];
            gj = *(const floatx4*)(sG + 16 * J + 4 * lq);
        }
        floatx4 va, vp;
        // scalar decay: the raw k rows, so the norms scale the product
        const float nr = THIN && norm_qk ? sKn[rr] : 1.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int jj = 16 * J + 4 * lq + e;
            float f = 1.f;  // scalar decay e^{g_r - g_j}, applied to the result
            if constexpr (HEADG) f = exp_neg(gr - gj[e]);
            if (THIN && norm_qk) f *= nr * sKn[jj];
            va[e] = (J < R || jj < rr) ? br * accA[e] * f : 0.f;
            vp[e] = (J < R || jj <= rr) ? accP[e] * f : 0.f;
        }
        *(floatx4*)(sA + rr * PA + 16 * J + 4 * lq) = va;
        if constexpr (!THIN) {
            if constexpr (WIDE) st4<E>(rP + wide_elem(rr, 16 * J + 4 * lq, C), vp);
            else st4<E>(rP + frag_elem<E>(rr, 16 * J + 4 * lq, C), vp);
        }
    }
    // blocks above the diagonal of P are zero
    if constexpr (!THIN) {
        for (int b = w; b < NB * NB; b += NW) {
            const int R = b / NB, J = b % NB;
            if (J > R) {
                const floatx4 z = {0.f, 0.f, 0.f, 0.f};
                if constexpr (WIDE) st4<E>(rP + wide_elem(16 * R + lr, 16 * J + 4 * lq, C), z);
                else st4<E>(rP + frag_elem<E>(16 * R + lr, 16 * J + 4 * lq, C), z);
            }
        }
    }
    __syncthreads();
    if constexpr (THIN) {
        // the K tile is done: its space takes T diag(beta), whose blocks above
        // the diagonal (written by nobody else) are zero (16-byte pieces,
        // which never straddle a 16-column block)
        constexpr int ZPR = C / VPIECE;
        constexpr int NZ = (C * ZPR + NT - 1) / NT;
#pragma unroll
        for (int it = 0; it < NZ; ++it) {
            const int i = tid + NT * it;
            if (i < C * ZPR) {
                const int r = i / ZPR, j = (i % ZPR) * VPIECE;
                if ((j >> 4) > (r >> 4)) *(uint4*)(sTb + r * PC + j) = make_uint4(0u, 0u, 0u, 0u);
            }
        }
    }

    // ================= T1: diagonal blocks by forward substitution ===========
    // Wave R < NB solves block R.  Lane (j, s) = (l/4, l%4) owns rows
    // 4s..4s+3 of column j of T_RR, with those rows of A_RR in registers.
    // Right-looking sweep: once t_m is final, its owner lane hands it to the
    // other three lanes of the quad (DPP broadcast) and every row takes its
    // A_RR[i][m] t_m term; the dependent chain is 15 steps long.  (A_RR[i][m]
    // is zero for m >= i, so no row needs masking.)  Results: T_RR^T (fp32) in
    // the diagonal block of sA, T_RR diag(beta) in operand precision in sTb.
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
        for (int ii = 0; ii < 4; ++ii) sTb[(16 * R + 4 * s4 + ii) * PC + 16 * R + j] = from_f32<E>(acc[ii] * bj);
    } else if constexpr (KDA) {
        // the other waves: zero the blocks of T diag(beta) above the diagonal
        // (its tile reuses the column operand's space), K~ = k e^{g} in place
        // (row operand x E_R) for W, and Q~ = q e^{g} straight to the record
        // (A operand of Q~ S)
        // (both loops have trip counts known here, so they are unrolled and
        // each thread's LDS reads go out together; the zeros go out as
        // 16-byte pieces, which never straddle a 16-column block)
        constexpr int NTO = NT - 64 * NB;               // threads of these waves
        constexpr int ZPR = C / VPIECE;                 // 16-byte pieces per row
        constexpr int NZ = (C * ZPR + NTO - 1) / NTO;
#pragma unroll
        for (int it = 0; it < NZ; ++it) {
            const int i = (tid - 64 * NB) + NTO * it;
            if (i < C * ZPR) {
                const int r = i / ZPR, j = (i % ZPR) * VPIECE;
                if ((j >> 4) > (r >> 4)) *(uint4*)(sTb + r * PC + j) = make_uint4(0u, 0u, 0u, 0u);
            }
        }
        constexpr int PER_ROW = DK / VPIECE;
        constexpr int NS = (2 * C * PER_ROW + NTO - 1) / NTO;
#pragma unroll
        for (int it = 0; it < NS; ++it) {
            const int i = (tid - 64 * NB) + NTO * it;
            if (i < 2 * C * PER_ROW) {
                const int which = i / (C * PER_ROW);
                const int rem = i % (C * PER_ROW);
                const int r = rem / PER_ROW, cc = (rem % PER_ROW) * VPIECE;
                const float* sc = sE + (r >> 4) * DK + cc;
                if (which == 0) {
                    E* p = sKr + r * PK + cc;
                    *(typename F::T*)p = F::load_scaled(p, sc);
                } else {
                    const E* p = sQr + r * PK + cc;
                    const typename F::T qs = F::load_scaled(p, sc);
                    if constexpr (WIDE) {
                        const bf16x4 lo = {qs[0], qs[1], qs[2], qs[3]}, hi = {qs[4], qs[5], qs[6], qs[7]};
                        *(bf16x4*)(rQt + wide_elem(r, cc, DK)) = lo;
                        *(bf16x4*)(rQt + wide_elem(r, cc + 4, DK)) = hi;
                    } else {
                        *(typename F::T*)(rQt + frag_elem<E>(r, cc, DK)) = qs;
                    }
                }
            }
        }
    }
    __syncthreads();

    // ================= T2: off-diagonal blocks, by distance ==================
    // T_RJ = -T_RR sum_{M=J}^{R-1} A_RM T_MJ; T_RJ^T is stored at block (J, R)
    // of sA, and T_RJ diag(beta) in sTb.  KDA: V enters LDS during the first
    // level.
#pragma unroll
    for (int d = 1; d < NB; ++d) {
        if (!THIN && d == 1) {
#pragma unroll
            for (int i = 0; i < VPT; ++i) {
                const int idx = tid + NT * i;
                if (idx < C * VPPR) {
                    const int r = idx / VPPR, cc = (idx % VPPR) * VPIECE;
                    *(uint4*)(sV + r * PVV + cc) = keep_or_zero(rv[i], r < n);
                }
            }
        }
        const int R = d + w, J = w;
        if (R < NB) {
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int M = J; M < R; ++M) {
                floatx4 af = *(const floatx4*)(sA + (16 * R + lr) * PA + 16 * M + 4 * lq);
                floatx4 bfv = *(const floatx4*)(sA + (16 * J + lr) * PA + 16 * M + 4 * lq);
                acc = Frag<float>::mma(acc, af, bfv);
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
            for (int e = 0; e < 4; ++e) sTb[(16 * R + 4 * lq + e) * PC + 16 * J + lr] = from_f32<E>(res[e] * bj);
        }
        __syncthreads();
    }

    // T^T for the chunkwise gradients: sA holds it on and above the diagonal
    // blocks (below them it still holds A)
    if constexpr (!THIN) {
        if (prm.tt) {
            float* dst = prm.tt + ((int64_t)bh * prm.ncs + cs) * C * C;
            for (int i = tid; i < C * C; i += NT) {
                const int r = i / C, j = i - r * C;
                dst[i] = (r >> 4) <= (j >> 4) ? sA[r * PA + j] : 0.f;
            }
        }
    }

    // ================= WU: W = T' K~ and U = T diag(beta) V ==================
    // Scalar decay: T diag(beta) goes out as it is.
    if constexpr (THIN) {
        constexpr int PPR = C * ESZ / 16;
        for (int i = tid; i < C * PPR; i += NT) {
            const int r = i / PPR, cc = (i % PPR) * (16 / ESZ);
            *(uint4*)(rTb + r * C + cc) = *(const uint4*)(sTb + r * PC + cc);
        }
        // the decay scalars g, e^g, e^{g_n - g}; raw k: 1/|k_t| for the
        // state pass (zero past the sequence end)
        if (tid < C) {
            const float g = sG[tid];
            rRs[tid] = g;
            rRs[C + tid] = sEg[tid];
            rRs[2 * C + tid] = exp_neg(sG[C - 1] - g);
            if (norm_qk) rRs[3 * C + tid] = tid < n ? sKn[tid] : 0.f;
        }
        return;
    }
    // KDA: W tile (R, cb) is computed transposed so each lane holds four
    // adjacent channels of one row; U tile (R, vb) lands directly in
    // accumulator order.
    const E* sTw = sTb;
    // every wave has the same number of tiles (a static trip count, so the
    // next tile's operand loads can go out before this tile's stores)
    static_assert((NB * (NCB + NVB)) % NW == 0, "W and U tiles per wave");
#pragma unroll 2
    for (int m = 0; m < NB * (NCB + NVB) / NW; ++m) {
        const int it = w + NW * m;
        if (it < NB * NCB) {
            const int R = it % NB, cb = it / NB;
            const int K = ((16 * (R + 1) + KS - 1) / KS) * KS;
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = mma_block_at<E>(acc, sKr, PK, 16 * cb, sTw + (16 * R) * PC, PC, K);
            if constexpr (WIDE) st4<E>(rW + wide_elem(16 * R + lr, 16 * cb + 4 * lq, DK), -acc);
            else st4<E>(rW + frag_elem<E>(16 * R + lr, 16 * cb + 4 * lq, DK), acc);
        } else {
            const int u = it - NB * NCB;
            const int R = u % NB, vb = u / NB;
            const int K = ((16 * (R + 1) + KS - 1) / KS) * KS;
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = mma_block_bt<E>(acc, sTb + (16 * R) * PC, PC, sV, PVV, 16 * vb, K);
            constexpr int PF = 16 / (4 * ESZ);  // column blocks per 16-byte lane piece
            st4<E>(rU + ((R * (NVB / PF) + vb / PF) * 64 + l) * 4 * PF + (vb % PF) * 4, acc);
        }
    }
    if constexpr (REV) {
        // the chunk's reverse record, from the record this workgroup has just
        // written (the barrier's workgroup-scope fence makes the workgroup's
        // global stores visible to all its threads)
        static_assert(WIDE && RevCfg<DK, DV>::NT == NT && RevCfg<DK, DV>::LDS_BYTES <= Cfg::LDS_BYTES,
                      "the reverse record fits this workgroup");
        __syncthreads();
        build_rev_record<DK, DV>(prm.ws, prm.rrecs, prm.dout, L, prm.ncs, bh, cs, smem);
    }
}

// ---- host-side dispatch -----------------------------------------------------

template <int DK, int DV, int C, typename E, int AMODE>
static hipError_t launch_intra_cfg(const IntraParams& prm, hipStream_t stream) {
    typedef IntraCfg<DK, DV, C, E, AMODE> Cfg;
    const int64_t grid = (int64_t)prm.BH * prm.ncs;
    // the wide record order exists for per-channel decay with bf16 operands
    constexpr bool CAN_WIDE = Cfg::KDA && sizeof(E) == 2;
    if (prm.wide && !CAN_WIDE) return hipErrorInvalidValue;
    if constexpr (CAN_WIDE) {
        if (prm.wide && prm.rrecs) {
            if (prm.c0 != 0 || !prm.dout || prm.cu) return hipErrorInvalidValue;
            if (prm.gate_bf16)
                hipLaunchKernelGGL((kda_intra_kernel<Cfg, true, true, true>), dim3((unsigned)grid),
                                   dim3(Cfg::NT), 0, stream, prm);
            else
                hipLaunchKernelGGL((kda_intra_kernel<Cfg, false, true, true>), dim3((unsigned)grid),
                                   dim3(Cfg::NT), 0, stream, prm);
            return hipGetLastError();
        }
        if (prm.wide) {
            if (prm.gate_bf16)
                hipLaunchKernelGGL((kda_intra_kernel<Cfg, true, true>), dim3((unsigned)grid),
                                   dim3(Cfg::NT), 0, stream, prm);
            else
                hipLaunchKernelGGL((kda_intra_kernel<Cfg, false, true>), dim3((unsigned)grid),
                                   dim3(Cfg::NT), 0, stream, prm);
            return hipGetLastError();
        }
    }
    if (prm.gate_bf16)
        hipLaunchKernelGGL((kda_intra_kernel<Cfg, true, false>), dim3((unsigned)grid), dim3(Cfg::NT), 0,
                           stream, prm);
    else
        hipLaunchKernelGGL((kda_intra_kernel<Cfg, false, false>), dim3((unsigned)grid), dim3(Cfg::NT), 0,
                           stream, prm);
    return hipGetLastError();
}

template <int DK, int DV, int C, typename E>
static hipError_t launch_intra_mode(const IntraParams& prm, int alpha_mode, hipStream_t stream) {
    switch (alpha_mode) {
        case KDA_ALPHA_NONE: return launch_intra_cfg<DK, DV, C, E, KDA_ALPHA_NONE>(prm, stream);
        case KDA_ALPHA_HEAD: return launch_intra_cfg<DK, DV, C, E, KDA_ALPHA_HEAD>(prm, stream);
        case KDA_ALPHA_CHANNEL: return launch_intra_cfg<DK, DV, C, E, KDA_ALPHA_CHANNEL>(prm, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_intra(const IntraParams& prm, int dk, int dv, int qkv_bf16, int alpha_mode,
                        hipStream_t stream) {
    if (prm.BH == 0 || prm.ncs == 0) return hipSuccess;
#define KDA_CASE(DK_, DV_)                                                          \
    if (dk == DK_ && dv == DV_)                                                     \
        return qkv_bf16 ? launch_intra_mode<DK_, DV_, 64, bf16>(prm, alpha_mode, stream) \
                        : launch_intra_mode<DK_, DV_, 32, float>(prm, alpha_mode, stream);
    KDA_CASE(128, 128)
    KDA_CASE(128, 64)
    KDA_CASE(64, 128)
    KDA_CASE(64, 64)
#undef KDA_CASE
    return hipErrorInvalidValue;
}

}  // namespace kda
