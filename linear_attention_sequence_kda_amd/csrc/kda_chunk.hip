// kda_chunk.hip -- fused chunkwise-parallel prefill of the KDA / gated delta rule
// for gfx950 (MI355X).
//
// Math: "22,580: From GPT-2 to Kimi K3" (yichencityu.github.io) section 6.3 gives
// the alpha = 1 chunk form; the gated, per-channel form below follows from
// unrolling the recurrence inside a chunk (the pages stop before printing it,
// sections 08 and 9.1).  For a chunk of C
// tokens entering with state S, with g_r = sum_{s<=r} ln(alpha_s) per key
// channel (inclusive, chunk-relative):
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
// One workgroup (4 waves) owns one (b, h) head and one slice of NV state
// columns; columns of S evolve independently, so slices never talk.  It walks
// the chunks in order with its fp32 state slice resident in registers.  Per
// chunk:
//   G  load q, k, ln(alpha), beta, v; per-channel decay factors in 16-token
//      sub-blocks; scaled K/Q tiles into LDS
//   AP A and P, 16x16 blocks, MFMA (k = key channels)
//   T  diagonal 16x16 blocks of T by forward substitution (one lane per column),
//      off-diagonal blocks by the block formula T_RJ = -T_RR sum_M A_RM T_MJ on
//      fp32 MFMA; T' = T diag(beta) rounded to the operand type
//   S  X = V - K~ S;  u = T' X;  o = Q~ S + P u;  S = e^{g_n} S + K^^T u
//
// Decay inside A and P, e^{g_r - g_j}, is split at the end of r's 16-token
// sub-block R (cumulative G_{R+1}): the row operand carries e^{g_r - G_{R+1}}
// (>= 1, at most e^{16 |ln alpha|}), the column operand e^{G_{J+1} - g_j} (<= 1)
// and, for J < R, a per-channel pair scale e^{G_{R+1} - G_{J+1}} (<= 1).  A
// diagonal pair therefore uses both stored operands unscaled (one bf16 rounding
// each).  The bound on the row factor is why the GPU path asks for
// ln(alpha) >= -5 per token and channel.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

template <int DK_, int NV_, int C_, typename E_>
struct ChunkCfg {
    typedef E_ E;
    static constexpr int DK = DK_, NV = NV_, C = C_;
    static constexpr int NB = C / 16;                  // 16-token sub-blocks per chunk
    static constexpr int NPAIR = NB * (NB + 1) / 2;    // (R, J <= R) block pairs
    static constexpr int ESZ = sizeof(E);
    static constexpr int PADE = 16 / ESZ;              // 16 bytes of padding per row
    static constexpr int PK = DK + PADE;               // pitch of [*][DK] tiles
    static constexpr int PC = C + PADE;                // pitch of [*][C] tiles
    static constexpr int PV = NV + PADE;               // pitch of [C][NV] tiles
    static constexpr int PA = C + 4;                   // pitch of the fp32 A/T tile
    static constexpr int NCB = DK / 16, NVB = NV / 16; // 16x16 blocks of the state slice
    static constexpr int NTHREADS = 256;

    // LDS byte offsets
    static constexpr int O_KR = 0;
    static constexpr int O_QR = O_KR + C * PK * ESZ;
    static constexpr int O_KC = O_QR + C * PK * ESZ;
    static constexpr int O_KHT = O_KC + C * PK * ESZ;
    static constexpr int O_TB = O_KHT + DK * PC * ESZ;
    static constexpr int O_P = O_TB + C * PC * ESZ;
    static constexpr int O_V = O_P + C * PC * ESZ;
    static constexpr int O_ST0 = O_V + C * PV * ESZ;
    static constexpr int O_ST1 = O_ST0 + NV * PK * ESZ;
    static constexpr int SZ_XT = (NV * PC > C * PV ? NV * PC : C * PV) * ESZ;  // X^T, then o
    static constexpr int O_XT = O_ST1 + NV * PK * ESZ;
    static constexpr int O_UT = O_XT + SZ_XT;
    static constexpr int O_A = O_UT + NV * PC * ESZ;
    static constexpr int O_Z = O_A + C * PA * 4;
    static constexpr int O_E = O_Z + NB * DK * 4;
    static constexpr int O_Y = O_E + NB * DK * 4;
    static constexpr int O_GN = O_Y + NPAIR * DK * 4;
    static constexpr int O_BETA = O_GN + DK * 4;
    static constexpr int LDS_BYTES = O_BETA + C * 4;

    static_assert(DK % 32 == 0 && NV % 16 == 0 && (C == 32 || C == 64), "tile shape");
    static_assert((NCB * NVB) % 4 == 0, "state blocks split evenly over 4 waves");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget of one gfx950 CU");
};

// ---- global loads of two adjacent elements ---------------------------------
__device__ __forceinline__ floatx2 ld2(const bf16* p) {
    bf16x2 v = *(const bf16x2*)p;
    floatx2 r;
    r[0] = (float)v[0];
    r[1] = (float)v[1];
    return r;
}
__device__ __forceinline__ floatx2 ld2(const float* p) { return *(const floatx2*)p; }

__device__ __forceinline__ float ld_gate(const void* p, int64_t i, bool bf) {
    return bf ? (float)((const bf16*)p)[i] : ((const float*)p)[i];
}
__device__ __forceinline__ floatx2 ld_gate2(const void* p, int64_t i, bool bf) {
    return bf ? ld2((const bf16*)p + i) : ld2((const float*)p + i);
}

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

__device__ __forceinline__ void pair_of(int p, int& R, int& J) {
    R = 0;
    while (p >= R + 1) {
        p -= R + 1;
        ++R;
    }
    J = p;
}

template <class Cfg>
__global__ void __launch_bounds__(256)
kda_chunk_kernel(ChunkParams prm) {
    typedef typename Cfg::E E;
    typedef Frag<E> F;
    constexpr int DK = Cfg::DK, NV = Cfg::NV, C = Cfg::C, NB = Cfg::NB;
    constexpr int PK = Cfg::PK, PC = Cfg::PC, PV = Cfg::PV, PA = Cfg::PA;
    constexpr int NCB = Cfg::NCB, NVB = Cfg::NVB;
    constexpr int SB_PER_WAVE = NCB * NVB / 4;

    __shared__ __attribute__((aligned(16))) char smem[Cfg::LDS_BYTES];
    E* sKr = (E*)(smem + Cfg::O_KR);
    E* sQr = (E*)(smem + Cfg::O_QR);
    E* sKc = (E*)(smem + Cfg::O_KC);
    E* sKhT = (E*)(smem + Cfg::O_KHT);
    E* sTb = (E*)(smem + Cfg::O_TB);
    E* sP = (E*)(smem + Cfg::O_P);
    E* sV = (E*)(smem + Cfg::O_V);
    E* sST0 = (E*)(smem + Cfg::O_ST0);
    E* sST1 = (E*)(smem + Cfg::O_ST1);
    E* sXT = (E*)(smem + Cfg::O_XT);
    E* sO = (E*)(smem + Cfg::O_XT);  // o tile reuses the X^T area after u is formed
    E* sUT = (E*)(smem + Cfg::O_UT);
    float* sA = (float*)(smem + Cfg::O_A);
    float* sZ = (float*)(smem + Cfg::O_Z);
    float* sE = (float*)(smem + Cfg::O_E);
    float* sY = (float*)(smem + Cfg::O_Y);
    float* sGn = (float*)(smem + Cfg::O_GN);
    float* sBeta = (float*)(smem + Cfg::O_BETA);

    const int tid = threadIdx.x;
    const int w = tid >> 6;
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
    const bool gbf = prm.gate_bf16 != 0;
    const int amode = prm.alpha_mode;

    const E* gq = (const E*)prm.q + (int64_t)bh * L * DK;
    const E* gk = (const E*)prm.k + (int64_t)bh * L * DK;
    const E* gv = (const E*)prm.v + (int64_t)bh * L * DV;
    E* go = (E*)prm.o + (int64_t)bh * L * DV;
    const int64_t gate_head = (int64_t)bh * L;  // token index base for beta / head-mode gate

    // ---- zero the triangular operand tiles once (upper blocks stay zero) ---
    for (int i = tid; i < C * PC; i += Cfg::NTHREADS) {
        sTb[i] = from_f32<E>(0.f);
        sP[i] = from_f32<E>(0.f);
    }

    // ---- initial state slice into registers, and its operand copy ----------
    floatx4 Sreg[SB_PER_WAVE];
#pragma unroll
    for (int i = 0; i < SB_PER_WAVE; ++i) {
        const int item = w + 4 * i;
        const int cb = item % NCB, vb = item / NCB;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = 16 * cb + 4 * lq + e;
            Sreg[i][e] = prm.S0 ? prm.S0[((int64_t)bh * DK + row) * DV + v0 + 16 * vb + lr] : 0.f;
        }
        store_acc_transposed<E>(sST0 + (16 * vb) * PK + 16 * cb, PK, Sreg[i]);
    }

    const int64_t nchunks = (L + C - 1) / C;
    for (int64_t ch = 0; ch < nchunks; ++ch) {
        const int64_t t0 = ch * C;
        const int n = (int)((L - t0) < C ? (L - t0) : C);  // valid tokens in this chunk
        E* sSTc = (ch & 1) ? sST1 : sST0;
        E* sSTn = (ch & 1) ? sST0 : sST1;

        // ================= G1: loads, in-block decay products ================
        constexpr int NCP = DK / 2;            // channel pairs
        constexpr int NBG = 256 / NCP;         // block groups
        const int cp = tid % NCP, bg = tid / NCP;
        const int c0 = 2 * cp;
        floatx2 ky[16];  // k * y for the K^ tile, kept across the barrier
        int myR = (bg < NB) ? bg : -1;
        static_assert(NBG >= 1, "");
        if (myR >= 0) {
            const int R = myR;
            floatx2 a[16], qv[16], kv[16];
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                const int r = 16 * R + s;
                const bool valid = r < n;
                const int64_t tok = t0 + r;
                floatx2 z2 = {0.f, 0.f};
                qv[s] = valid ? ld2(gq + tok * DK + c0) : z2;
                kv[s] = valid ? ld2(gk + tok * DK + c0) : z2;
                if (amode == KDA_ALPHA_CHANNEL) {
                    a[s] = valid ? ld_gate2(prm.log_alpha, (gate_head + tok) * DK + c0, gbf) : z2;
                } else if (amode == KDA_ALPHA_HEAD) {
                    float x = valid ? ld_gate(prm.log_alpha, gate_head + tok, gbf) : 0.f;
                    a[s][0] = x;
                    a[s][1] = x;
                } else {
                    a[s] = z2;
                }
            }
            // alpha = exp(ln alpha); x_s = prod_{s'<=s} alpha (within block)
            floatx2 x[16];
            floatx2 run = {1.f, 1.f};
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                if (amode != KDA_ALPHA_NONE) {
                    a[s][0] = exp_neg(a[s][0]);
                    a[s][1] = exp_neg(a[s][1]);
                } else {
                    a[s][0] = 1.f;
                    a[s][1] = 1.f;
                }
                run = run * a[s];
                x[s] = run;
            }
            // y_s = prod_{s' > s} alpha = e^{G_{R+1} - g_s} (within block, <= 1)
            floatx2 yrun = {1.f, 1.f};
#pragma unroll
            for (int s = 15; s >= 0; --s) {
                ky[s] = kv[s] * yrun;
                yrun = yrun * a[s];
            }
            // x'_s = x_s / Z_R = e^{g_s - G_{R+1}} (>= 1): rows are referenced to
            // the end of their block, so a diagonal block pair needs no rescale
            floatx2 rz;
            rz[0] = 1.f / x[15][0];
            rz[1] = 1.f / x[15][1];
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                const int r = 16 * R + s;
                const floatx2 xp = x[s] * rz;
                st2<E>(sKr + r * PK + c0, kv[s][0] * xp[0], kv[s][1] * xp[1]);
                st2<E>(sQr + r * PK + c0, qv[s][0] * xp[0], qv[s][1] * xp[1]);
                st2<E>(sKc + r * PK + c0, ky[s][0], ky[s][1]);
            }
            sZ[R * DK + c0] = x[15][0];
            sZ[R * DK + c0 + 1] = x[15][1];
        }
        if (tid < C) {
            const int r = tid;
            sBeta[r] = (r < n) ? ld_gate(prm.beta, gate_head + t0 + r, gbf) : 0.f;
        }
        {
            // v slice [C][NV] -> sV, 16-byte pieces
            constexpr int PIECE = 16 / Cfg::ESZ;           // elements per piece
            constexpr int PPR = NV / PIECE;                // pieces per row
            for (int i = tid; i < C * PPR; i += Cfg::NTHREADS) {
                const int r = i / PPR, cc = (i % PPR) * PIECE;
                uint4 val = {0u, 0u, 0u, 0u};
                if (r < n) val = *(const uint4*)(gv + (t0 + r) * DV + v0 + cc);
                *(uint4*)(sV + r * PV + cc) = val;
            }
        }
        __syncthreads();

        // ================= G2: cross-block decay factors, K^ tile ============
        if (myR >= 0) {
            const int R = myR;
            floatx2 Zb[NB];
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                Zb[b][0] = sZ[b * DK + c0];
                Zb[b][1] = sZ[b * DK + c0 + 1];
            }
            floatx2 Fr = {1.f, 1.f};  // e^{g_n - G_{R+1}} = prod of later blocks
#pragma unroll
            for (int b = 0; b < NB; ++b)
                if (b > R) Fr = Fr * Zb[b];
            // K^ = k y F, transposed: [channel][token]
#pragma unroll
            for (int s = 0; s < 16; s += Frag<E>::W) {
#pragma unroll
                for (int ch2 = 0; ch2 < 2; ++ch2) {
                    E* dst = sKhT + (c0 + ch2) * PC + 16 * R + s;
                    if constexpr (sizeof(E) == 2) {
                        bf16x8 vv;
#pragma unroll
                        for (int e = 0; e < 8; ++e) vv[e] = (bf16)(ky[s + e][ch2] * Fr[ch2]);
                        *(bf16x8*)dst = vv;
                    } else {
                        floatx4 vv;
#pragma unroll
                        for (int e = 0; e < 4; ++e) vv[e] = ky[s + e][ch2] * Fr[ch2];
                        *(floatx4*)dst = vv;
                    }
                }
            }
            if (R == 0) {
                // block-end factors E'_R = e^{G_{R+1}}, pair scales
                // Y'_RJ = e^{G_{R+1} - G_{J+1}} (1 on the diagonal), e^{g_n}
                floatx2 run = {1.f, 1.f};
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    run = run * Zb[b];
                    sE[b * DK + c0] = run[0];
                    sE[b * DK + c0 + 1] = run[1];
                }
                sGn[c0] = run[0];
                sGn[c0 + 1] = run[1];
                int p = 0;
#pragma unroll
                for (int rb = 0; rb < NB; ++rb) {
#pragma unroll
                    for (int jb = 0; jb <= rb; ++jb, ++p) {
                        floatx2 y = {1.f, 1.f};
#pragma unroll
                        for (int m = 0; m < NB; ++m)
                            if (m > jb && m <= rb) y = y * Zb[m];
                        sY[p * DK + c0] = y[0];
                        sY[p * DK + c0 + 1] = y[1];
                    }
                }
            }
        }
        __syncthreads();

        // ================= AP: A (fp32) and P (operand type) =================
        for (int p = w; p < Cfg::NPAIR; p += 4) {
            int R, J;
            pair_of(p, R, J);
            floatx4 accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
            const E* pa = sKc + (16 * J + lr) * PK + F::W * lq;
            const float* ps = sY + p * DK + F::W * lq;
            const E* pk = sKr + (16 * R + lr) * PK + F::W * lq;
            const E* pq = sQr + (16 * R + lr) * PK + F::W * lq;
            if (J == R) {
#pragma unroll
                for (int kk = 0; kk < DK; kk += F::KS) {
                    typename F::T af = F::load(pa + kk);
                    accA = F::mma(accA, af, F::load(pk + kk));
                    accP = F::mma(accP, af, F::load(pq + kk));
                }
            } else {
#pragma unroll
                for (int kk = 0; kk < DK; kk += F::KS) {
                    typename F::T af = F::load_scaled(pa + kk, ps + kk);
                    accA = F::mma(accA, af, F::load(pk + kk));
                    accP = F::mma(accP, af, F::load(pq + kk));
                }
            }
            // lane holds [m = j = 16J + 4lq + e][n = r = 16R + lr]
            const int rr = 16 * R + lr;
            const float br = sBeta[rr];
            floatx4 va, vp;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int jj = 16 * J + 4 * lq + e;
                va[e] = (J < R || jj < rr) ? br * accA[e] : 0.f;
                vp[e] = (J < R || jj <= rr) ? accP[e] : 0.f;
            }
            *(floatx4*)(sA + rr * PA + 16 * J + 4 * lq) = va;
            E* dp = sP + rr * PC + 16 * J + 4 * lq;
            if constexpr (sizeof(E) == 2) {
                bf16x4 t;
                t[0] = (bf16)vp[0];
                t[1] = (bf16)vp[1];
                t[2] = (bf16)vp[2];
                t[3] = (bf16)vp[3];
                *(bf16x4*)dp = t;
            } else {
                *(floatx4*)dp = vp;
            }
        }
        __syncthreads();

        // ================= T1: diagonal blocks by forward substitution =======
        // Lane (R, j) owns column j of T_RR and solves
        //   t_i = [i == j] - sum_{m < i} A_RR[i][m] t_m,  i = 0..15.
        // The result is stored transposed in the diagonal block of sA.
        if (w == 0 && l < 16 * NB) {
            const int R = l >> 4, j = l & 15;
            const float* Ab = sA + (16 * R) * PA + 16 * R;
            float t[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float s = (i == j) ? 1.f : 0.f;
#pragma unroll
                for (int m = 0; m < i; ++m) s -= Ab[i * PA + m] * t[m];
                t[i] = s;
            }
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            float* dst = sA + (16 * R + j) * PA + 16 * R;
#pragma unroll
            for (int i = 0; i < 16; i += 4) {
                floatx4 v4 = {t[i], t[i + 1], t[i + 2], t[i + 3]};
                *(floatx4*)(dst + i) = v4;
            }
        }
        __syncthreads();

        // ================= T2: off-diagonal blocks, by distance ===============
        // T_RJ = -T_RR sum_{M=J}^{R-1} A_RM T_MJ; T_RJ^T is stored at block (J, R).
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
                floatx4 res = Frag<float>::mma(z, tf, acc);
                *(floatx4*)(sA + (16 * J + lr) * PA + 16 * R + 4 * lq) = -res;
            }
            __syncthreads();
        }

        // ================= T': T diag(beta) in operand precision =============
        {
            constexpr int NG = 256 / C;
            const int r = tid % C, grp = tid / C;
            const int Rr = r >> 4;
            for (int jc = grp; jc < C / 4; jc += NG) {
                const int j = 4 * jc;
                if ((j >> 4) > Rr) continue;
                float tv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) tv[e] = sA[(j + e) * PA + r] * sBeta[j + e];
                E* dst = sTb + r * PC + j;
                if constexpr (sizeof(E) == 2) {
                    bf16x4 t4;
                    t4[0] = (bf16)tv[0];
                    t4[1] = (bf16)tv[1];
                    t4[2] = (bf16)tv[2];
                    t4[3] = (bf16)tv[3];
                    *(bf16x4*)dst = t4;
                } else {
                    floatx4 t4 = {tv[0], tv[1], tv[2], tv[3]};
                    *(floatx4*)dst = t4;
                }
            }
        }
        __syncthreads();

        // ================= S1: X = V - (K e^g) S ==============================
        for (int item = w; item < NB * NVB; item += 4) {
            const int R = item % NB, vb = item / NB;
            floatx4 acc;
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] = to_f32(sV[(16 * R + 4 * lq + e) * PV + 16 * vb + lr]);
            acc = mma_block_scaled_a<E, true>(acc, sKr + (16 * R) * PK, PK, sE + R * DK,
                                              sSTc + (16 * vb) * PK, PK, DK);
            store_acc_transposed<E>(sXT + (16 * vb) * PC + 16 * R, PC, acc);
        }
        __syncthreads();

        // ================= S2: u = T' X =======================================
        for (int item = w; item < NB * NVB; item += 4) {
            const int R = item % NB, vb = item / NB;
            constexpr int KS = Frag<E>::KS;
            const int K = ((16 * (R + 1) + KS - 1) / KS) * KS;
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = mma_block<E>(acc, sTb + (16 * R) * PC, PC, sXT + (16 * vb) * PC, PC, K);
            store_acc_transposed<E>(sUT + (16 * vb) * PC + 16 * R, PC, acc);
        }
        __syncthreads();

        // ================= S3: o = (Q e^g) S + P u ============================
        for (int item = w; item < NB * NVB; item += 4) {
            const int R = item % NB, vb = item / NB;
            constexpr int KS = Frag<E>::KS;
            const int K = ((16 * (R + 1) + KS - 1) / KS) * KS;
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = mma_block_scaled_a<E, false>(acc, sQr + (16 * R) * PK, PK, sE + R * DK,
                                               sSTc + (16 * vb) * PK, PK, DK);
            acc = mma_block<E>(acc, sP + (16 * R) * PC, PC, sUT + (16 * vb) * PC, PC, K);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                sO[(16 * R + 4 * lq + e) * PV + 16 * vb + lr] = from_f32<E>(acc[e]);
        }

        // ================= S4: S = e^{g_n} S + K^^T u =========================
#pragma unroll
        for (int i = 0; i < SB_PER_WAVE; ++i) {
            const int item = w + 4 * i;
            const int cb = item % NCB, vb = item / NCB;
            floatx4 acc = Sreg[i];
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] *= sGn[16 * cb + 4 * lq + e];
            acc = mma_block<E>(acc, sKhT + (16 * cb) * PC, PC, sUT + (16 * vb) * PC, PC, C);
            Sreg[i] = acc;
            store_acc_transposed<E>(sSTn + (16 * vb) * PK + 16 * cb, PK, acc);
        }
        __syncthreads();

        // ================= o tile -> HBM (valid rows only) ====================
        {
            constexpr int PIECE = 16 / Cfg::ESZ;
            constexpr int PPR = NV / PIECE;
            for (int i = tid; i < C * PPR; i += Cfg::NTHREADS) {
                const int r = i / PPR, cc = (i % PPR) * PIECE;
                if (r < n) *(uint4*)(go + (t0 + r) * DV + v0 + cc) = *(const uint4*)(sO + r * PV + cc);
            }
        }
    }

    // ---- final state --------------------------------------------------------
    if (prm.S_final) {
#pragma unroll
        for (int i = 0; i < SB_PER_WAVE; ++i) {
            const int item = w + 4 * i;
            const int cb = item % NCB, vb = item / NCB;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = 16 * cb + 4 * lq + e;
                prm.S_final[((int64_t)bh * DK + row) * DV + v0 + 16 * vb + lr] = Sreg[i][e];
            }
        }
    }
}

// ---- host-side dispatch -----------------------------------------------------

template <class Cfg>
static hipError_t launch_cfg(const ChunkParams& prm, hipStream_t stream) {
    const int total = prm.BH * prm.n_slices;
    hipLaunchKernelGGL(kda_chunk_kernel<Cfg>, dim3(total), dim3(Cfg::NTHREADS), 0, stream, prm);
    return hipGetLastError();
}

int chunk_slice_width(int dk, int dv, int qkv_bf16, int64_t BH) {
    (void)qkv_bf16;
    // Prefer 32-column slices while that still gives >= 256 workgroups; else 16.
    if (dk == 64 && qkv_bf16 && BH * (dv / 64) >= 256) return 64;
    if (BH * (dv / 32) >= 256) return 32;
    return 16;
}

hipError_t launch_chunk(ChunkParams prm, int dk, int qkv_bf16, int nv, hipStream_t stream) {
    if (prm.BH == 0) return hipSuccess;
    prm.n_slices = prm.DV / nv;
#define KDA_CASE(DK_, NV_, C_, E_)                                             \
    if (dk == DK_ && nv == NV_ && (qkv_bf16 != 0) == (sizeof(E_) == 2))        \
        return launch_cfg<ChunkCfg<DK_, NV_, C_, E_>>(prm, stream);
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
