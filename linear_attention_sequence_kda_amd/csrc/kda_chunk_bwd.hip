// kda_chunk_bwd.hip -- chunkwise gradients of the gated delta rule
// (gfx950 / MI355X): the kernels of kda_chunk_bwd besides the prefill's own
// intra-chunk kernel and state pass.
//
// "Chunkwise DeltaNet makes the recurrence trainable on GPUs" ("22580: From
// GPT-2 to Kimi3, Explained", zharfai.com) is the motivation; the pages print
// the forward chunk form only ("22,580: From GPT-2 to Kimi K3"
// (yichencityu.github.io) section 6.3, with section 9.1's per-channel decay),
// so what follows is that form differentiated.  Per chunk of C tokens, with
// g_r the chunk-relative cumulative ln(alpha) (per key channel), K~ = K e^g,
// the forward computes
//
//   Y = diag(beta) (V - K~ S),  u = T Y,  T = (I + A)^-1,
//   A_rj = beta_r sum_c k_rc k_jc e^{g_rc - g_jc} (j < r),
//   O = (Q e^g) S + P u,  P_rj = sum_c q_rc k_jc e^{g_rc - g_jc} (j <= r),
//   S' = diag(e^{g_n}) S + (K e^{g_n - g})^T u.
//
// Given G = dJ/dS' and dO, the gradient flowing into u is
// du = P^T dO + (K e^{g_n - g}) G and the one into S is
// dJ/dS = diag(e^{g_n}) G + (Q e^g)^T dO - W^T du (W = T diag(beta) K~).
// That recursion runs backwards over the chunks; it has the forward state
// pass's shape, so it runs as that pass over "reverse records" (built by the
// intra-chunk kernel's gradient form, kda_rev_record.h),
// one per chunk in reverse chunk order: W <- K e^{g_n-g}, U <- P^T dO,
// K^T <- -W^T, decay e^{g_n}, and a second product of the same step,
// K2^T <- (Q e^g)^T with U2 <- dO; the state pass's scan form keeps G and du
// per chunk.  With S (forward scan), u, G and du per chunk, every chunk's
// gradients are independent:
//
//   dY = T^T du,  dv = beta dY,  dbeta = sum_n (V - K~ S) dY + sum_c k R,
//   dA = -(dY u^T) strictly lower,  dP = dO u^T lower,
//   R  = decayed(dA) K,   RP = decayed(dP) K            (rows r, sums j <= r)
//   RU = decayed^T(diag(beta) dA) K + decayed^T(dP) Q   (rows j, sums r >= j)
//   dq = RP + e^g (dO S^T)
//   dk = [beta R - beta e^g (dY S^T)] + [RU + e^{g_n-g} (u G^T)]
//   dg = q dq + k ([...] - [...]) (+ the e^{g_n} terms on the last row),
//   d ln(alpha)_t = sum_{r >= t} dg_r within the chunk,
//
// "decayed" being the sums with the factor e^{g_rc - g_jc} inside.  Those are
// split at 16-token blocks through an anchor token a per block (e^{g_r - g_a}
// on the result, e^{g_a - g_j} on the operand): below the diagonal block both
// factors are <= 1; a diagonal block whose total decay is at least -60 in
// every channel of a wave joins the same bf16 MFMA sum (its factors stay
// within e^60), a stronger one is summed directly in fp32.  dP's diagonal
// (no decay) stays out of the sums: its terms cancel exactly in dg and are
// added to dq and dk alone.
#include <type_traits>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

// ---- gate widening ---------------------------------------------------------------
template <bool GBF>
__global__ void __launch_bounds__(256) kda_gate_widen_kernel(GateWiden prm) {
    const int64_t per_row = prm.DK / 4;
    const int64_t total = prm.rows * per_row;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * 256) {
        const int64_t row = i / per_row;
        const int c4 = (int)(i - row * per_row) * 4;
        float la = 0.f;
        if (prm.log_alpha) {
            if constexpr (GBF) la = (float)((const bf16*)prm.log_alpha)[row];
            else la = ((const float*)prm.log_alpha)[row];
        }
        *(floatx4*)(prm.la + row * prm.DK + c4) = floatx4{la, la, la, la};
        if (c4 == 0) {
            if constexpr (GBF) prm.b[row] = (float)((const bf16*)prm.beta)[row];
            else prm.b[row] = ((const float*)prm.beta)[row];
        }
    }
}

hipError_t launch_gate_widen(const GateWiden& prm, hipStream_t stream) {
    if (prm.rows == 0) return hipSuccess;
    const int64_t total = prm.rows * (prm.DK / 4);
    int64_t grid = (total + 255) / 256;
    if (grid > 65536) grid = 65536;
    if (prm.gate_bf16)
        hipLaunchKernelGGL((kda_gate_widen_kernel<true>), dim3((unsigned)grid), dim3(256), 0, stream, prm);
    else
        hipLaunchKernelGGL((kda_gate_widen_kernel<false>), dim3((unsigned)grid), dim3(256), 0, stream, prm);
    return hipGetLastError();
}

// ---- chunk-parallel gradients -------------------------------------------------------
// One workgroup of 8 waves per (head, chunk).  Wave w owns the 16 key
// channels 16w.. of every [C, dk] result (dq, dk, dg) and the 16 value
// columns 16w.. of every [C, dv] one; a lane holds rows 16R + 4(l/16) + i,
// column l % 16 of each 16 x 16 block (the MFMA accumulator layout).
template <int DK_, int DV_>
struct GradCfg {
    static constexpr int DK = DK_, DV = DV_, C = 64, NB = 4, NT = 512;
    static constexpr int NCBK = DK / 16, NVB = DV / 16;
    // bf16 tiles: rows padded by 32 bytes; fp32 tiles by 16
    static constexpr int PK = DK + 16, PV = DV + 16, PCC = C + 16;
    static constexpr int PG = DK + 4, PT = C + 4, PDU = C + 4;
    // per-wave operands of the decayed sums: [C][16] bf16 row-major tiles
    static constexpr int XL = C * 16 * 2, XW = 3 * XL;
    // persistent areas
    static constexpr int O_G = 0;                            // g, fp32 [C][PG]
    static constexpr int O_K = O_G + C * PG * 4;             // k, bf16 [C][PK]
    static constexpr int O_DA = O_K + C * PK * 2;            // dA, bf16 [C][PCC]
    static constexpr int O_DP = O_DA + C * PCC * 2;          // dP
    static constexpr int O_BETA = O_DP + C * PCC * 2;        // beta [C]
    // dbeta partials, one row of C per wave for each of its three terms,
    // summed in a fixed order at the end (the same bits on every run)
    static constexpr int O_DB = O_BETA + C * 4;              // [3][8][C]
    static constexpr int O_ROW = O_DB + 3 * 8 * C * 4;       // row sums [C]
    static constexpr int O_PD = O_ROW + C * 4;               // diagonal of dP [C]
    static constexpr int O_EN = O_PD + C * 4;                // last-row dg terms [DK]
    static constexpr int O_PH = O_EN + DK * 4;               // phase area
    // phase area: (0) T^T fp32 [C][PT] + du^T fp32 [DV][PDU]; (1, 2) dY | dO |
    // S, later u, bf16 [C or DK][PV]; (3) G bf16 [DK][PV] over dY and dO;
    // (4) q bf16 [C][PK] + per-wave x~ tiles; (5) dg fp32 [C][PG]
    static constexpr int PH0 = C * PT * 4 + DV * PDU * 4;
    static constexpr int PH12 = 2 * C * PV * 2 + (DK > C ? DK : C) * PV * 2;
    static constexpr int PH4 = C * PK * 2 + NCBK * XW;
    static constexpr int PH5 = C * PG * 4;
    static constexpr int M01 = PH0 > PH12 ? PH0 : PH12;
    static constexpr int M45 = PH4 > PH5 ? PH4 : PH5;
    static constexpr int LDS_BYTES = O_PH + (M01 > M45 ? M01 : M45);
    static_assert(DK <= 2 * C, "G fits over dY and dO");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget of one gfx950 CU");
};

// sum over the 16 lanes of a DPP row, in every lane of it (rotations within
// the row; every lane of the wave must be active)
__device__ __forceinline__ float sum16(float x) {
    auto ror = [](float v, auto ctl) {
        return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                     decltype(ctl)::value, 0xf, 0xf, false));
    };
    x += ror(x, std::integral_constant<int, 0x128>{});  // row_ror:8
    x += ror(x, std::integral_constant<int, 0x124>{});  // row_ror:4
    x += ror(x, std::integral_constant<int, 0x122>{});  // row_ror:2
    x += ror(x, std::integral_constant<int, 0x121>{});  // row_ror:1
    return x;
}

template <int DK, int DV, bool GBF, bool SCAL>
__global__ void __launch_bounds__(512) kda_chunk_grad_kernel(ChunkGradParams prm) {
    typedef GradCfg<DK, DV> Cfg;
    typedef Frag<bf16> F;
    constexpr int C = Cfg::C, NB = Cfg::NB, NT = Cfg::NT, NCBK = Cfg::NCBK, NVB = Cfg::NVB;
    constexpr int PK = Cfg::PK, PV = Cfg::PV, PCC = Cfg::PCC, PG = Cfg::PG, PT = Cfg::PT;
    constexpr int PDU = Cfg::PDU;
    __shared__ __attribute__((aligned(16))) char smem[Cfg::LDS_BYTES];
    float* sG = (float*)(smem + Cfg::O_G);
    bf16* sK = (bf16*)(smem + Cfg::O_K);
    bf16* sdA = (bf16*)(smem + Cfg::O_DA);
    bf16* sdP = (bf16*)(smem + Cfg::O_DP);
    float* sBeta = (float*)(smem + Cfg::O_BETA);
    float* sDB = (float*)(smem + Cfg::O_DB);
    float* sRow = (float*)(smem + Cfg::O_ROW);
    float* sPd = (float*)(smem + Cfg::O_PD);
    float* sEn = (float*)(smem + Cfg::O_EN);
    char* ph = smem + Cfg::O_PH;
    float* sTT = (float*)ph;
    float* sdu = (float*)(ph + C * PT * 4);
    bf16* sDY = (bf16*)ph;
    bf16* sDO = (bf16*)(ph + C * PV * 2);
    bf16* sS = (bf16*)(ph + 2 * C * PV * 2);
    bf16* sU = sS;
    bf16* sGG = (bf16*)ph;
    bf16* sQ = (bf16*)ph;
    float* sDg = (float*)ph;

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63, lr = l & 15, q = l >> 4;
    const int nc = prm.nc;
    const int bh = blockIdx.x / nc, c = blockIdx.x - bh * nc;
    const int64_t L = prm.L;
    const int64_t t0 = (int64_t)c * C;
    const int n = (int)(L - t0 < C ? L - t0 : C);
    const int64_t row0 = (int64_t)bh * L + t0;
    const int64_t xf = (int64_t)bh * nc + c;             // forward-scan entry
    const int64_t xr = (int64_t)bh * nc + (nc - 1 - c);  // reverse-scan entry
    auto gate_at = [&](const void* base, int64_t i) -> float {
        if constexpr (GBF) return (float)((const bf16*)base)[i];
        else return ((const float*)base)[i];
    };

    // Every global load is issued one phase ahead, into registers, and goes
    // to LDS after that phase's barrier: tiles of 8-element pieces, piece i of
    // a [rows][cols] tile at row i / (cols / 8), column 8 (i % (cols / 8)).
    constexpr int NP_CV = (C * DV / 8 + NT - 1) / NT;   // [C][DV] pieces per thread
    constexpr int NP_CK = (C * DK / 8 + NT - 1) / NT;   // [C][DK]
    constexpr int NP_KV = (DK * DV / 8 + NT - 1) / NT;  // [DK][DV]
    constexpr int NP_TT = C * C / 4 / NT;               // T^T, fp32 4-element pieces
    static_assert((C * DV / 8) % NT == 0 && (C * DK / 8) % NT == 0 && (C * C / 4) % NT == 0,
                  "every thread takes whole pieces");
    // (loads are unconditional, from clamped addresses, and masked after:
    // a load under a branch would be waited for at the branch's end)
    auto ld_rows = [&](uint4 (&dst)[NP_CV > NP_CK ? NP_CV : NP_CK], const bf16* base, int cols,
                       int np) {
        for (int it = 0; it < np; ++it) {
            const int i = tid + NT * it;  // (C * cols / 8 is a multiple of NT)
            const int r = i / (cols / 8), c8 = (i % (cols / 8)) * 8;
            const uint4 v = *(const uint4*)(base + (int64_t)(r < n ? r : n - 1) * cols + c8);
            dst[it] = keep_or_zero(v, r < n);
        }
    };

    constexpr int NPR = NP_CV > NP_CK ? NP_CV : NP_CK;
    auto st_rows = [&](const uint4 (&src)[NPR], bf16* dst, int pitch, int cols, int np) {
        for (int it = 0; it < np; ++it) {
            const int i = tid + NT * it;
            if (i < C * cols / 8) {
                const int r = i / (cols / 8), c8 = (i % (cols / 8)) * 8;
                *(uint4*)(dst + r * pitch + c8) = src[it];
            }
        }
    };
    // fp32 [DK][DV] state tiles
    auto ld_state = [&](floatx4 (&dst)[NP_KV][2], const float* base) {
#pragma unroll
        for (int it = 0; it < NP_KV; ++it) {
            const int i = tid + NT * it;
            const int r = i / (DV / 8), c8 = (i % (DV / 8)) * 8;
            if (i < DK * DV / 8) {
                dst[it][0] = *(const floatx4*)(base + r * DV + c8);
                dst[it][1] = *(const floatx4*)(base + r * DV + c8 + 4);
            }
        }
    };
    auto st_state = [&](const floatx4 (&src)[NP_KV][2], bf16* dst) {
#pragma unroll
        for (int it = 0; it < NP_KV; ++it) {
            const int i = tid + NT * it;
            if (i < DK * DV / 8) {
                const int r = i / (DV / 8), c8 = (i % (DV / 8)) * 8;
                const floatx4 a = src[it][0], b = src[it][1];
                *(bf16x8*)(dst + r * PV + c8) = bf16x8{(bf16)a[0], (bf16)a[1], (bf16)a[2], (bf16)a[3],
                                                       (bf16)b[0], (bf16)b[1], (bf16)b[2], (bf16)b[3]};
            }
        }
    };

    // ---- T^T, du and k; beta, g (cumulative ln alpha per channel) -------------------
    // (loads in the order of first use: the gates, then T^T, du and k, then dO
    // and S for the next phase; loads complete in order)
    // gates: four threads per channel, 16 rows each
    const int gch = tid >> 2, gp = tid & 3;
    float gv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int r = 16 * gp + i;
        // (one decay per token: the row's value serves every channel)
        const int64_t rg = row0 + (r < n ? r : n - 1);
        const float x = gate_at(prm.la, SCAL ? rg * prm.la_rs : rg * DK + (gch < DK ? gch : DK - 1));
        gv[i] = (gch < DK && r < n) ? x : 0.f;
    }
    const float bload = gate_at(prm.beta, row0 + ((tid & (C - 1)) < n ? (tid & (C - 1)) : n - 1));
    floatx4 rtt[NP_TT];
    uint4 rdu[NPR], rk[NPR], rdo[NPR];
    floatx4 rs[NP_KV][2];
    {
        const float* gtt = prm.tt + xf * C * C;
#pragma unroll
        for (int it = 0; it < NP_TT; ++it) {
            const int i = tid + NT * it;
            rtt[it] = *(const floatx4*)(gtt + (i / (C / 4)) * C + (i % (C / 4)) * 4);
        }
        // du has no rows past the sequence end to drop (the scan wrote zeros)
        const bf16* gdu = (const bf16*)prm.du_all + xr * C * DV;
#pragma unroll
        for (int it = 0; it < NP_CV; ++it) {
            const int i = tid + NT * it;
            rdu[it] = make_uint4(0u, 0u, 0u, 0u);
            if (i < C * DV / 8) rdu[it] = *(const uint4*)(gdu + (i / (DV / 8)) * DV + (i % (DV / 8)) * 8);
        }
        ld_rows(rk, (const bf16*)prm.k + row0 * DK, DK, NP_CK);
        ld_rows(rdo, (const bf16*)prm.dout + row0 * DV, DV, NP_CV);
        ld_state(rs, prm.S_all + xf * DK * DV);
    }
    if (tid < C) sBeta[tid] = tid < n ? bload : 0.f;
    for (int i = tid; i < 3 * 8 * C; i += NT) sDB[i] = 0.f;
    {
        // prefix within each thread's 16 rows, offsets across its four threads
        const int ch = gch, p = gp;
        float* v = gv;
        float run = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            run += v[i];
            v[i] = run;
        }
        const int base = l & ~3;
        const float s0 = __shfl(run, base), s1 = __shfl(run, base + 1), s2 = __shfl(run, base + 2);
        const float off = (p > 0 ? s0 : 0.f) + (p > 1 ? s1 : 0.f) + (p > 2 ? s2 : 0.f);
        if (ch < DK) {
#pragma unroll
            for (int i = 0; i < 16; ++i) sG[(16 * p + i) * PG + ch] = v[i] + off;
        }
    }
#pragma unroll
    for (int it = 0; it < NP_TT; ++it) {
        const int i = tid + NT * it;
        *(floatx4*)(sTT + (i / (C / 4)) * PT + (i % (C / 4)) * 4) = rtt[it];
    }
#pragma unroll
    for (int it = 0; it < NP_CV; ++it) {
        const int i = tid + NT * it;
        if (i < C * DV / 8) {
            const int r = i / (DV / 8), j8 = (i % (DV / 8)) * 8;
            const bf16x8 v = __builtin_bit_cast(bf16x8, rdu[it]);
            // transposed, so that dY = T^T du reads both operands k-contiguous
#pragma unroll
            for (int e = 0; e < 8; ++e) sdu[(j8 + e) * PDU + r] = (float)v[e];
        }
    }
    st_rows(rk, sK, PK, DK, NP_CK);
    __syncthreads();

    // ---- dY = T^T du (fp32 MFMA); dv = beta dY  (dO and S arriving; u and v on their way)
    uint4 ru[NPR], rv[NPR];
    {
        // u has no rows past the sequence end to drop (zero records there)
        const bf16* gu = (const bf16*)prm.u_all + xf * C * DV;
#pragma unroll
        for (int it = 0; it < NP_CV; ++it) {
            const int i = tid + NT * it;
            ru[it] = make_uint4(0u, 0u, 0u, 0u);
            if (i < C * DV / 8) ru[it] = *(const uint4*)(gu + (i / (DV / 8)) * DV + (i % (DV / 8)) * 8);
        }
    }
    ld_rows(rv, (const bf16*)prm.v + row0 * DV, DV, NP_CV);
    floatx4 dY[NB];
    if (w < NVB) {
#pragma unroll
        for (int R = 0; R < NB; ++R) {
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
            dY[R] = mma_block<float>(acc, sTT + 16 * R * PT, PT, sdu + 16 * w * PDU, PDU, C);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * R + 4 * q + i;
                if (r < n) prm.dv_out[(row0 + r) * DV + 16 * w + lr] = sBeta[r] * dY[R][i];
            }
        }
    }
    __syncthreads();

    // ---- dY, dO and S to bf16 tiles (u and v on their way) -------------------------
    if (w < NVB) {
#pragma unroll
        for (int R = 0; R < NB; ++R)
#pragma unroll
            for (int i = 0; i < 4; ++i) sDY[(16 * R + 4 * q + i) * PV + 16 * w + lr] = (bf16)dY[R][i];
    }
    st_rows(rdo, sDO, PV, DV, NP_CV);
    st_state(rs, sS);
    __syncthreads();

    // ---- dO S^T, dY S^T; dbeta's first term ---------------------------------------
    // (V - K~ S) . dY = v . dY - sum_c k e^g (dY S^T): the second part comes
    // with dY S^T, so V - K~ S is never formed
    floatx4 dq[NB], dka[NB], dkb[NB];
#pragma unroll
    for (int R = 0; R < NB; ++R) {
        dq[R] = floatx4{0.f, 0.f, 0.f, 0.f};
        dka[R] = dq[R];
        dkb[R] = dq[R];
    }
    // v . dY by rows: the DV/8 pieces of a row sit in adjacent lanes
#pragma unroll
    for (int it = 0; it < NP_CV; ++it) {
        const int i = tid + NT * it;
        const int r = i / (DV / 8), c8 = (i % (DV / 8)) * 8;
        float part = 0.f;
        if (i < C * DV / 8) {
            const bf16x8 dyv = *(const bf16x8*)(sDY + r * PV + c8);
            const bf16x8 vv = __builtin_bit_cast(bf16x8, rv[it]);
#pragma unroll
            for (int e = 0; e < 8; ++e) part += (float)vv[e] * (float)dyv[e];
        }
#pragma unroll
        for (int o = 1; o < DV / 8; o <<= 1) part += __shfl_xor(part, o);
        if (i < C * DV / 8 && (i % (DV / 8)) == 0) sDB[r] = part;
    }
    if (w < NCBK) {
        const int ch = 16 * w + lr;
#pragma unroll
        for (int R = 0; R < NB; ++R) {
            floatx4 z = {0.f, 0.f, 0.f, 0.f};
            const floatx4 m1 = mma_block<bf16>(z, sDO + 16 * R * PV, PV, sS + 16 * w * PV, PV, DV);
            const floatx4 m2 = mma_block<bf16>(z, sDY + 16 * R * PV, PV, sS + 16 * w * PV, PV, DV);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * R + 4 * q + i;
                const float eg = __expf(sG[r * PG + ch]);
                dq[R][i] = eg * m1[i];
                dka[R][i] = -sBeta[r] * eg * m2[i];
                const float part = sum16((float)sK[r * PK + ch] * eg * m2[i]);
                if (lr == 0) sDB[(16 + w) * C + r] = -part;
            }
        }
    }
    __syncthreads();

    // ---- u over S; dA = -(dY u^T) strictly lower, dP = dO u^T lower (G on its way) --
    // dP's diagonal is kept apart (fp32): its terms carry no decay, enter dq as
    // dP_rr k_r and dk as dP_rr q_r and cancel exactly in dg, so they are
    // added to dq and dk at the end and never enter dg or the decayed sums
    st_rows(ru, sU, PV, DV, NP_CV);
    floatx4 rg[NP_KV][2];
    ld_state(rg, prm.G_all + xr * DK * DV);
    __syncthreads();
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int t = w + 8 * m;           // 32 blocks: (matrix, R, J)
        const int mat = t >> 4, R = (t >> 2) & 3, J = t & 3;
        bf16* dst = mat ? sdP : sdA;
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        if (J <= R) acc = mma_block<bf16>(acc, (mat ? sDO : sDY) + 16 * R * PV, PV, sU + 16 * J * PV, PV, DV);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * R + 4 * q + i, j = 16 * J + lr;
            float x = j < r ? (mat ? acc[i] : -acc[i]) : 0.f;
            // one decay per token: the factor e^{g_r - g_j} (<= 1 below the
            // diagonal) goes into the tile here, in fp32
            if constexpr (SCAL) x *= j < r ? __expf(sG[r * PG] - sG[j * PG]) : 0.f;
            dst[r * PCC + j] = (bf16)x;
            if (mat && j == r) sPd[r] = acc[i];
        }
    }
    __syncthreads();

    // ---- G over dY and dO; the e^{g_n} G.S term; u G^T  (q on its way) -------------
    // (S and G stay fp32 in memory: the sum G.S below is a long dot product
    // whose terms largely cancel in d ln(alpha), which bf16 copies of S or G
    // would not resolve)
    st_state(rg, sGG);
    {
        // d g_n += e^{g_n} sum_j G[c][j] S[c][j]: this thread's fp32 pieces of
        // G against the fp32 pieces of S it loaded for the S tile (the same
        // elements; the DV/8 pieces of a row in adjacent lanes)
#pragma unroll
        for (int it = 0; it < NP_KV; ++it) {
            const int i = tid + NT * it;
            const int r = i / (DV / 8);
            const floatx4 a = rs[it][0], b = rs[it][1];
            float d = a[0] * rg[it][0][0] + a[1] * rg[it][0][1] + a[2] * rg[it][0][2] +
                      a[3] * rg[it][0][3] + b[0] * rg[it][1][0] + b[1] * rg[it][1][1] +
                      b[2] * rg[it][1][2] + b[3] * rg[it][1][3];
#pragma unroll
            for (int o = 1; o < DV / 8; o <<= 1) d += __shfl_xor(d, o);
            if (i < DK * DV / 8 && (i % (DV / 8)) == 0) sEn[r] = __expf(sG[(C - 1) * PG + r]) * d;
        }
    }
    uint4 rq[NPR];
    ld_rows(rq, (const bf16*)prm.q + row0 * DK, DK, NP_CK);
    __syncthreads();
    if (w < NCBK) {
        const int ch = 16 * w + lr;
        const float gn = sG[(C - 1) * PG + ch];
        float en = 0.f;
#pragma unroll
        for (int R = 0; R < NB; ++R) {
            floatx4 z = {0.f, 0.f, 0.f, 0.f};
            const floatx4 m3 = mma_block<bf16>(z, sU + 16 * R * PV, PV, sGG + 16 * w * PV, PV, DV);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * R + 4 * q + i;
                const float t = __expf(gn - sG[r * PG + ch]) * m3[i];
                dkb[R][i] = t;
                en += (float)sK[r * PK + ch] * t;
            }
        }
        en = sum_over_lq(en);
        if (q == 0) atomicAdd(sEn + ch, en);
    }
    __syncthreads();

    // ---- q; the decayed products ---------------------------------------------------
    st_rows(rq, sQ, PK, DK, NP_CK);
    __syncthreads();
    bf16* xl = (bf16*)(ph + C * PK * 2 + w * Cfg::XW);  // [C][16]: lower sums' operand
    bf16* xuk = (bf16*)((char*)xl + Cfg::XL);           // [C][16]: upper sums' operands
    bf16* xuq = (bf16*)((char*)xuk + Cfg::XL);
    const int ch = 16 * w + lr;
    // Each wave builds and reads only its own operand tiles here (everything
    // else the loop reads was written before it), so the waves need no
    // workgroup barrier inside it: a wave's LDS accesses take effect in order
    // once they have issued, and the fence keeps the compiler from moving them.
    auto wave_fence = []() {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
        __builtin_amdgcn_wave_barrier();
        asm volatile("" ::: "memory");
    };
    if constexpr (SCAL) {
        // One decay per token (or none): D_rj = e^{g_r - g_j} is one scalar per
        // pair, already inside the dA and dP tiles, so the three decayed sums
        // are plain products:
        //   R = (dA o D) K,  RP = (dP o D) K,  RU = (dA o D)^T (beta K) + (dP o D)^T Q
        if (w < NCBK) {
            {
                // this wave's 16 channels of beta K, [C][16] (one row per lane)
                const float br = sBeta[l];
                const bf16x8 k0 = *(const bf16x8*)(sK + l * PK + 16 * w);
                const bf16x8 k1 = *(const bf16x8*)(sK + l * PK + 16 * w + 8);
                bf16x8 x0, x1;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    x0[e] = (bf16)(br * (float)k0[e]);
                    x1[e] = (bf16)(br * (float)k1[e]);
                }
                *(bf16x8*)(xuk + l * 16) = x0;
                *(bf16x8*)(xuk + l * 16 + 8) = x1;
            }
            wave_fence();
#pragma unroll
            for (int R = 0; R < NB; ++R) {
                // columns j < r <= 16 R + 15 (the tiles are zero from the diagonal on)
                constexpr int KS = Frag<bf16>::KS;
                const int KR = (16 * R + 16 + KS - 1) / KS * KS;
                floatx4 accR = {0.f, 0.f, 0.f, 0.f}, accP = accR;
                accR = mma_block_bt<bf16>(accR, sdA + 16 * R * PCC, PCC, sK, PK, 16 * w, KR);
                accP = mma_block_bt<bf16>(accP, sdP + 16 * R * PCC, PCC, sK, PK, 16 * w, KR);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * R + 4 * q + i;
                    dq[R][i] += accP[i];
                    dka[R][i] += sBeta[r] * accR[i];
                    const float part = sum16((float)sK[r * PK + ch] * accR[i]);
                    if (lr == 0) sDB[(8 + w) * C + r] = part;
                }
            }
#pragma unroll
            for (int J = 0; J < NB; ++J) {
                // rows r > j >= 16 J; both operands read transposed
                constexpr int KS = Frag<bf16>::KS;
                floatx4 acc = {0.f, 0.f, 0.f, 0.f};
                for (int kk = 16 * J / KS * KS; kk < C; kk += KS) {
                    acc = F::mma(acc, load_frag_tr(sdA, PCC, kk, 16 * J), load_frag_tr(xuk, 16, kk, 0));
                    acc = F::mma(acc, load_frag_tr(sdP, PCC, kk, 16 * J), load_frag_tr(sQ, PK, kk, 16 * w));
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) dkb[J][i] += acc[i];
            }
        }
    } else {
        // One anchor per AB-token block: the sums of row tiles (lower) and of
        // column tiles (upper) inside block s share one set of operand tiles.
        constexpr int AB = 64, TPB = AB / 16;
        static_assert(C % AB == 0 && AB % 32 == 0, "whole blocks of k steps");
#pragma unroll
        for (int s = 0; s < C / AB; ++s) {
            const int b0 = AB * s;  // the block's first row
            // Block s is "moderate" for this wave when its total decay is at
            // least -60 in each of the wave's 16 channels: then one anchor per
            // sum covers the block's own rows too (their factors stay below
            // e^60) and the whole sum runs on MFMA.  Otherwise the block's own
            // rows are summed directly and only the rows off it take anchored
            // MFMA operands.
            const float zb = w < NCBK ? sG[(b0 + AB - 1) * PG + ch] - (s ? sG[(b0 - 1) * PG + ch] : 0.f)
                                      : 0.f;
            const bool mild = __all(zb >= -60.f);
            // lower sums of the block's rows are anchored at la = b0 - 1 (rows
            // j < b0, and with a mild block also its rows), upper sums of its
            // columns at ua = b0 + AB - 1 (rows r > ua, and with a mild block
            // also its rows)
            const int la = b0 - 1, ua = b0 + AB - 1;
            const int lrows = mild ? b0 + AB : b0;  // rows of the lower operand
            const int ufirst = mild ? b0 : ua + 1;  // first row of the upper ones
            // (each lane builds 8 channels of one row per step: one 16-byte k or q
            // piece, two of g, one of the anchor's g)
            if (w < NCBK) {
                const int h8 = 16 * w + 8 * (l & 1);  // this lane's 8 channels
                if (lrows > 0) {
                    floatx4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0;
                    if (la >= 0) {
                        a0 = *(const floatx4*)(sG + la * PG + h8);
                        a1 = *(const floatx4*)(sG + la * PG + h8 + 4);
                    }
                    for (int t = l; t < lrows * 2; t += 64) {
                        const int j = t >> 1;
                        const bf16x8 kv = *(const bf16x8*)(sK + j * PK + h8);
                        const floatx4 g0 = *(const floatx4*)(sG + j * PG + h8);
                        const floatx4 g1 = *(const floatx4*)(sG + j * PG + h8 + 4);
                        bf16x8 x;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            x[e] = (bf16)((float)kv[e] * __expf(a0[e] - g0[e]));
                            x[4 + e] = (bf16)((float)kv[4 + e] * __expf(a1[e] - g1[e]));
                        }
                        *(bf16x8*)(xl + j * 16 + 8 * (l & 1)) = x;
                    }
                }
                if (ufirst < C) {
                    const floatx4 a0 = *(const floatx4*)(sG + ua * PG + h8);
                    const floatx4 a1 = *(const floatx4*)(sG + ua * PG + h8 + 4);
                    for (int t = l; t < (C - ufirst) * 2; t += 64) {
                        const int r = ufirst + (t >> 1);
                        const float br = sBeta[r];
                        const bf16x8 kv = *(const bf16x8*)(sK + r * PK + h8);
                        const bf16x8 qv = *(const bf16x8*)(sQ + r * PK + h8);
                        const floatx4 g0 = *(const floatx4*)(sG + r * PG + h8);
                        const floatx4 g1 = *(const floatx4*)(sG + r * PG + h8 + 4);
                        bf16x8 xk, xq;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float f0 = __expf(g0[e] - a0[e]), f1 = __expf(g1[e] - a1[e]);
                            xk[e] = (bf16)(br * (float)kv[e] * f0);
                            xk[4 + e] = (bf16)(br * (float)kv[4 + e] * f1);
                            xq[e] = (bf16)((float)qv[e] * f0);
                            xq[4 + e] = (bf16)((float)qv[4 + e] * f1);
                        }
                        *(bf16x8*)(xuk + r * 16 + 8 * (l & 1)) = xk;
                        *(bf16x8*)(xuq + r * 16 + 8 * (l & 1)) = xq;
                    }
                }
            }
            wave_fence();
            if (w < NCBK) {
                // lower sums of the block's row tiles: R = decayed(dA) K,
                // RP = decayed(dP) K (j < r; the tiles are zero from the
                // diagonal on, so the operand's rows past a tile's own add zero)
#pragma unroll
                for (int R = TPB * s; R < TPB * (s + 1); ++R) {
                    floatx4 accR = {0.f, 0.f, 0.f, 0.f}, accP = accR;
                    if (lrows > 0) {
                        accR = mma_block_bt<bf16>(accR, sdA + 16 * R * PCC, PCC, xl, 16, 0, lrows);
                        accP = mma_block_bt<bf16>(accP, sdP + 16 * R * PCC, PCC, xl, 16, 0, lrows);
                        const float ga = la >= 0 ? sG[la * PG + ch] : 0.f;
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float f = __expf(sG[(16 * R + 4 * q + i) * PG + ch] - ga);
                            accR[i] *= f;
                            accP[i] *= f;
                        }
                    }
                    if (!mild) {
                        // the block's own rows j < r, directly (exponents <= 0)
                        float gr[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) gr[i] = sG[(16 * R + 4 * q + i) * PG + ch];
#pragma unroll 4
                        for (int j = b0; j < 16 * R + 16; ++j) {
                            const float gj = sG[j * PG + ch], kj = (float)sK[j * PK + ch];
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const int r = 16 * R + 4 * q + i;
                                const float e = __expf(fminf(gr[i] - gj, 0.f)) * kj;
                                accP[i] += (float)sdP[r * PCC + j] * e;
                                accR[i] += (float)sdA[r * PCC + j] * e;
                            }
                        }
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int r = 16 * R + 4 * q + i;
                        dq[R][i] += accP[i];
                        dka[R][i] += sBeta[r] * accR[i];
                        const float part = sum16((float)sK[r * PK + ch] * accR[i]);
                        if (lr == 0) sDB[(8 + w) * C + r] = part;
                    }
                }
                // upper sums of the block's column tiles:
                // RU = decayed^T(beta dA) K + decayed^T(dP) Q (r > j)
#pragma unroll
                for (int J = TPB * s; J < TPB * (s + 1); ++J) {
                    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
                    if (ufirst < C) {
                        // both operands read transposed: A[j][r] = dA[r][j], B[c][r] = x~[r][c]
                        for (int kk = ufirst; kk < C; kk += 32) {
                            acc = F::mma(acc, load_frag_tr(sdA, PCC, kk, 16 * J), load_frag_tr(xuk, 16, kk, 0));
                            acc = F::mma(acc, load_frag_tr(sdP, PCC, kk, 16 * J), load_frag_tr(xuq, 16, kk, 0));
                        }
                        const float ga = sG[ua * PG + ch];
#pragma unroll
                        for (int i = 0; i < 4; ++i) acc[i] *= __expf(ga - sG[(16 * J + 4 * q + i) * PG + ch]);
                    }
                    if (!mild) {
                        float gj[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) gj[i] = sG[(16 * J + 4 * q + i) * PG + ch];
#pragma unroll 4
                        for (int r = 16 * J + 1; r <= ua; ++r) {
                            const float g_r = sG[r * PG + ch];
                            const float kr = sBeta[r] * (float)sK[r * PK + ch], qr = (float)sQ[r * PK + ch];
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const int j = 16 * J + 4 * q + i;
                                const float e = __expf(fminf(g_r - gj[i], 0.f));
                                acc[i] += e * ((float)sdP[r * PCC + j] * qr + (float)sdA[r * PCC + j] * kr);
                            }
                        }
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) dkb[J][i] += acc[i];
                }
            }
            wave_fence();
        }
    }

    // ---- outputs: dq, dk; dg = q dq + k (dka - dkb) -> reverse sums; dbeta -----------
    floatx4 dg[NB];
    if (w < NCBK) {
#pragma unroll
        for (int R = 0; R < NB; ++R)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * R + 4 * q + i;
                if (r < n) {
                    const float pd = sPd[r];
                    prm.dq[(row0 + r) * DK + ch] = dq[R][i] + pd * (float)sK[r * PK + ch];
                    prm.dk[(row0 + r) * DK + ch] = dka[R][i] + dkb[R][i] + pd * (float)sQ[r * PK + ch];
                }
                dg[R][i] = (float)sQ[r * PK + ch] * dq[R][i] +
                           (float)sK[r * PK + ch] * (dka[R][i] - dkb[R][i]);
            }
    }
    __syncthreads();
    if (w < NCBK) {
#pragma unroll
        for (int R = 0; R < NB; ++R)
#pragma unroll
            for (int i = 0; i < 4; ++i) sDg[(16 * R + 4 * q + i) * PG + ch] = dg[R][i];
    }
    __syncthreads();
    if (prm.dla_mode == 2) {
        // per channel: suffix sums over rows, four threads per channel
        const int c4 = tid >> 2, p = tid & 3;
        float v[16], run = 0.f;
#pragma unroll
        for (int i = 15; i >= 0; --i) {
            run += c4 < DK ? sDg[(16 * p + i) * PG + c4] : 0.f;
            v[i] = run;
        }
        const int base = l & ~3;
        const float t1 = __shfl(run, base + 1), t2 = __shfl(run, base + 2), t3 = __shfl(run, base + 3);
        if (c4 < DK) {
            const float off = (p < 1 ? t1 : 0.f) + (p < 2 ? t2 : 0.f) + (p < 3 ? t3 : 0.f) + sEn[c4];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int r = 16 * p + i;
                if (r < n) prm.dla[(row0 + r) * DK + c4] = v[i] + off;
            }
        }
    } else if (prm.dla_mode == 1) {
        // one decay per token: sum over channels, then suffix sums over rows
        if (tid < C) {
            float s = 0.f;
            for (int c2 = 0; c2 < DK; ++c2) s += sDg[tid * PG + c2];
            sRow[tid] = s;
        }
        __syncthreads();
        if (w == 0) {
            float x = sRow[l];
            float en = 0.f;
            for (int c2 = l; c2 < DK; c2 += 64) en += sEn[c2];
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) en += __shfl_xor(en, o);
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const float y = __shfl_down(x, o);
                if (l + o < 64) x += y;
            }
            if (l < n) prm.dla[row0 + l] = x + en;
        }
    }
    if (tid < n) {
        float db = 0.f;
#pragma unroll
        for (int v = 0; v < 3 * 8; ++v) db += sDB[v * C + tid];
        prm.dbeta[row0 + tid] = db;
    }
}

hipError_t launch_chunk_grad(const ChunkGradParams& prm, int dk, int dv, hipStream_t stream) {
    if (prm.BH == 0 || prm.nc == 0) return hipSuccess;
    const unsigned grid = (unsigned)((int64_t)prm.BH * prm.nc);
#define KDA_CASE(DK_, DV_)                                                                     \
    if (dk == DK_ && dv == DV_) {                                                              \
        if (prm.dla_mode != 2 && prm.gate_bf16)                                                \
            hipLaunchKernelGGL((kda_chunk_grad_kernel<DK_, DV_, true, true>), dim3(grid), dim3(512), 0, stream, prm); \
        else if (prm.dla_mode != 2)                                                            \
            hipLaunchKernelGGL((kda_chunk_grad_kernel<DK_, DV_, false, true>), dim3(grid), dim3(512), 0, stream, prm); \
        else if (prm.gate_bf16)                                                                \
            hipLaunchKernelGGL((kda_chunk_grad_kernel<DK_, DV_, true, false>), dim3(grid), dim3(512), 0, stream, prm); \
        else                                                                                   \
            hipLaunchKernelGGL((kda_chunk_grad_kernel<DK_, DV_, false, false>), dim3(grid), dim3(512), 0, stream, prm); \
        return hipGetLastError();                                                              \
    }
    KDA_CASE(128, 128)
    KDA_CASE(128, 64)
    KDA_CASE(64, 128)
    KDA_CASE(64, 64)
#undef KDA_CASE
    return hipErrorInvalidValue;
}

}  // namespace kda
