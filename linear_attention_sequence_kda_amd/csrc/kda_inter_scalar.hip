// kda_inter_scalar.hip -- inter-chunk kernel of the chunkwise prefill for one
// decay per token (Gated DeltaNet) or none (DeltaNet), gfx950 / MI355X.
//
// "22,580: From GPT-2 to Kimi K3" (yichencityu.github.io), section 6.3: one
// state is carried from chunk to chunk; inside a chunk the delta corrections
// come from the WY factors T = (I + A)^-1.  With one decay per token the decay
// leaves every channel sum (section 08), so with g_r the chunk-relative
// cumulative ln(alpha), T' = T diag(beta) from the intra-chunk kernel's record
// and the stored q, k, v:
//
//   X = V - diag(e^g) (K S)                     (k against the decayed state)
//   u = T' X
//   P_rj = (Q K^T)_rj e^{g_r - g_j}   (j <= r)
//   O = diag(e^g) (Q S) + P u
//   S <- e^{g_n} S + K^T diag(e^{g_n - g}) u
//
// (merging T' V - T' diag(e^g) K S into T' X keeps W = T' diag(e^g) K off the
// chip and out of memory).  Every MFMA operand is a stored bf16 (or fp32)
// input, or T', X and u rounded once to the input type; decays are applied to
// the fp32 results.
//
// One workgroup owns one (b, h) head and a slice of NV state columns (columns
// of S evolve independently, so slices never talk) and walks the chunks in
// order; the fp32 state slice lives in registers of eight compute waves, with
// a transposed operand copy in LDS.  Eight data waves keep two chunks of
// inputs (k, the v slice, T' from the record) in flight in registers, write
// each into one half of a two-slot LDS ring one chunk ahead of use, and store
// the previous chunk's o tile.  q is only ever a B operand (of Q S and of
// P), so the compute waves load their q fragments straight from memory into
// registers, two chunks ahead, and q never passes through LDS.  Per chunk the
// compute waves run three phases, each ended by a barrier:
//   1  X = V - e^g (K S),  Q S (kept in registers),  P
//   2  u = T' X  (and e^{g_n-g} u)
//   3  S = e^{g_n} S + K^T (e^{g_n-g} u),  o = e^g Q S + P u
// Inputs are read through buffer resources bounded by the head's sequence, so
// the ragged last chunk reads zeros past token L and its o stores past token L
// are dropped, with no branch.
//
// LA instance: normalized linear attention with the feature map
// phi(x) = elu(x) + 1 ("22,580: From GPT-2 to Kimi K3", section 4: the state
// takes phi(k)^T v, a normalizer z takes phi(k), and the output is
// phi(q) S / (phi(q) z), read after the write).  The same walk with
// alpha = beta = 1 and no delta term: X = V, u = X (no record, no T'), and
//   den_r = phi(q_r) z_prev + sum_{j <= r} P_rj,   o = (Q S + P V) / den
//   z <- z + phi(K)^T 1   (an MFMA of the K^T operand against ones over the
//                         chunk's valid tokens)
// q arrives as phi(q) (kda_feature_map_kernel writes it once per call: every
// compute wave holds q fragments, so applying phi there would repeat the
// exponentials for each wave and column slice); the data waves apply phi to k
// on its way into the ring, once per workgroup.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

template <int DK_, int NV_, int C_, typename E_>
struct ScalarInterCfg {
    typedef E_ E;
    static constexpr int DK = DK_, NV = NV_, C = C_;
    static constexpr int NB = C / 16, NCB = DK / 16, NVB = NV / 16;
    static constexpr int NPAIR = NB * (NB + 1) / 2;
    static constexpr int ESZ = sizeof(E);
    static constexpr int PADE = 32 / ESZ;
    static constexpr int PK = DK + PADE;   // k tile [C][DK], S^T [NV][DK]
    static constexpr int PV = NV + PADE;   // v slice, o tile [C][NV]
    static constexpr int PC = C + PADE;    // T', P [C][C]; X^T, u^T [NV][C]
    static constexpr int NWC = 8, NWP = 8; // compute waves, data waves
    static constexpr int NT = 64 * (NWC + NWP);
    static constexpr int NTILE = NB * NVB;             // X / Q S / u / o tiles
    static constexpr int ITL = (NTILE + NWC - 1) / NWC;
    // state tiles (cb, vb): wave w < NSW holds cb = CBW w .. CBW w + CBW-1
    // for every vb, so the K^T fragments of a channel block and the u^T
    // fragments of a column block are each read by as few waves as possible
    static constexpr int CBW = 2;
    static constexpr int NSW = NCB / CBW;
    // ring slot: k tile, v slice, T', decay scalars
    static constexpr int O_SK = 0;
    static constexpr int O_SV = O_SK + C * PK * ESZ;
    static constexpr int O_STB = O_SV + C * PV * ESZ;
    static constexpr int O_SRS = O_STB + C * PC * ESZ;
    static constexpr int SLOT = O_SRS + 1024;
    // 1 KiB pieces of one chunk: k, v slice, T', scalars
    static constexpr int NKP = C * DK * ESZ / 1024;
    static constexpr int NVP = C * NV * ESZ / 1024;
    static constexpr int NTP = C * C * ESZ / 1024;
    static constexpr int NPIECE = NKP + NVP + NTP + 1;
    // LDS
    static constexpr int O_RING = 0;
    static constexpr int O_SINK = O_RING + 2 * SLOT;
    static constexpr int O_ST = O_SINK + 1024;
    static constexpr int O_XT = O_ST + NV * PK * ESZ;
    static constexpr int O_P = O_XT + NV * PC * ESZ;
    static constexpr int O_UT = O_P + C * PC * ESZ;
    static constexpr int O_UHT = O_UT + NV * PC * ESZ;
    static constexpr int O_O = O_UHT + NV * PC * ESZ;
    static constexpr int LDS_BYTES = O_O + 2 * C * PV * ESZ;   // o tiles of two chunks
    static_assert(DK % 32 == 0 && NV % 16 == 0 && (C == 32 || C == 64), "tile shape");
    static_assert(NV * ESZ >= 32 && (C * NV * ESZ) % 1024 == 0, "v slice pieces");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget of one gfx950 CU");
};

// NORM: q and k arrive raw (KDA_IN_NORM_QK); a separate instance, so the
// registers the row norms take never cost the plain path.  LA: linear
// attention (see above).
template <class Cfg, bool NORM, bool LA>
__global__ void __launch_bounds__(Cfg::NT) kda_inter_scalar_kernel(InterParams prm) {
    typedef typename Cfg::E E;
    typedef Frag<E> F;
    constexpr int DK = Cfg::DK, NV = Cfg::NV, C = Cfg::C, NB = Cfg::NB;
    constexpr int NCB = Cfg::NCB, NVB = Cfg::NVB;
    constexpr int PK = Cfg::PK, PV = Cfg::PV, PC = Cfg::PC;
    constexpr int NWC = Cfg::NWC, NWP = Cfg::NWP;
    constexpr int NTILE = Cfg::NTILE, ITL = Cfg::ITL, CBW = Cfg::CBW, NSW = Cfg::NSW;
    constexpr int ESZ = Cfg::ESZ, W = F::W, KS = F::KS;
    constexpr int SLOT = Cfg::SLOT;
    constexpr RecLayout RL = rec_layout_thin(C, ESZ);

    __shared__ __attribute__((aligned(16))) char smem[Cfg::LDS_BYTES];
    char* ring = smem + Cfg::O_RING;
    E* sST = (E*)(smem + Cfg::O_ST);
    E* sXT = (E*)(smem + Cfg::O_XT);
    E* sP = (E*)(smem + Cfg::O_P);
    E* sUT = (E*)(smem + Cfg::O_UT);
    E* sUHT = (E*)(smem + Cfg::O_UHT);
    E* sO = (E*)(smem + Cfg::O_O);

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63;
    const int lr = l & 15, lq = l >> 4;

    // ---- which (head, column slice) this workgroup owns --------------------
    // Dispatch places workgroup i on XCD i % 8; give all slices of a head the
    // same XCD so their shared q and k reads hit one L2.
    const int total = prm.BH * prm.n_slices;
    int pidx = blockIdx.x;
    if ((total & 7) == 0) pidx = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
    const int bh = pidx / prm.n_slices;
    const int slice = pidx - bh * prm.n_slices;
    const int v0 = slice * NV;
    const SeqRange sr = seq_range(prm.cu, prm.L, prm.H, bh);
    const int64_t L = sr.len;
    const int DV = prm.DV;
    // chunks of this span that hold tokens of this head (fewer than the span's
    // for a packed sequence that ends early)
    int64_t left = (L + C - 1) / C - prm.c0;
    const int ncs = (int)(left < 0 ? 0 : (left < prm.ncs ? left : prm.ncs));

    if (w >= NWC) {
        // ======================= data waves ==================================
        // Chunk x travels HBM -> registers (set x % 2) -> LDS slot x % 2.  In
        // iteration c (compute chunk c) a data wave writes chunk c+1's
        // registers to slot (c+1) % 2 (free since the compute waves left it
        // at the end of chunk c-1) before the first barrier, stores o of
        // chunk c-1 (its own LDS tile of two) before the second, and loads
        // chunk c+3 into the set just emptied before the third, so each
        // barrier interval carries a share of the traffic (the compute
        // waves' own q requests go out at the end of the first).  Past the last chunk the
        // last one is loaded again, and o pieces beyond the tile go past the
        // buffer end.
        // linear attention reads no record: k and the v slice only
        constexpr int NPIECE = LA ? Cfg::NKP + Cfg::NVP : Cfg::NPIECE;
        constexpr int NL = (NPIECE + NWP - 1) / NWP;
        constexpr int PPO = NV * ESZ / 16, NPO = C * PPO;  // o pieces per chunk
        constexpr int NS = (NPO + 64 * NWP - 1) / (64 * NWP);
        const int pw = w - NWC;
        typedef int v4i __attribute__((ext_vector_type(4)));
        const int64_t hq = sr.base * DK * ESZ, hv = sr.base * DV * ESZ;
        const char* recs = (const char*)prm.ws + (int64_t)bh * prm.ncs * RL.bytes;
        const __amdgpu_buffer_rsrc_t orsrc =
            make_rsrc((const char*)prm.o + hv, (uint32_t)(L * DV * ESZ));
        // piece j of this wave: source (1 k, 2 v, 3 record), per-lane source
        // offset within the chunk, per-lane LDS offset within a slot (~0u:
        // the sink)
        int src[NL];
        uint32_t goff[NL], loff[NL];
#pragma unroll
        for (int j = 0; j < NL; ++j) {
            const int i0 = pw + NWP * j;
            const int i = i0 < NPIECE ? i0 : pw;
            int sidx;
            uint32_t g, d;
            if (i < Cfg::NKP) {
                // k: rows of DK elements, 16-byte lanes
                const int p = i;
                constexpr int LPR = DK * ESZ / 16, RPP = 64 / LPR;
                const int r = p * RPP + l / LPR, cc = (l % LPR) * (16 / ESZ);
                sidx = 1;
                g = (r * DK + cc) * ESZ;
                d = Cfg::O_SK + (r * PK + cc) * ESZ;
            } else if (i < Cfg::NKP + Cfg::NVP) {
                const int p = i - Cfg::NKP;
                constexpr int LPR = NV * ESZ / 16, RPP = 64 / LPR;
                const int r = p * RPP + l / LPR, cc = (l % LPR) * (16 / ESZ);
                sidx = 2;
                g = (r * DV + v0 + cc) * ESZ;
                d = Cfg::O_SV + (r * PV + cc) * ESZ;
            } else if (i < Cfg::NKP + Cfg::NVP + Cfg::NTP) {
                // T': [C][C] row-major in the record
                const int p = i - Cfg::NKP - Cfg::NVP;
                constexpr int LPR = C * ESZ / 16, RPP = 64 / LPR;
                const int r = p * RPP + l / LPR, cc = (l % LPR) * (16 / ESZ);
                sidx = 3;
                g = RL.tb + (r * C + cc) * ESZ;
                d = Cfg::O_STB + (r * PC + cc) * ESZ;
            } else {
                sidx = 3;
                g = RL.rs + l * 16;
                d = Cfg::O_SRS + l * 16;
            }
            src[j] = __builtin_amdgcn_readfirstlane(sidx);
            goff[j] = g;
            loff[j] = i0 < NPIECE ? d : ~0u;
        }
        struct DSet {
            v4i v[NL];
        };
        // Buffer resources start at the chunk and end at the sequence end
        // (or the record end), so tokens past L read as zeros.
        auto fetch = [&](DSet& st, int cs) {
            // wave-uniform by construction; said so, the buffer resources
            // below are scalar (no per-lane loop over resource values)
            cs = __builtin_amdgcn_readfirstlane(cs < ncs ? cs : ncs - 1);
            const int64_t t0 = (prm.c0 + cs) * C;
            const __amdgpu_buffer_rsrc_t rk =
                make_rsrc((const char*)prm.k + hq + t0 * DK * ESZ, (uint32_t)((L - t0) * DK * ESZ));
            const __amdgpu_buffer_rsrc_t rv =
                make_rsrc((const char*)prm.v + hv + t0 * DV * ESZ, (uint32_t)((L - t0) * DV * ESZ));
            const __amdgpu_buffer_rsrc_t rr = make_rsrc(recs + (int64_t)cs * RL.bytes, RL.bytes);
#pragma unroll
            for (int j = 0; j < NL; ++j) {
                const __amdgpu_buffer_rsrc_t res = src[j] == 1 ? rk : src[j] == 2 ? rv : rr;
                st.v[j] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(res, (int)goff[j], 0, 0));
            }
        };
        auto put = [&](const DSet& st, int cs) {
            char* slot = ring + (cs & 1) * SLOT;
            char* sink = smem + Cfg::O_SINK + l * 16;
#pragma unroll
            for (int j = 0; j < NL; ++j) {
                v4i x = st.v[j];
                if constexpr (LA) {
                    // phi(k) on the way into the ring
                    if (src[j] == 1) {
                        if constexpr (ESZ == 2)
                            x = __builtin_bit_cast(v4i, elu1(__builtin_bit_cast(bf16x8, x)));
                        else
                            x = __builtin_bit_cast(v4i, elu1(__builtin_bit_cast(floatx4, x)));
                    }
                }
                *(v4i*)(loff[j] == ~0u ? sink : slot + loff[j]) = x;
            }
        };
        // o tile of chunk cs (cs < 0: every store falls past the buffer end)
        auto store_o = [&](int cs) {
            const int64_t t0 = (prm.c0 + cs) * C;
            const E* so = sO + (cs & 1) * C * PV;
#pragma unroll
            for (int k = 0; k < NS; ++k) {
                const int i = (tid - 64 * NWC) + 64 * NWP * k;
                const int ic = i < NPO ? i : 0;
                const int r = ic / PPO, cc = (ic % PPO) * (16 / ESZ);
                const uint4 val = *(const uint4*)(so + r * PV + cc);
                const uint32_t off = (cs >= 0 && i < NPO) ? (uint32_t)(((t0 + r) * DV + v0 + cc) * ESZ)
                                                          : 0x80000000u;
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i, val), orsrc, (int)off, 0, 0);
            }
        };
        // These waves meet the compute waves' barriers with a bare s_barrier
        // (a full __syncthreads would also wait for the loads in flight); the
        // empty asm statements keep LDS accesses on their side of it.
        auto bare_barrier = []() {
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        };
        // chunk x: loads issued in iteration x-3 into set x % 2, written to
        // its slot in iteration x-1, used by the compute waves in iteration x
        DSet s0, s1;
        if (ncs > 0) {
            fetch(s0, 0);
            store_o(-1);
            fetch(s1, 1);
            store_o(-1);
            put(s0, 0);
            fetch(s0, 2);
            store_o(-1);
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
        bare_barrier();
        auto iteration = [&](DSet& nx, int cs) {
            put(nx, cs + 1);
            __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): slot writes done
            bare_barrier();                      // 1
            store_o(cs - 1);
            __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): o reads done
            bare_barrier();                      // 2
            fetch(nx, cs + 3);
            bare_barrier();                      // 3
        };
        for (int cs = 0; cs < ncs; cs += 2) {
            iteration(s1, cs);
            if (cs + 1 >= ncs) break;
            iteration(s0, cs + 1);
        }
        if (ncs > 0) store_o(ncs - 1);
        return;
    }

    // ========================= compute waves =====================================
    // Tiles (X, Q S, u, o): wave w owns (Rw, vb) for vb = jw, jw + NWC/NB,
    // ... < NVB, with jw = w / NB; successive groups of NB waves take the row
    // blocks in opposite orders, so the two compute waves that share a SIMD
    // (w and w + 4) hold a short and a long row of the triangular products.
    // State tile t: cb = t % NCB, vb = t / NCB.
    static_assert(NWC % NB == 0, "whole groups of NB waves");
    const int jw = w / NB;
    const int Rw = (jw & 1) ? NB - 1 - w % NB : w % NB;
    static_assert(NCB % CBW == 0 && NSW <= NWC, "state tile blocks");
    floatx4 Sreg[CBW][NVB];
#pragma unroll
    for (int a = 0; a < CBW; ++a)
#pragma unroll
        for (int b = 0; b < NVB; ++b) {
            Sreg[a][b] = floatx4{0.f, 0.f, 0.f, 0.f};
            if (w < NSW) {
                const int cb = CBW * w + a;
                if (prm.S_in) {
                    const float* s0 = prm.S_in + (int64_t)bh * DK * DV + v0;
#pragma unroll
                    for (int e = 0; e < 4; ++e) Sreg[a][b][e] = s0[(16 * cb + 4 * lq + e) * DV + 16 * b + lr];
                }
                store_acc_transposed<E>(sST + (16 * b) * PK + 16 * cb, PK, Sreg[a][b]);
            }
        }
    // blocks of P above the diagonal stay zero
    for (int i = tid; i < C * PC; i += 64 * NWC) sP[i] = from_f32<E>(0.f);
    // linear attention: u and the state update's operand are X itself, and
    // the u areas hold the normalizer instead: z_prev of two chunks [2][DK]
    // and each wave group's share of the row sums of P plus phi(q) z_prev
    // [NWC/NB][C]
    E* sUTc = LA ? sXT : sUT;
    E* sUHTc = LA ? sXT : sUHT;
    float* sZ = (float*)(smem + Cfg::O_UT);
    float* sRow = sZ + 2 * DK;
    static_assert(!LA || (2 * DK + (NWC / NB) * C) * 4 <= NV * PC * ESZ, "normalizer in LDS");
    // z lives in LDS only (z_prev of chunk c in half c % 2)
    if constexpr (LA) {
        for (int i = tid; i < DK; i += 64 * NWC) sZ[i] = prm.z_in ? prm.z_in[(int64_t)bh * DK + i] : 0.f;
    }
    __syncthreads();

    // Every tile and P block of wave w has row block Rw.  q rows Rw come
    // straight from memory as the B operand of (Q S)^T and of P: lane l
    // holds q[16 Rw + l%16][KS kk + W (l/16) .. + W].
    // Chunk x lands in register set x % 2, loaded two chunks ahead (past the
    // last chunk the last one is loaded again); rows past token L read zero.
    constexpr int NKA = DK / KS;
    typedef typename F::T FT;
    struct QSet {
        FT f[NKA];
    };
    const char* qhead = (const char*)prm.q + sr.base * DK * ESZ;
    auto load_q = [&](QSet& qs, int cs) {
        // wave-uniform (scalar buffer resources, as in the data waves)
        cs = __builtin_amdgcn_readfirstlane(cs < ncs ? cs : ncs - 1);
        const int64_t t0 = (prm.c0 + cs) * C;
        const __amdgpu_buffer_rsrc_t r =
            make_rsrc(qhead + t0 * DK * ESZ, (uint32_t)((L - t0) * DK * ESZ));
#pragma unroll
        for (int kk = 0; kk < NKA; ++kk) {
            const int off = ((16 * Rw + lr) * DK + KS * kk + W * lq) * ESZ;
            qs.f[kk] = __builtin_bit_cast(FT, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
        }
    };

    floatx4 oacc[ITL];
    constexpr bool norm_qk = NORM;
    auto chunk = [&](int cs, QSet& qc) {
        const char* slot = ring + (cs & 1) * SLOT;
        const E* sK = (const E*)(slot + Cfg::O_SK);
        const E* sV = (const E*)(slot + Cfg::O_SV);
        const E* sTb = (const E*)(slot + Cfg::O_STB);
        const float* rs = (const float*)(slot + Cfg::O_SRS);  // g, e^g, e^{g_n-g}, e^{g_n}

        // ---------------- phase 1: X, Q S, P ----------------
        // S^T rows vb serve X and Q S, read once per wave.
        // KDA_IN_NORM_QK: q and k arrive raw.  1/|q_r| comes from the q
        // fragments (summed over the four lanes that hold a row), 1/|k_t|
        // from the record; both scale the fp32 products.
        float qinv = 1.f;  // 1/|q| of row 16 Rw + lr
        // LA: this wave's share of phi(q_r) . z_prev, row 16 Rw + lr (the
        // waves of a row block split the channel steps kk between them)
        float qz = 0.f;
        if constexpr (LA) {
            const float* zp = sZ + (cs & 1) * DK;
#pragma unroll
            for (int kk = 0; kk < NKA; ++kk)
                if (kk % (NWC / NB) == jw)
#pragma unroll
                    for (int e = 0; e < W; ++e)
                        qz += to_f32(qc.f[kk][e]) * zp[KS * kk + W * lq + e];
            qz = sum_over_lq(qz);
        }
        if constexpr (norm_qk) {
            float sq = 0.f;
#pragma unroll
            for (int kk = 0; kk < NKA; ++kk) sq += frag_sumsq(qc.f[kk]);
            qinv = inv_norm(sum_over_lq(sq));
        }
        // P blocks (Rw, J) for J = jw, jw + NWC / NB, ... <= Rw:
        // lane holds (Q K^T)[r = 16 Rw + lr][j = 16J + 4lq + e]
        const int r = 16 * Rw + lr;
        const float gr = LA ? 0.f : rs[r];
        float rsum = 0.f;  // LA: this wave's share of sum_j P_rj
        auto p_block = [&](int J, const FT* kj) {
            floatx4 pa = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < NKA; ++kk) pa = F::mma(pa, kj[kk], qc.f[kk]);
            floatx4 gj = {0.f, 0.f, 0.f, 0.f};
            if constexpr (!LA) gj = *(const floatx4*)(rs + 16 * J + 4 * lq);
            floatx4 sc = {qinv, qinv, qinv, qinv};
            // raw k: 1/|k_j| from the record
            if constexpr (norm_qk) sc *= *(const floatx4*)(rs + 3 * C + 16 * J + 4 * lq);
            floatx4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = 16 * J + 4 * lq + e;
                if constexpr (LA) {
                    v[e] = (J < Rw || j <= r) ? pa[e] : 0.f;
                    rsum += v[e];
                } else {
                    v[e] = (J < Rw || j <= r) ? pa[e] * sc[e] * exp_neg(gr - gj[e]) : 0.f;
                }
            }
            st4<E>(sP + r * PC + 16 * J + 4 * lq, v);
        };
        // blocks below the diagonal, each with its own K rows
        for (int J = jw; J < Rw; J += NWC / NB) {
            FT kj[NKA];
            const E* pkj = sK + (16 * J + lr) * PK + W * lq;
#pragma unroll
            for (int kk = 0; kk < NKA; ++kk) kj[kk] = F::load(pkj + KS * kk);
            p_block(J, kj);
        }
        // K rows Rw serve the diagonal block (if this wave owns it) and X,
        // read once
        const bool diag = jw <= Rw && (Rw - jw) % (NWC / NB) == 0;
        FT kr[NKA];
        if (!LA || diag) {
            const E* pkr = sK + (16 * Rw + lr) * PK + W * lq;
#pragma unroll
            for (int kk = 0; kk < NKA; ++kk) kr[kk] = F::load(pkr + KS * kk);
        }
        if (diag) p_block(Rw, kr);
        if constexpr (LA) {
            rsum = sum_over_lq(rsum);
            if (lq == 0) sRow[jw * C + r] = rsum + qz;
        }
        // S^T rows vb serve X and Q S, read once per wave.
#pragma unroll
        for (int i = 0; i < ITL; ++i) {
            const int vb = jw + (NWC / NB) * i;
            if (vb < NVB) {
                const int R = Rw;
                FT st[NKA];
                const E* pst = sST + (16 * vb + lr) * PK + W * lq;
#pragma unroll
                for (int kk = 0; kk < NKA; ++kk) st[kk] = F::load(pst + KS * kk);
                if constexpr (LA) {
                    // X = V: no delta term; Q S kept for o
                    floatx4 qs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kk = 0; kk < NKA; ++kk) qs = F::mma(qs, st[kk], qc.f[kk]);
                    oacc[i] = qs;
                    floatx4 xv;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        xv[e] = to_f32(sV[(16 * R + 4 * lq + e) * PV + 16 * vb + lr]);
                    store_acc_transposed<E>(sXT + (16 * vb) * PC + 16 * R, PC, xv);
                    continue;
                }
                // (K S)[16R + 4lq + e][16vb + lr] -> X = V - e^g (K S), stored transposed
                floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < NKA; ++kk) acc = F::mma(acc, kr[kk], st[kk]);
                // transposed: lane holds (Q S)[16R + lr][16vb + 4lq + e], times e^{g_r}
                floatx4 qs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < NKA; ++kk) qs = F::mma(qs, st[kk], qc.f[kk]);
                oacc[i] = qs * (rs[C + 16 * R + lr] * qinv);
                floatx4 eg = *(const floatx4*)(rs + C + 16 * R + 4 * lq);
                if constexpr (norm_qk) eg *= *(const floatx4*)(rs + 3 * C + 16 * R + 4 * lq);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    acc[e] = to_f32(sV[(16 * R + 4 * lq + e) * PV + 16 * vb + lr]) - eg[e] * acc[e];
                store_acc_transposed<E>(sXT + (16 * vb) * PC + 16 * R, PC, acc);
            }
        }
        load_q(qc, cs + 2);
        __syncthreads();

        // ---------------- phase 2: u = T' X ----------------
#pragma unroll
        for (int i = 0; i < ITL; ++i) {
            const int vb = jw + (NWC / NB) * i;
            if (!LA && vb < NVB) {
                const int R = Rw;
                const int K = ((16 * (R + 1) + KS - 1) / KS) * KS;
                floatx4 acc = {0.f, 0.f, 0.f, 0.f};
                acc = mma_block<E>(acc, sTb + (16 * R) * PC, PC, sXT + (16 * vb) * PC, PC, K);
                store_acc_transposed<E>(sUT + (16 * vb) * PC + 16 * R, PC, acc);
                // the state update takes raw K^T: e^{g_n-g_t} / |k_t| on u
                floatx4 egn = *(const floatx4*)(rs + 2 * C + 16 * R + 4 * lq);
                if constexpr (norm_qk) egn *= *(const floatx4*)(rs + 3 * C + 16 * R + 4 * lq);
                store_acc_transposed<E>(sUHT + (16 * vb) * PC + 16 * R, PC, acc * egn);
            }
        }
        __syncthreads();

        // ---------------- phase 3: S update, o ----------------
        const float gnv = LA ? 1.f : rs[2 * C - 1];  // e^{g_n}
        if (w < NSW) {
            constexpr int NKP = C / KS;
            typename F::T kt[CBW][NKP];
#pragma unroll
            for (int a = 0; a < CBW; ++a)
#pragma unroll
                for (int kk = 0; kk < NKP; ++kk) kt[a][kk] = load_frag_tr(sK, PK, KS * kk, 16 * (CBW * w + a));
#pragma unroll
            for (int b = 0; b < NVB; ++b) {
                const E* pu = sUHTc + (16 * b + lr) * PC + W * lq;
                typename F::T uf[NKP];
#pragma unroll
                for (int kk = 0; kk < NKP; ++kk) uf[kk] = F::load(pu + KS * kk);
#pragma unroll
                for (int a = 0; a < CBW; ++a) {
                    floatx4 acc = Sreg[a][b] * gnv;
#pragma unroll
                    for (int kk = 0; kk < NKP; ++kk) acc = F::mma(acc, kt[a][kk], uf[kk]);
                    Sreg[a][b] = acc;
                    store_acc_transposed<E>(sST + (16 * b) * PK + 16 * (CBW * w + a), PK, acc);
                }
            }
            if constexpr (LA) {
                // z += phi(K)^T 1 over this chunk's valid tokens; z_prev of
                // the next chunk goes to the other half of sZ
                const int64_t t0 = (prm.c0 + cs) * C;
                const int n = (int)(L - t0 < C ? L - t0 : C);
                const float* zp = sZ + (cs & 1) * DK;
                float* zn = sZ + ((cs + 1) & 1) * DK;
#pragma unroll
                for (int a = 0; a < CBW; ++a) {
                    const int c0 = 16 * (CBW * w + a) + 4 * lq;
                    floatx4 acc = *(const floatx4*)(zp + c0);
#pragma unroll
                    for (int kk = 0; kk < NKP; ++kk)
                        acc = F::mma(acc, kt[a][kk], ones_below<E>(KS * kk + W * lq, n));
                    if (lr == 0) *(floatx4*)(zn + c0) = acc;
                }
            }
        }
#pragma unroll
        for (int i = 0; i < ITL; ++i) {
            const int vb = jw + (NWC / NB) * i;
            if (vb < NVB) {
                const int R = Rw;
                const int K = ((16 * (R + 1) + KS - 1) / KS) * KS;
                floatx4 acc = oacc[i];
                acc = mma_block<E>(acc, sUTc + (16 * vb) * PC, PC, sP + (16 * R) * PC, PC, K);
                if constexpr (LA) {
                    // lane holds row 16R + lr: divide by phi(q_r) z_r, the sum
                    // of the row block's waves' shares
                    float den = 0.f;
#pragma unroll
                    for (int g = 0; g < NWC / NB; ++g) den += sRow[g * C + 16 * R + lr];
                    acc = acc * (1.f / den);
                }
                st4<E>(sO + (cs & 1) * C * PV + (16 * R + lr) * PV + 16 * vb + 4 * lq, acc);
            }
        }
        __syncthreads();
    };
    QSet qa, qb;
    if (ncs > 0) {
        load_q(qa, 0);
        load_q(qb, 1);
    }
    for (int cs = 0; cs < ncs; cs += 2) {
        chunk(cs, qa);
        if (cs + 1 >= ncs) break;
        chunk(cs + 1, qb);
    }

    if constexpr (LA) {
        // the last chunk's barrier has published z; chunk c wrote half (c+1) % 2
        if (prm.z_out)
            for (int i = tid; i < DK; i += 64 * NWC) prm.z_out[(int64_t)bh * DK + i] = sZ[(ncs & 1) * DK + i];
    }
    // ---- state out --------------------------------------------------------------
    if (prm.S_out && w < NSW) {
        float* so = prm.S_out + (int64_t)bh * DK * DV + v0;
#pragma unroll
        for (int a = 0; a < CBW; ++a)
#pragma unroll
            for (int b = 0; b < NVB; ++b) {
                const int cb = CBW * w + a;
#pragma unroll
                for (int e = 0; e < 4; ++e) so[(16 * cb + 4 * lq + e) * DV + 16 * b + lr] = Sreg[a][b][e];
            }
    }
}

// ---- host-side dispatch -----------------------------------------------------

template <int DK, int NV, int C, typename E>
static hipError_t launch_scalar_cfg(const InterParams& prm, hipStream_t stream) {
    typedef ScalarInterCfg<DK, NV, C, E> Cfg;
    const int total = prm.BH * prm.n_slices;
    if (prm.linear_attn)
        hipLaunchKernelGGL((kda_inter_scalar_kernel<Cfg, false, true>), dim3(total),
                           dim3(Cfg::NT), 0, stream, prm);
    else if (prm.flags & KDA_IN_NORM_QK)
        hipLaunchKernelGGL((kda_inter_scalar_kernel<Cfg, true, false>), dim3(total),
                           dim3(Cfg::NT), 0, stream, prm);
    else
        hipLaunchKernelGGL((kda_inter_scalar_kernel<Cfg, false, false>), dim3(total),
                           dim3(Cfg::NT), 0, stream, prm);
    return hipGetLastError();
}

hipError_t launch_inter_scalar(InterParams prm, int dk, int qkv_bf16, int nv, hipStream_t stream) {
    if (prm.BH == 0) return hipSuccess;
    prm.n_slices = prm.DV / nv;
#define KDA_CASE(DK_, NV_, C_, E_)                                      \
    if (dk == DK_ && nv == NV_ && (qkv_bf16 != 0) == (sizeof(E_) == 2)) \
        return launch_scalar_cfg<DK_, NV_, C_, E_>(prm, stream);
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
