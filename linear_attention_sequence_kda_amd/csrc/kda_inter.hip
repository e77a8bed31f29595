// kda_inter.hip -- inter-chunk kernel of the two-kernel chunkwise prefill
// (gfx950 / MI355X): the part of the method that is serial over chunks.
//
// "22,580: From GPT-2 to Kimi K3" (yichencityu.github.io), section 6.3: one
// state is carried from chunk to chunk; per chunk, with the factors the
// intra-chunk kernel left in the chunk's record,
//
//   u = U - W S
//   O = (Q * e^g) S + P u
//   S <- diag(e^{g_n}) S + (K * e^{g_n - g})^T u
//
// (section 08 and 9.1 for the decay; with one decay per token the e^g factors
// are scalars per row, applied to Q S and to u, and K is the stored input).
//
// One workgroup owns one (b, h) head and a slice of NV state columns
// (columns of S evolve independently, so slices never talk) and walks the
// chunks in order.  Its fp32 state slice lives in registers as 16x16 blocks
// spread over eight compute waves, with a transposed operand copy in LDS.
//
// Eight more waves only move data.  They keep two chunks' records in flight
// in registers (a chunk's loads cost about one and a half microseconds of
// latency, several chunks' worth of compute) and write each into one half of
// a two-slot LDS ring one chunk ahead of use (the record is stored in 1 KiB
// wave pieces in exactly the order the compute waves read their MFMA
// fragments, so each piece is one load and one LDS write), and they write the
// previous chunk's o tile to HBM.  The compute waves never issue a global
// memory instruction inside the loop.  Per chunk:
//   phase A  u tiles: u = U - W S        (then u, and e^{g_n-g} u, to LDS)
//            o tiles: o = (Q S) e^g      (kept in registers)
//   phase B  S tiles: S = e^{g_n} S + K^T u  (new operand copy to LDS)
//            o tiles: o += P u, to an LDS tile
// with one barrier after each phase; the data waves wait for their copies
// between the two barriers.  o tiles are computed transposed (lane = one
// token, four adjacent columns); the o store goes through a buffer resource
// bounded by the sequence end, so the ragged last chunk needs no branch.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

template <int DK_, int NV_, int C_, typename E_, bool KDA_>
struct InterCfg {
    typedef E_ E;
    static constexpr int DK = DK_, NV = NV_, C = C_;
    static constexpr bool KDA = KDA_;
    static constexpr int NB = C / 16, NCB = DK / 16, NVB = NV / 16;
    static constexpr int ESZ = sizeof(E);
    static constexpr int KS = 64 / ESZ;    // MFMA k step (16-byte lane pieces x 4)
    static constexpr int NKA = DK / KS, NKP = C / KS;
    static constexpr int PADE = 32 / ESZ;
    static constexpr int PK = DK + PADE;   // S^T operand copy [NV][DK]
    static constexpr int PC = C + PADE;    // u^T [NV][C]
    static constexpr int PO = NV + PADE;   // o tile [C][NV]
    static constexpr int NWC = 8;          // compute waves
    static constexpr int NWP = 8;          // data waves
    // chunks the data waves keep in flight in registers: the pass waits on
    // memory latency, so each chunk takes about latency / NSET
    static constexpr int NSET = 3;
    static constexpr int NT = 64 * (NWC + NWP);
    // Phase-A items: (role, R, column group) with role u (u = U - W S) or o
    // (o = Q S ...), R a 16-token block, and the NVB column blocks of the
    // slice split into NG groups of VG blocks, so one wave reads a W or Q row
    // block once and uses it for every column block of its group.
    static constexpr int NG = (2 * NB >= NWC || NVB == 1) ? 1 : (NWC / (2 * NB) < NVB ? NWC / (2 * NB) : NVB);
    static constexpr int VG = NVB / NG;
    static constexpr int NIA = 2 * NB * NG;
    // State items: (cb, column group): K^T row block cb for SG column blocks.
    static constexpr int NGS = (NCB >= NWC || NVB == 1) ? 1 : (NWC / NCB < NVB ? NWC / NCB : NVB);
    static constexpr int SG = NVB / NGS;
    static constexpr int NIS = NCB * NGS;
    static_assert(NIA <= NWC && NIS <= NWC, "one phase-A item and one state item per wave");
    static_assert(VG * NG == NVB && SG * NGS == NVB, "column groups");
    // ring slot: 1 KiB pieces W [NB][NKA], Q [NB][NKA], P [NB][NKP],
    // K^T [NCB][NKP], U [NB][NUP], decay scalars
    static constexpr int PF = 16 / (4 * ESZ);            // U blocks per lane piece
    static constexpr int NUP = (NVB + PF - 1) / PF;      // U pieces per R in a slice
    static constexpr int P_W = 0, P_Q = P_W + NB * NKA, P_P = P_Q + NB * NKA;
    static constexpr int P_KT = P_P + NB * NKP, P_U = P_KT + NCB * NKP;
    static constexpr int P_SC = P_U + NB * NUP;          // decay scalars (gam | rs)
    static constexpr int NPIECE = P_SC + 1;
    static constexpr int O_SC = P_SC * 1024;
    static constexpr int SLOT = NPIECE * 1024;
    // LDS: ring, a 1 KiB sink for the data waves' padding pieces, ...
    static constexpr int O_RING = 0;
    static constexpr int O_SINK = O_RING + 2 * SLOT;
    static constexpr int O_ST = O_SINK + 1024;
    static constexpr int O_UT = O_ST + NV * PK * ESZ;
    static constexpr int O_UHT = O_UT + NV * PC * ESZ;
    static constexpr int O_O = O_UHT + (KDA ? 0 : NV * PC * ESZ);
    static constexpr int LDS_BYTES = O_O + C * PO * ESZ;
    static_assert(DK % 32 == 0 && NV % 16 == 0 && (C == 32 || C == 64), "tile shape");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget of one gfx950 CU");
};

template <class Cfg>
__global__ void __launch_bounds__(Cfg::NT) kda_inter_kernel(InterParams prm) {
    typedef typename Cfg::E E;
    typedef Frag<E> F;
    typedef typename F::T FT;
    constexpr int DK = Cfg::DK, NV = Cfg::NV, C = Cfg::C, NB = Cfg::NB;
    constexpr bool KDA = Cfg::KDA;
    constexpr int PK = Cfg::PK, PC = Cfg::PC, PO = Cfg::PO, NCB = Cfg::NCB, NVB = Cfg::NVB;
    constexpr int NWC = Cfg::NWC, NWP = Cfg::NWP, NG = Cfg::NG, VG = Cfg::VG, NIA = Cfg::NIA;
    constexpr int NGS = Cfg::NGS, SG = Cfg::SG, NIS = Cfg::NIS;
    constexpr int ESZ = Cfg::ESZ, W = F::W, KS = F::KS;
    constexpr int NKA = Cfg::NKA, NKP = Cfg::NKP, PF = Cfg::PF, NUP = Cfg::NUP;
    constexpr int SLOT = Cfg::SLOT, O_SC = Cfg::O_SC;
    static_assert(KS == Cfg::KS, "k step");

    __shared__ __attribute__((aligned(16))) char smem[Cfg::LDS_BYTES];
    char* ring = smem + Cfg::O_RING;
    E* sST = (E*)(smem + Cfg::O_ST);
    E* sUT = (E*)(smem + Cfg::O_UT);
    E* sUHT = (E*)(smem + Cfg::O_UHT);
    E* sO = (E*)(smem + Cfg::O_O);

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63;
    const int lr = l & 15, lq = l >> 4;

    // ---- which (head, column slice) this workgroup owns --------------------
    // Dispatch places workgroup i on XCD i % 8; give all slices of a head the
    // same XCD so their shared record reads hit one L2.
    const int total = prm.BH * prm.n_slices;
    int pidx = blockIdx.x;
    if ((total & 7) == 0) pidx = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
    const int bh = pidx / prm.n_slices;
    const int slice = pidx - bh * prm.n_slices;
    const int v0 = slice * NV;
    const SeqRange sr = seq_range(prm.cu, prm.L, prm.H, bh);
    const int64_t L = sr.len;
    const int DV = prm.DV;
    const RecLayout rl = rec_layout(DK, DV, C, ESZ, KDA);
    const char* recs = (const char*)prm.ws + (int64_t)bh * prm.ncs * rl.bytes;
    // chunks of this span that hold tokens of this head (fewer than the span's
    // for a packed sequence that ends early)
    int64_t left = (L + C - 1) / C - prm.c0;
    const int ncs = (int)(left < 0 ? 0 : (left < prm.ncs ? left : prm.ncs));

    if (w >= NWC) {
        // ======================= data waves ==================================
        // Chunk x travels HBM -> registers (set x % 2) -> LDS slot x % 2.
        // In iteration c a data wave writes chunk c+1's registers to slot
        // (c+1) % 2 (free since the compute waves left it at the end of chunk
        // c-1), loads chunk c+3 into the set just emptied and stores o of
        // chunk c-1.  Past the last chunk it re-reads the last record, and o
        // pieces beyond the tile go past the buffer end.
        constexpr int NL = (Cfg::NPIECE + NWP - 1) / NWP;  // 1 KiB pieces per wave
        constexpr int PPR = NV * ESZ / 16, NPC = C * PPR;   // o pieces per chunk
        constexpr int NS = (NPC + 64 * NWP - 1) / (64 * NWP);
        const int pw = w - NWC;
        const __amdgpu_buffer_rsrc_t orsrc =
            make_rsrc((const char*)prm.o + sr.base * DV * ESZ, (uint32_t)(L * DV * ESZ));
        const int gp0 = (slice * NVB) / PF;  // first U piece column of the slice
        // record and ring offsets of this wave's j-th piece (wave-uniform;
        // pieces past the list re-read a valid piece and land in the sink)
        uint32_t pg[NL], pl[NL];
#pragma unroll
        for (int j = 0; j < NL; ++j) {
            const int i0 = pw + NWP * j;
            const int i = i0 < Cfg::NPIECE ? i0 : pw;
            uint32_t g;
            if (i < Cfg::P_Q) g = rl.w + (i - Cfg::P_W) * 1024;
            else if (i < Cfg::P_P) g = rl.qt + (i - Cfg::P_Q) * 1024;
            else if (i < Cfg::P_KT) g = rl.p + (i - Cfg::P_P) * 1024;
            else if (i < Cfg::P_U) g = rl.kt + (i - Cfg::P_KT) * 1024;
            else if (i < Cfg::P_SC) {
                const int u = i - Cfg::P_U, R = u / NUP, jj = u % NUP;
                g = rl.ut + (R * (DV / (16 * PF)) + gp0 + jj) * 1024;
            } else {
                g = KDA ? rl.gam : rl.rs;
            }
            pg[j] = __builtin_amdgcn_readfirstlane(g);
            pl[j] = __builtin_amdgcn_readfirstlane(i0 < Cfg::NPIECE ? i0 * 1024 : -1);
        }
        const uint32_t l16 = l * 16;
        typedef int v4i __attribute__((ext_vector_type(4)));
        struct DSet {
            v4i v[NL];
        };
        // Loads through a buffer resource over the record (the only vector
        // register involved is the lane offset).
        auto fetch = [&](DSet& st, int cs) {
            // wave-uniform by construction; said so, the buffer resources
            // below are scalar (no per-lane loop over resource values)
            cs = __builtin_amdgcn_readfirstlane(cs < ncs ? cs : ncs - 1);
            const __amdgpu_buffer_rsrc_t rr = make_rsrc(recs + (int64_t)cs * rl.bytes, rl.bytes);
#pragma unroll
            for (int j = 0; j < NL; ++j)
                st.v[j] = __builtin_bit_cast(
                    v4i, __builtin_amdgcn_raw_buffer_load_b128(rr, (int)l16, (int)pg[j], 0));
        };
        auto put = [&](const DSet& st, int cs) {
            char* slot = ring + (cs & 1) * SLOT;
            char* sink = smem + Cfg::O_SINK;
#pragma unroll
            for (int j = 0; j < NL; ++j) *(v4i*)((pl[j] == 0xffffffffu ? sink : slot + pl[j]) + l16) = st.v[j];
        };
        // o tile of chunk cs (cs < 0: every store falls past the buffer end)
        auto store_o = [&](int cs) {
            const int64_t t0 = (prm.c0 + cs) * C;
#pragma unroll
            for (int k = 0; k < NS; ++k) {
                const int i = (tid - 64 * NWC) + 64 * NWP * k;
                const int ic = i < NPC ? i : 0;
                const int r = ic / PPR, cc = (ic % PPR) * (16 / ESZ);
                const uint4 val = *(const uint4*)(sO + r * PO + cc);
                const uint32_t off = (cs >= 0 && i < NPC) ? (uint32_t)(((t0 + r) * DV + v0 + cc) * ESZ)
                                                          : 0x80000000u;
                typedef int v4i __attribute__((ext_vector_type(4)));
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i, val), orsrc, (int)off, 0, 0);
            }
        };
        // These waves meet the compute waves' barriers with a bare s_barrier:
        // a full __syncthreads would also wait for the loads in flight.  The
        // empty asm statements keep the compiler from moving LDS accesses
        // across the barriers.
        auto bare_barrier = []() {
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        };
        // chunk x: loads issued in iteration x-NSET-1 into set x % NSET,
        // written to its slot in iteration x-1, used by the compute waves in
        // iteration x
        constexpr int NSET = Cfg::NSET;
        DSet sets[NSET];
        if (ncs > 0) {
#pragma unroll
            for (int j = 0; j < NSET; ++j) fetch(sets[j], j);
            store_o(-1);
            put(sets[0], 0);
            fetch(sets[0], NSET);
            store_o(-1);
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
        bare_barrier();
        // iteration cs: chunk cs+1 is in `nx`, which then takes chunk cs+1+NSET
        auto iteration = [&](DSet& nx, int cs) {
            put(nx, cs + 1);
            fetch(nx, cs + 1 + NSET);
            store_o(cs - 1);
            __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): slot writes, o reads done
            bare_barrier();                      // A
            bare_barrier();                      // B
        };
        for (int c0 = 0; c0 < ncs; c0 += NSET) {
            bool done = false;
#pragma unroll
            for (int j = 0; j < NSET; ++j) {
                if (!done) {
                    iteration(sets[(j + 1) % NSET], c0 + j);
                    done = c0 + j + 1 >= ncs;
                }
            }
            if (done) break;
        }
        if (ncs > 0) store_o(ncs - 1);
        return;
    }

    // ========================= compute waves =====================================
    // phase A: item w < NIA is (role, R, group): role u for w < NB*NG, else o.
    // state: item w < NIS is (cb, group).
    const bool aval = w < NIA;
    const int ai = aval ? w : 0;
    const bool isU = ai < NB * NG;
    const int aR = (isU ? ai : ai - NB * NG) / NG;
    const int avb0 = ((isU ? ai : ai - NB * NG) % NG) * VG;  // first column block
    const bool sval = w < NIS;
    const int si = sval ? w : 0;
    const int scb = si / NGS;
    const int svb0 = (si % NGS) * SG;

    // ---- initial state slice --------------------------------------------------
    // Lane element e of state block g is S[16scb + 4lq + e][v0 + 16(svb0 + g) + lr].
    floatx4 Sreg[SG];
#pragma unroll
    for (int g = 0; g < SG; ++g) Sreg[g] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (prm.S_in && sval) {
        const float* s0 = prm.S_in + (int64_t)bh * DK * DV + v0;
#pragma unroll
        for (int g = 0; g < SG; ++g)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                Sreg[g][e] = s0[(16 * scb + 4 * lq + e) * DV + 16 * (svb0 + g) + lr];
    }
    if (sval) {
#pragma unroll
        for (int g = 0; g < SG; ++g)
            store_acc_transposed<E>(sST + (16 * (svb0 + g)) * PK + 16 * scb, PK, Sreg[g]);
    }
    __syncthreads();

    auto piece = [&](const char* slot, int i) -> FT { return *(const FT*)(slot + i * 1024 + l * 16); };
    floatx4 oacc[VG];
    for (int cs = 0; cs < ncs; ++cs) {
        const char* slot = ring + (cs & 1) * SLOT;
        const float* sc = (const float*)(slot + O_SC);
        // ---------------- phase A ----------------
        if (aval) {
            const int R = aR;
            if (isU) {
                // u[16R + 4lq + e][16vb + lr] = U - sum_c W[r][c] S[c][v]
                FT wf[NKA];
#pragma unroll
                for (int kk = 0; kk < NKA; ++kk) wf[kk] = piece(slot, Cfg::P_W + R * NKA + kk);
                floatx4 ru = {1.f, 1.f, 1.f, 1.f};
                if constexpr (!KDA) ru = *(const floatx4*)(sc + C + 16 * R + 4 * lq);
#pragma unroll
                for (int g = 0; g < VG; ++g) {
                    const int vb = avb0 + g;
                    const E* pst = sST + (16 * vb + lr) * PK + W * lq;
                    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kk = 0; kk < NKA; ++kk) acc = F::mma(acc, wf[kk], F::load(pst + KS * kk));
                    // U block (R, vb): piece gvb / PF - gp0 of row R, half gvb % PF
                    const int gvb = slice * NVB + vb;
                    const int j = gvb / PF - (slice * NVB) / PF;
                    const uint4 q4 = *(const uint4*)(slot + (Cfg::P_U + R * NUP + j) * 1024 + l * 16);
                    floatx4 uf;
                    if constexpr (ESZ == 2) {
                        const int h = gvb % PF;
                        const uint32_t x = h == 0 ? q4.x : q4.z, y = h == 0 ? q4.y : q4.w;
                        uf = floatx4{__uint_as_float(x << 16), __uint_as_float(x & 0xffff0000u),
                                     __uint_as_float(y << 16), __uint_as_float(y & 0xffff0000u)};
                    } else {
                        uf = floatx4{__uint_as_float(q4.x), __uint_as_float(q4.y), __uint_as_float(q4.z),
                                     __uint_as_float(q4.w)};
                    }
                    const floatx4 u = uf - acc;
                    store_acc_transposed<E>(sUT + (16 * vb) * PC + 16 * R, PC, u);
                    if constexpr (!KDA) store_acc_transposed<E>(sUHT + (16 * vb) * PC + 16 * R, PC, u * ru);
                }
            } else {
                // transposed: lane holds (Q S)[r = 16R + lr][v = 16vb + 4lq + e]
                FT qf[NKA];
#pragma unroll
                for (int kk = 0; kk < NKA; ++kk) qf[kk] = piece(slot, Cfg::P_Q + R * NKA + kk);
#pragma unroll
                for (int g = 0; g < VG; ++g) {
                    const int vb = avb0 + g;
                    const E* pst = sST + (16 * vb + lr) * PK + W * lq;
                    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kk = 0; kk < NKA; ++kk) acc = F::mma(acc, F::load(pst + KS * kk), qf[kk]);
                    if constexpr (!KDA) acc *= sc[16 * R + lr];
                    oacc[g] = acc;
                }
            }
        }
        __syncthreads();
        // ---------------- phase B ----------------
        if (sval) {
            const E* ub = KDA ? sUT : sUHT;
            FT kf[NKP];
#pragma unroll
            for (int kk = 0; kk < NKP; ++kk) kf[kk] = piece(slot, Cfg::P_KT + scb * NKP + kk);
            floatx4 gm;
            if constexpr (KDA) gm = *(const floatx4*)(sc + 16 * scb + 4 * lq);
            else gm = floatx4{sc[2 * C], sc[2 * C], sc[2 * C], sc[2 * C]};
#pragma unroll
            for (int g = 0; g < SG; ++g) {
                const int vb = svb0 + g;
                floatx4 acc = Sreg[g] * gm;
                const E* pu = ub + (16 * vb + lr) * PC + W * lq;
#pragma unroll
                for (int kk = 0; kk < NKP; ++kk) acc = F::mma(acc, kf[kk], F::load(pu + KS * kk));
                Sreg[g] = acc;
                store_acc_transposed<E>(sST + (16 * vb) * PK + 16 * scb, PK, acc);
            }
        }
        if (aval && !isU) {
            const int R = aR;
            FT pf[NKP];
#pragma unroll
            for (int kk = 0; kk < NKP; ++kk) pf[kk] = piece(slot, Cfg::P_P + R * NKP + kk);
#pragma unroll
            for (int g = 0; g < VG; ++g) {
                const int vb = avb0 + g;
                floatx4 acc = oacc[g];
                const E* pu = sUT + (16 * vb + lr) * PC + W * lq;
#pragma unroll
                for (int kk = 0; kk < NKP; ++kk)
                    if (KS * kk < 16 * (R + 1)) acc = F::mma(acc, F::load(pu + KS * kk), pf[kk]);
                st4<E>(sO + (16 * R + lr) * PO + 16 * vb + 4 * lq, acc);
            }
        }
        __syncthreads();
    }

    // ---- state out --------------------------------------------------------------
    if (prm.S_out && sval) {
        float* so = prm.S_out + (int64_t)bh * DK * DV + v0;
#pragma unroll
        for (int g = 0; g < SG; ++g)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                so[(16 * scb + 4 * lq + e) * DV + 16 * (svb0 + g) + lr] = Sreg[g][e];
    }
}

// ---- host-side dispatch -----------------------------------------------------

template <int DK, int NV, int C, typename E, bool KDA>
static hipError_t launch_inter_cfg(const InterParams& prm, hipStream_t stream) {
    typedef InterCfg<DK, NV, C, E, KDA> Cfg;
    const int total = prm.BH * prm.n_slices;
    hipLaunchKernelGGL((kda_inter_kernel<Cfg>), dim3(total), dim3(Cfg::NT), 0, stream, prm);
    return hipGetLastError();
}

int chunk_slice_width(int dk, int dv, int qkv_bf16, int64_t BH) {
    // Prefer wide slices while that still gives >= 256 workgroups; else 16.
    if (dk == 64 && qkv_bf16 && BH * (dv / 64) >= 256) return 64;
    if (BH * (dv / 32) >= 256) return 32;
    return 16;
}

hipError_t launch_inter(InterParams prm, int dk, int qkv_bf16, int alpha_mode, int nv,
                        hipStream_t stream) {
    if (prm.BH == 0) return hipSuccess;
    prm.n_slices = prm.DV / nv;
    const bool kda = alpha_mode == KDA_ALPHA_CHANNEL;
#define KDA_CASE(DK_, NV_, C_, E_)                                             \
    if (dk == DK_ && nv == NV_ && (qkv_bf16 != 0) == (sizeof(E_) == 2))        \
        return kda ? launch_inter_cfg<DK_, NV_, C_, E_, true>(prm, stream)     \
                   : launch_inter_cfg<DK_, NV_, C_, E_, false>(prm, stream);
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
