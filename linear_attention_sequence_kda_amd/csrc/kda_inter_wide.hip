// kda_inter_wide.hip -- state pass of the chunkwise prefill for per-channel
// decay with bf16 operands, one workgroup per (head, 64 or 128 state
// columns) (gfx950 / MI355X).
//
// "22,580: From GPT-2 to Kimi K3" (yichencityu.github.io), section 6.3: one
// state is carried from chunk to chunk; per chunk, with the factors the
// intra-chunk kernel left in the chunk's record (section 9.1 for the
// per-channel decay inside them),
//
//   u = U - W S,   O = (Q * e^g) S + P u,   S <- diag(e^{g_n}) S + (K * e^{g_n - g})^T u
//
// Layout.  NWC compute waves (on separate SIMDs) each own NV / NWC columns of
// the state slice and keep them in MFMA accumulator registers, fp32, for the
// whole sequence: lane l holds S[16 cb + 4 (l/16) + i][16 vb + l % 16].  The
// record stores every operand with its contraction index in wide_elem order
// (kda_device.h), in which a pair of 16-row accumulator blocks is an MFMA
// operand as it stands, so
//   u     = U + (-W) S          B operand: S as held (rows = channels)
//   O^T   = S^T Q~^T + u^T P^T  A operands: S and u as held
//   S     = e^{g_n} S + K^T u   B operand: u as held (rows = tokens)
// run on registers alone: no operand copy of S or u goes through LDS and the
// compute waves never wait for each other inside a chunk.  Every compute
// wave reads all of a chunk's W, Q~, K^T and P from LDS, so LDS traffic grows
// with the number of compute waves: two waves of 32 columns each read half of
// what four waves of 16 read, for the same MFMA work.  O^T leaves a lane as
// four adjacent columns of one token, written into a double-buffered LDS o
// tile; the compute waves issue no memory operation inside the loop.
//
// Four data waves copy each chunk's record (1 KiB pieces, the order the
// compute waves read them) from memory through registers into one half of a
// two-slot LDS ring, keeping NSET chunks in flight in registers, and store
// the previous chunk's o tile with 16-byte writes; one barrier per chunk
// hands the slots over.  Tokens past the sequence end have zero records, and
// o stores past it are dropped by the buffer resource's bound.
#include "kda_device.h"
#include "kda_internal.h"

#ifndef KDA_WIDE_NSET16
#define KDA_WIDE_NSET16 5
#endif
#ifndef KDA_WIDE_NSET32
#define KDA_WIDE_NSET32 3
#endif
#ifndef KDA_WIDE_NSET64
#define KDA_WIDE_NSET64 3
#endif
#ifndef KDA_QUAD_NSET
#define KDA_QUAD_NSET 2
#endif

namespace kda {

template <int DK_, int NV_, int NWC_, int NSET_>
struct WideCfg {
    typedef bf16 E;
    static constexpr int DK = DK_, NV = NV_, C = 64;
    static constexpr int NB = C / 16;      // 16-token blocks
    static constexpr int NKA = DK / 32;    // channel k steps
    static constexpr int NKP = C / 32;     // token k steps
    static constexpr int NCB = DK / 16;    // 16-channel blocks
    // compute waves, and data waves filling the workgroup to 8 waves
    static constexpr int NWC = NWC_, NWD = 8 - NWC_;
    static constexpr int NT = 64 * (NWC + NWD);
    static constexpr int NVW = NV / NWC;   // columns of one compute wave
    static constexpr int NVBW = NVW / 16;  // their 16-column blocks
    // U pieces per 16-token block (one piece holds two column blocks; a
    // 16-column slice uses half of one)
    static constexpr int NUR = NV >= 32 ? NV / 32 : 1;
    // ring slot: pieces W [NB][NKA], Q~ [NB][NKA], K^T [NCB][NKP], P [NB][NKP],
    // U [NB][NUR], e^{g_n}
    static constexpr int P_W = 0, P_Q = P_W + NB * NKA, P_K = P_Q + NB * NKA;
    static constexpr int P_P = P_K + NCB * NKP, P_U = P_P + NB * NKP, P_G = P_U + NB * NUR;
    static constexpr int NPIECE = P_G + 1;
    static constexpr int SLOT = NPIECE * 1024;
    // o tile [C][NV] bf16, two of them (chunk parity); rows padded by 16 bytes
    static constexpr int PO = NV + 8;
    static constexpr int O_RING = 0, O_SINK = 2 * SLOT, O_O = O_SINK + 1024;
    static constexpr int LDS_BYTES = O_O + 2 * C * PO * 2;
    static constexpr int NL = (NPIECE + NWD - 1) / NWD;  // pieces per data wave
    static constexpr int NSET = NSET_;                   // chunks in flight in registers
    static_assert(NVW % 16 == 0 && NV % 16 == 0 && DK % 32 == 0, "tile shape");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget of one gfx950 CU");
};

// two fp32 accumulator quads -> one bf16 operand fragment (nearest even)
__device__ __forceinline__ bf16x8 pack_frag(floatx4 a, floatx4 b) {
    bf16x8 r;
    r[0] = (bf16)a[0];
    r[1] = (bf16)a[1];
    r[2] = (bf16)a[2];
    r[3] = (bf16)a[3];
    r[4] = (bf16)b[0];
    r[5] = (bf16)b[1];
    r[6] = (bf16)b[2];
    r[7] = (bf16)b[3];
    return r;
}

// SCAN: the scan form for the chunkwise gradients (no o; the state entering
// a chunk and the chunk's u are written out, InterParams::S_all / u_all).
// REV (with SCAN): reverse records, whose steps add a second product
// S += K2^T U2 (K2^T in the Q~ pieces, U2 in the P pieces).
template <class Cfg, bool SCAN = false, bool REV = false>
__global__ void __launch_bounds__(Cfg::NT) kda_inter_wide_kernel(InterParams prm) {
    typedef bf16 E;
    typedef Frag<E> F;
    constexpr int DK = Cfg::DK, NV = Cfg::NV, C = Cfg::C, NB = Cfg::NB;
    constexpr int NKA = Cfg::NKA, NKP = Cfg::NKP, NCB = Cfg::NCB, NWC = Cfg::NWC;
    constexpr int NWD = Cfg::NWD, NVBW = Cfg::NVBW, NUR = Cfg::NUR, SLOT = Cfg::SLOT;
    constexpr int NL = Cfg::NL;

    __shared__ __attribute__((aligned(16))) char smem[Cfg::LDS_BYTES];
    char* ring = smem + Cfg::O_RING;
    E* sO = (E*)(smem + Cfg::O_O);
    constexpr int PO = Cfg::PO;

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63;
    const int lr = l & 15, lq = l >> 4;

    // ---- which (head, column slice) this workgroup owns --------------------
    // Workgroup i runs on XCD i % 8: the slices of one head share an XCD, so
    // their reads of the head's records meet in one L2.
    const int total = prm.BH * prm.n_slices;
    int pidx = blockIdx.x;
    if ((total & 7) == 0) pidx = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
    const int bh = pidx / prm.n_slices;
    const int slice = pidx - bh * prm.n_slices;
    const int v0 = slice * NV;
    const SeqRange sr = seq_range(prm.cu, prm.L, prm.H, bh);
    const int64_t L = sr.len;
    const int DV = prm.DV;
    const RecLayout rl = rec_layout(DK, DV, C, 2, true);
    const uint32_t rstride = REV ? rev_rec_bytes(DK, DV) : rl.bytes;
    const char* recs = (const char*)prm.ws + (int64_t)bh * prm.ncs * rstride;
    // chunks of this span that hold tokens of this head
    int64_t left = (L + C - 1) / C - prm.c0;
    const int ncs = (int)(left < 0 ? 0 : (left < prm.ncs ? left : prm.ncs));

    // Data and compute waves meet at a bare s_barrier: a full __syncthreads
    // would also wait for the memory operations in flight (the data waves'
    // prefetch, the compute waves' o stores).  The empty asm statements keep
    // LDS accesses on their side of it; LDS traffic is drained explicitly.
    auto bare_barrier = []() {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };

    if (w >= NWC) {
        // ======================= data waves ==================================
        // Chunk x: loaded into register set x % NSET in iteration x-NSET-1,
        // written to ring slot x % 2 in iteration x-1, used in iteration x.
        // Past the last chunk the last record is read again; pieces past the
        // list land in the sink.
        const int dw = w - NWC;
        uint32_t pg[NL], pl[NL];
#pragma unroll
        for (int j = 0; j < NL; ++j) {
            const int i0 = dw + NWD * j;
            const int i = i0 < Cfg::NPIECE ? i0 : dw;
            uint32_t g;
            if (i < Cfg::P_Q) g = rl.w + (i - Cfg::P_W) * 1024;
            else if (i < Cfg::P_K) g = rl.qt + (i - Cfg::P_Q) * 1024;
            else if (i < Cfg::P_P) g = rl.kt + (i - Cfg::P_K) * 1024;
            else if (i < Cfg::P_U) g = rl.p + (i - Cfg::P_P) * 1024;
            else if (i < Cfg::P_G) {
                const int u = i - Cfg::P_U, R = u / NUR, jj = u % NUR;
                g = rl.ut + (R * (DV / 32) + (v0 >> 5) + jj) * 1024;
            } else {
                g = rl.gam;
            }
            // the scan form never reads Q~ or P: such pieces load the (small,
            // cached) decay piece instead of streaming their own bytes
            if (SCAN && !REV && i >= Cfg::P_Q && (i < Cfg::P_K || (i >= Cfg::P_P && i < Cfg::P_U))) g = rl.gam;
            // reverse records: the P pieces carry U2 (this slice's pieces of
            // the section after the record's own), the rest the decay piece
            if (REV && i >= Cfg::P_P && i < Cfg::P_U) {
                const int u = i - Cfg::P_P;
                g = u < NB * NUR ? rl.bytes + ((u / NUR) * (DV / 32) + (v0 >> 5) + u % NUR) * 1024 : rl.gam;
            }
            pg[j] = __builtin_amdgcn_readfirstlane(g);
            pl[j] = __builtin_amdgcn_readfirstlane(i0 < Cfg::NPIECE ? (uint32_t)i0 * 1024u : 0xffffffffu);
        }
        const uint32_t l16 = l * 16;
        typedef int v4i __attribute__((ext_vector_type(4)));
        struct DSet {
            v4i v[NL];
        };
        auto fetch = [&](DSet& st, int cs) {
            cs = __builtin_amdgcn_readfirstlane(cs < ncs ? cs : ncs - 1);
            const __amdgpu_buffer_rsrc_t rr = make_rsrc(recs + (int64_t)cs * rstride, rstride);
#pragma unroll
            for (int j = 0; j < NL; ++j)
                st.v[j] = __builtin_bit_cast(
                    v4i, __builtin_amdgcn_raw_buffer_load_b128(rr, (int)l16, (int)pg[j], 0));
        };
        auto put = [&](const DSet& st, int cs) {
            char* slot = ring + (cs & 1) * SLOT;
            char* sink = smem + Cfg::O_SINK;
#pragma unroll
            for (int j = 0; j < NL; ++j)
                *(v4i*)((pl[j] == 0xffffffffu ? sink : slot + pl[j]) + l16) = st.v[j];
        };
        // o tile of chunk cs (cs < 0: every store falls past the buffer end)
        constexpr int PPR = NV * 2 / 16, NPO = C * PPR;  // 16-byte pieces
        constexpr int NS = (NPO + 64 * NWD - 1) / (64 * NWD);
        const __amdgpu_buffer_rsrc_t orsrc =
            make_rsrc((const char*)prm.o + sr.base * DV * 2, (uint32_t)(L * DV * 2));
        auto store_o = [&](int cs) {
            const int64_t t0 = (prm.c0 + cs) * C;
            const E* so = sO + (cs & 1) * C * PO;
#pragma unroll
            for (int k = 0; k < NS; ++k) {
                const int i = (tid - 64 * NWC) + 64 * NWD * k;
                const int ic = i < NPO ? i : 0;
                const int r = ic / PPR, cc = (ic % PPR) * 8;
                const uint4 val = *(const uint4*)(so + r * PO + cc);
                const uint32_t off = (cs >= 0 && i < NPO) ? (uint32_t)(((t0 + r) * DV + v0 + cc) * 2)
                                                          : 0x80000000u;
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i, val), orsrc, (int)off, 0, 0);
            }
        };
        constexpr int NSET = Cfg::NSET;
        DSet sets[NSET];
        if (ncs > 0) {
#pragma unroll
            for (int j = 0; j < NSET; ++j) fetch(sets[j], j);
            put(sets[0], 0);
            fetch(sets[0], NSET);
        }
        bare_barrier();
        for (int c0 = 0; c0 < ncs; c0 += NSET) {
            bool done = false;
#pragma unroll
            for (int j = 0; j < NSET; ++j) {
                if (!done) {
                    const int cs = c0 + j;
                    DSet& nx = sets[(j + 1) % NSET];
                    put(nx, cs + 1);
                    fetch(nx, cs + 1 + NSET);
                    if constexpr (!SCAN) store_o(cs - 1);
                    bare_barrier();
                    done = cs + 1 >= ncs;
                }
            }
            if (done) break;
        }
        if (ncs > 0 && !SCAN) {
            asm volatile("" ::: "memory");
            store_o(ncs - 1);
        }
        return;
    }

    // ========================= compute waves =====================================
    // wave w owns columns v0 + NVW w .. + NVW - 1: blocks vb = NVBW w + b
    floatx4 Sacc[NCB][NVBW];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int b = 0; b < NVBW; ++b) {
            Sacc[cb][b] = floatx4{0.f, 0.f, 0.f, 0.f};
            if (prm.S_in) {
                const float* s0 = prm.S_in + (int64_t)bh * DK * DV + v0 + 16 * (NVBW * w + b) + lr;
#pragma unroll
                for (int e = 0; e < 4; ++e) Sacc[cb][b][e] = s0[(16 * cb + 4 * lq + e) * DV];
            }
        }
    // the initial state loads are complete before the loop (nothing left
    // for the loop head to wait on)
    __builtin_amdgcn_s_waitcnt(0);
    bare_barrier();

    // The loop body is software-pipelined by hand: each group of LDS operand
    // reads is issued one step ahead of the MFMAs that use it, and
    // sched_barrier keeps the compiler from sinking the reads next to their
    // uses (each 1 KiB piece feeds only NVBW MFMAs, too few to hide an LDS
    // round trip behind).
    static_assert(NB == 4, "the pipeline below is written for 4 token blocks");
    constexpr int HC = NCB / 2;  // channel blocks per state-update half
    auto sched_fence = []() { __builtin_amdgcn_sched_barrier(0); };
    for (int cs = 0; cs < ncs; ++cs) {
        const char* slot = ring + (cs & 1) * SLOT;
        // scan form: is this chunk's entry kept, and where
        const int64_t xg = prm.c0 + cs;
        const bool keep = SCAN && (xg & ((1 << prm.scan_shift) - 1)) == 0;
        const int64_t xi = xg >> prm.scan_shift;
        if constexpr (SCAN) {
            if (keep) {
                float* sd = prm.S_all + ((int64_t)bh * prm.n_store + xi) * DK * DV + v0 + lr;
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                    for (int b = 0; b < NVBW; ++b)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            sd[(16 * cb + 4 * lq + e) * DV + 16 * (NVBW * w + b)] = Sacc[cb][b][e];
            }
        }
        auto piece = [&](int i) -> bf16x8 { return *(const bf16x8*)(slot + i * 1024 + l * 16); };
        // U block (R, vb) in accumulator order: two blocks per piece, the
        // slot's pieces starting at column block 2 (v0 / 32)
        auto u_init = [&](int R, int b, int base = Cfg::P_U) -> floatx4 {
            const int vbg = (v0 >> 4) + NVBW * w + b;  // column block of the head
            const int up = (vbg >> 1) - (v0 >> 5);
            const uint4 q4 = *(const uint4*)(slot + (base + R * NUR + up) * 1024 + l * 16);
            const uint32_t x = (vbg & 1) ? q4.z : q4.x, y = (vbg & 1) ? q4.w : q4.y;
            return floatx4{__uint_as_float(x << 16), __uint_as_float(x & 0xffff0000u),
                           __uint_as_float(y << 16), __uint_as_float(y & 0xffff0000u)};
        };
        E* so = sO + (cs & 1) * C * PO;
        const float* gam = (const float*)(slot + Cfg::P_G * 1024);
        bf16x8 wf[NB][NKA], qf[NB][NKA], pf[NB][NKP], kf[NCB][NKP], Sb[NKA][NVBW], ub[NKP][NVBW];
        floatx4 u[NB][NVBW];
        // u = U + (-W) S: lane holds u[16R + 4lq + e][16 vb + lr]
        auto u_block = [&](int R) {
#pragma unroll
            for (int kk = 0; kk < NKA; ++kk)
#pragma unroll
                for (int b = 0; b < NVBW; ++b) u[R][b] = F::mma(u[R][b], wf[R][kk], Sb[kk][b]);
        };
        // O^T = S^T Q~^T + u^T P^T: lane holds o[16R + lr][16 vb + 4lq + e],
        // into this chunk's LDS o tile
        auto o_block = [&](int R) {
            floatx4 oacc[NVBW];
#pragma unroll
            for (int b = 0; b < NVBW; ++b) oacc[b] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < NKA; ++kk)
#pragma unroll
                for (int b = 0; b < NVBW; ++b) oacc[b] = F::mma(oacc[b], Sb[kk][b], qf[R][kk]);
#pragma unroll
            for (int kk = 0; kk < NKP; ++kk)
                if (32 * kk <= 16 * R + 15)
#pragma unroll
                    for (int b = 0; b < NVBW; ++b) oacc[b] = F::mma(oacc[b], ub[kk][b], pf[R][kk]);
#pragma unroll
            for (int b = 0; b < NVBW; ++b)
                st4<E>(so + (16 * R + lr) * PO + 16 * (NVBW * w + b) + 4 * lq, oacc[b]);
        };
        auto read_w = [&](int R) {
#pragma unroll
            for (int kk = 0; kk < NKA; ++kk) wf[R][kk] = piece(Cfg::P_W + R * NKA + kk);
        };
        auto read_q = [&](int R) {
#pragma unroll
            for (int kk = 0; kk < NKA; ++kk) qf[R][kk] = piece(Cfg::P_Q + R * NKA + kk);
#pragma unroll
            for (int kk = 0; kk < NKP; ++kk)
                if (32 * kk <= 16 * R + 15) pf[R][kk] = piece(Cfg::P_P + R * NKP + kk);
        };
        auto read_k = [&](int cb0, int cb1) {
#pragma unroll
            for (int cb = cb0; cb < cb1; ++cb)
#pragma unroll
                for (int kk = 0; kk < NKP; ++kk) kf[cb][kk] = piece(Cfg::P_K + cb * NKP + kk);
        };
        // S = e^{g_n} S + K^T u for channel blocks cb0 .. cb1-1
        auto s_update = [&](int cb0, int cb1) {
#pragma unroll
            for (int cb = cb0; cb < cb1; ++cb) {
                const floatx4 g4 = *(const floatx4*)(gam + 16 * cb + 4 * lq);
#pragma unroll
                for (int b = 0; b < NVBW; ++b) {
                    floatx4 acc = Sacc[cb][b] * g4;
#pragma unroll
                    for (int kk = 0; kk < NKP; ++kk) acc = F::mma(acc, kf[cb][kk], ub[kk][b]);
                    Sacc[cb][b] = acc;
                }
            }
        };
        auto pack_s = [&]() {
#pragma unroll
            for (int kk = 0; kk < NKA; ++kk)
#pragma unroll
                for (int b = 0; b < NVBW; ++b) Sb[kk][b] = pack_frag(Sacc[2 * kk][b], Sacc[2 * kk + 1][b]);
        };
        auto store_u = [&]() {
            if (keep) {
                bf16* ud = (bf16*)prm.u_all + ((int64_t)bh * prm.n_store + xi) * C * DV + v0 + lr;
#pragma unroll
                for (int R = 0; R < NB; ++R)
#pragma unroll
                    for (int b = 0; b < NVBW; ++b)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            ud[(16 * R + 4 * lq + e) * DV + 16 * (NVBW * w + b)] = (bf16)u[R][b][e];
            }
        };
        auto pack_u = [&]() {
#pragma unroll
            for (int kk = 0; kk < NKP; ++kk)
#pragma unroll
                for (int b = 0; b < NVBW; ++b) ub[kk][b] = pack_frag(u[2 * kk][b], u[2 * kk + 1][b]);
        };
        if constexpr (NVBW == 1) {
            // one column block: registers hold W, Q~ and P of the whole chunk
            // at once, so every LDS round trip but the first overlaps MFMAs
#pragma unroll
            for (int R = 0; R < NB; ++R) read_w(R);
#pragma unroll
            for (int R = 0; R < NB; ++R) u[R][0] = u_init(R, 0);
            if constexpr (!SCAN) {
#pragma unroll
                for (int R = 0; R < NB; ++R) read_q(R);
            }
            sched_fence();
            pack_s();
#pragma unroll
            for (int R = 0; R < NB; ++R) u_block(R);
            sched_fence();
            read_k(0, NCB);
            sched_fence();
            pack_u();
            if constexpr (SCAN) {
                store_u();
            } else {
#pragma unroll
                for (int R = 0; R < NB; ++R) o_block(R);
            }
            s_update(0, NCB);
            if constexpr (REV) {
                // the step's second product, S += K2^T U2
#pragma unroll
                for (int R = 0; R < NB; ++R) u[R][0] = u_init(R, 0, Cfg::P_P);
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                    for (int kk = 0; kk < NKP; ++kk) kf[cb][kk] = piece(Cfg::P_Q + cb * NKP + kk);
                sched_fence();
                pack_u();
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) {
                    floatx4 acc = Sacc[cb][0];
#pragma unroll
                    for (int kk = 0; kk < NKP; ++kk) acc = F::mma(acc, kf[cb][kk], ub[kk][0]);
                    Sacc[cb][0] = acc;
                }
            }
        } else {
            // two column blocks: the reads of each group go out one step
            // ahead of the MFMAs that use them
#pragma unroll
            for (int R = 0; R < NB; ++R) read_w(R);
#pragma unroll
            for (int R = 0; R < NB; ++R)
#pragma unroll
                for (int b = 0; b < NVBW; ++b) u[R][b] = u_init(R, b);
            sched_fence();
            pack_s();
            u_block(0);
            u_block(1);
            sched_fence();
            if constexpr (!SCAN) {
                read_q(0);
                read_q(1);
            }
            sched_fence();
            u_block(2);
            u_block(3);
            sched_fence();
            if constexpr (!SCAN) {
                read_q(2);
                read_q(3);
            }
            sched_fence();
            pack_u();
            if constexpr (SCAN) {
                store_u();
            } else {
                o_block(0);
                o_block(1);
            }
            sched_fence();
            read_k(0, HC);
            sched_fence();
            if constexpr (!SCAN) {
                o_block(2);
                o_block(3);
            }
            sched_fence();
            read_k(HC, NCB);
            sched_fence();
            s_update(0, NCB);
        }
        bare_barrier();
    }

    // ---- state out --------------------------------------------------------------
    if (prm.S_out) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int b = 0; b < NVBW; ++b) {
                float* so = prm.S_out + (int64_t)bh * DK * DV + v0 + 16 * (NVBW * w + b) + lr;
#pragma unroll
                for (int e = 0; e < 4; ++e) so[(16 * cb + 4 * lq + e) * DV] = Sacc[cb][b][e];
            }
    }
}

// ---- 16-column slices: four waves, operands straight from memory -----------
// On gfx950 a CU writes LDS at only about 64-80 bytes per clock (reads reach
// about 240), so staging every record piece through an LDS ring costs more
// than loading it (measured on the long-context shape: the ring's writes
// alone about 1,500 cycles per chunk, the record loads alone about 630).
// Here nothing of the record passes through LDS.  The chunk's work is dealt
// over four waves, one per SIMD, so that each needs only about a quarter of
// the record, which it loads itself into registers two chunks ahead: wave j
// takes u's token block j (u_j = U_j - W_j S, needing all of S), the state's
// channel blocks of its quarter (S <- e^{g_n} S + K^T u, needing all of u)
// and o's token block j.  S and u cross between the waves as bf16 operand
// fragments through two small LDS exchange areas, two barriers per chunk:
//   X1 .. X2   u_j, its fragment half to the exchange
//   X2 .. X1   state update; the new S fragment to the exchange; o_j of the
//              chunk, stored from registers
// and each group of a wave's registers is refilled with chunk c + 2 as soon
// as its last use in chunk c is issued.
// Every column goes through the same operations, in the same order, as in
// the other widths' kernel, so the results are the same bit for bit.
template <int DK_, int NSET_>
struct QuadCfg {
    static constexpr int DK = DK_, NV = 16, C = 64;
    static constexpr int NB = C / 16, NKA = DK / 32, NKP = C / 32, NCB = DK / 16;
    static constexpr int NW = 4, NT = 64 * NW;
    static constexpr int CBW = NCB / NW;  // state channel blocks per wave
    static constexpr int NSET = NSET_;    // chunks of operands in flight per wave
    static constexpr int O_XS = 0, O_XU = NKA * 1024, LDS_BYTES = O_XU + NKP * 1024;
    static_assert(NB == NW && (CBW == 1 || CBW == 2), "one token block per wave");
};

// fp32 accumulator quad -> four bf16 (nearest even): half an operand fragment
__device__ __forceinline__ bf16x4 pack_half(floatx4 a) {
    bf16x4 r;
    r[0] = (bf16)a[0];
    r[1] = (bf16)a[1];
    r[2] = (bf16)a[2];
    r[3] = (bf16)a[3];
    return r;
}

template <class Cfg>
__global__ void __launch_bounds__(Cfg::NT, 2) kda_inter_quad_kernel(InterParams prm) {
    typedef bf16 E;
    typedef Frag<E> F;
    typedef int v2i __attribute__((ext_vector_type(2)));
    typedef int v4i __attribute__((ext_vector_type(4)));
    constexpr int DK = Cfg::DK, NV = Cfg::NV, C = Cfg::C, NKA = Cfg::NKA, NKP = Cfg::NKP;
    constexpr int CBW = Cfg::CBW, NSET = Cfg::NSET;

    __shared__ __attribute__((aligned(16))) char smem[Cfg::LDS_BYTES];
    char* xs = smem + Cfg::O_XS;
    char* xu = smem + Cfg::O_XU;

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63;
    const int lr = l & 15, lq = l >> 4;

    // workgroup i runs on XCD i % 8: the slices of one head share an XCD and
    // so one L2 for their reads of the head's records
    const int total = prm.BH * prm.n_slices;
    int pidx = blockIdx.x;
    if ((total & 7) == 0) pidx = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
    const int bh = pidx / prm.n_slices;
    const int slice = pidx - bh * prm.n_slices;
    const int v0 = slice * NV;
    const SeqRange sr = seq_range(prm.cu, prm.L, prm.H, bh);
    const int64_t L = sr.len;
    const int DV = prm.DV;
    const RecLayout rl = rec_layout(DK, DV, C, 2, true);
    const char* recs = (const char*)prm.ws + (int64_t)bh * prm.ncs * rl.bytes;
    int64_t left = (L + C - 1) / C - prm.c0;
    const int ncs = (int)(left < 0 ? 0 : (left < prm.ncs ? left : prm.ncs));
    // Chunk steps, rounded up to whole rounds of the register sets; steps past
    // the last chunk repeat its loads and arithmetic but keep neither the state
    // nor o.  A loop body without branches around its memory operations keeps
    // the compiler's memory-counter waits exact across the back edge.
    const int nsteps = ncs > 0 ? (ncs + NSET - 1) / NSET * NSET : 0;

    auto bare_barrier = []() {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };

    // ---- this wave's operands of one chunk, straight from its record ----------
    struct OSet {
        bf16x8 wf[NKA];       // W_w (stored negated), contraction blocks kk
        bf16x8 kf[CBW][NKP];  // K^T rows of this wave's channel blocks
        bf16x8 qf[NKA];       // Q~_w
        bf16x8 pf[NKP];       // P_w (blocks past the diagonal not loaded)
        v2i uf;               // U_w: this slice's half of the 32-column piece
        floatx4 g[CBW];       // e^{g_n} of this lane's state rows
    };
    const uint32_t l16 = l * 16;
    const int vh = (v0 >> 4) & 1;
    // piece offsets in the record (wave-uniform)
    const uint32_t off_w = rl.w + w * NKA * 1024, off_q = rl.qt + w * NKA * 1024;
    const uint32_t off_k = rl.kt + CBW * w * NKP * 1024, off_p = rl.p + w * NKP * 1024;
    const uint32_t off_u = rl.ut + (w * (DV / 32) + (v0 >> 5)) * 1024;
    // The loads of one chunk go out in three groups, each as soon as the
    // registers it refills are free, so that the texture path (about 64-100
    // bytes per clock per CU) streams them while the waves compute instead of
    // stalling all four waves on one burst.
    auto rsrc_of = [&](int cs) {
        cs = __builtin_amdgcn_readfirstlane(cs < ncs ? cs : ncs - 1);
        return make_rsrc(recs + (int64_t)cs * rl.bytes, rl.bytes);
    };
    auto ld = [&](__amdgpu_buffer_rsrc_t rr, uint32_t off) -> bf16x8 {
        return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rr, (int)l16, (int)off, 0));
    };
    auto fetch_u = [&](OSet& st, __amdgpu_buffer_rsrc_t rr) {  // W, U: used before X2
#pragma unroll
        for (int kk = 0; kk < NKA; ++kk) st.wf[kk] = ld(rr, off_w + kk * 1024);
        st.uf = __builtin_bit_cast(v2i, __builtin_amdgcn_raw_buffer_load_b64(rr, (int)(l16 + vh * 8), (int)off_u, 0));
    };
    auto fetch_s = [&](OSet& st, __amdgpu_buffer_rsrc_t rr) {  // K^T, e^{g_n}: the update
#pragma unroll
        for (int i = 0; i < CBW; ++i) {
#pragma unroll
            for (int kk = 0; kk < NKP; ++kk) st.kf[i][kk] = ld(rr, off_k + (i * NKP + kk) * 1024);
            st.g[i] = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(
                rr, (int)((16 * (CBW * w + i) + 4 * lq) * 4), (int)rl.gam, 0));
        }
    };
    auto fetch_o = [&](OSet& st, __amdgpu_buffer_rsrc_t rr) {  // Q~, P: o
#pragma unroll
        for (int kk = 0; kk < NKA; ++kk) st.qf[kk] = ld(rr, off_q + kk * 1024);
#pragma unroll
        for (int kk = 0; kk < NKP; ++kk)
            if (32 * kk <= 16 * w + 15) st.pf[kk] = ld(rr, off_p + kk * 1024);
    };
    auto fetch = [&](OSet& st, int cs) {
        const __amdgpu_buffer_rsrc_t rr = rsrc_of(cs);
        fetch_u(st, rr);
        fetch_s(st, rr);
        fetch_o(st, rr);
    };
    auto sched_fence = []() { __builtin_amdgcn_sched_barrier(0); };

    // ---- state: this wave's channel blocks, all 16 columns -------------------
    floatx4 Sacc[CBW];
#pragma unroll
    for (int i = 0; i < CBW; ++i) {
        Sacc[i] = floatx4{0.f, 0.f, 0.f, 0.f};
        if (prm.S_in) {
            const float* s0 = prm.S_in + (int64_t)bh * DK * DV + v0 + lr;
#pragma unroll
            for (int e = 0; e < 4; ++e) Sacc[i][e] = s0[(16 * (CBW * w + i) + 4 * lq + e) * DV];
        }
    }
    // this wave's S rows as (half of) operand fragment CBW w / 2 of S
    auto write_s = [&]() {
        if constexpr (CBW == 2)
            *(bf16x8*)(xs + w * 1024 + l * 16) = pack_frag(Sacc[0], Sacc[1]);
        else
            *(bf16x4*)(xs + (w >> 1) * 1024 + l * 16 + (w & 1) * 8) = pack_half(Sacc[0]);
    };
    // o rows 16 w .. 16 w + 15 of the slice, 4 bf16 per lane; rows past the
    // sequence (and every row of a step past the last chunk) fall outside
    // the buffer resource and are dropped
    const __amdgpu_buffer_rsrc_t orsrc =
        make_rsrc((const char*)prm.o + sr.base * DV * 2, (uint32_t)(L * DV * 2));

    OSet sets[NSET];
    if (ncs > 0) {
#pragma unroll
        for (int j = 0; j < NSET; ++j) fetch(sets[j], j);
    }
    write_s();
    bare_barrier();  // X1 of step 0
    for (int c0 = 0; c0 < nsteps; c0 += NSET) {
#pragma unroll
        for (int j = 0; j < NSET; ++j) {
            const int cs = c0 + j;
            const bool live = cs < ncs;
            OSet& st = sets[j];
            const __amdgpu_buffer_rsrc_t rnext = rsrc_of(cs + NSET);
            // ---- X1 .. X2: u_w = U_w + (-W_w) S ----
            bf16x8 sb[NKA];
#pragma unroll
            for (int kk = 0; kk < NKA; ++kk) sb[kk] = *(const bf16x8*)(xs + kk * 1024 + l * 16);
            const uint32_t ux = (uint32_t)st.uf[0], uy = (uint32_t)st.uf[1];
            floatx4 u = {__uint_as_float(ux << 16), __uint_as_float(ux & 0xffff0000u),
                         __uint_as_float(uy << 16), __uint_as_float(uy & 0xffff0000u)};
#pragma unroll
            for (int kk = 0; kk < NKA; ++kk) u = F::mma(u, st.wf[kk], sb[kk]);
            *(bf16x4*)(xu + (w >> 1) * 1024 + l * 16 + (w & 1) * 8) = pack_half(u);
            sched_fence();
            fetch_u(st, rnext);
            sched_fence();
            bare_barrier();  // X2
            // ---- X2 .. X1: S = e^{g_n} S + K^T u; o_w = S^T Q~_w^T + u^T P_w^T ----
            bf16x8 ub[NKP];
#pragma unroll
            for (int kk = 0; kk < NKP; ++kk) ub[kk] = *(const bf16x8*)(xu + kk * 1024 + l * 16);
#pragma unroll
            for (int i = 0; i < CBW; ++i) {
                floatx4 acc = Sacc[i] * st.g[i];
#pragma unroll
                for (int kk = 0; kk < NKP; ++kk) acc = F::mma(acc, st.kf[i][kk], ub[kk]);
#pragma unroll
                for (int e = 0; e < 4; ++e) Sacc[i][e] = live ? acc[e] : Sacc[i][e];
            }
            write_s();
            sched_fence();
            fetch_s(st, rnext);
            sched_fence();
            floatx4 oacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < NKA; ++kk) oacc = F::mma(oacc, sb[kk], st.qf[kk]);
#pragma unroll
            for (int kk = 0; kk < NKP; ++kk)
                if (32 * kk <= 16 * w + 15) oacc = F::mma(oacc, ub[kk], st.pf[kk]);
            const int64_t row = (prm.c0 + cs) * C + 16 * w + lr;
            const uint32_t off = live && row < L ? (uint32_t)((row * DV + v0 + 4 * lq) * 2) : 0x80000000u;
            buf_st4<E>(orsrc, off, oacc);
            sched_fence();
            fetch_o(st, rnext);
            bare_barrier();  // X1 of step cs + 1
        }
    }
    if (prm.S_out) {
        float* so = prm.S_out + (int64_t)bh * DK * DV + v0 + lr;
#pragma unroll
        for (int i = 0; i < CBW; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) so[(16 * (CBW * w + i) + 4 * lq + e) * DV] = Sacc[i][e];
    }
}

// ---- host-side dispatch -----------------------------------------------------

template <int DK, int NV, int NWC, int NSET, bool SCAN = false, bool REV = false>
static hipError_t launch_wide_cfg(const InterParams& prm, hipStream_t stream) {
    typedef WideCfg<DK, NV, NWC, NSET> Cfg;
    const int total = prm.BH * prm.n_slices;
    hipLaunchKernelGGL((kda_inter_wide_kernel<Cfg, SCAN, REV>), dim3(total), dim3(Cfg::NT), 0, stream,
                       prm);
    return hipGetLastError();
}

template <int DK, int NSET>
static hipError_t launch_quad_cfg(const InterParams& prm, hipStream_t stream) {
    typedef QuadCfg<DK, NSET> Cfg;
    const int total = prm.BH * prm.n_slices;
    hipLaunchKernelGGL((kda_inter_quad_kernel<Cfg>), dim3(total), dim3(Cfg::NT), 0, stream, prm);
    return hipGetLastError();
}

int wide_slice_width(int dk, int dv, int qkv_bf16, int alpha_mode, int64_t BH) {
    if (!qkv_bf16 || alpha_mode != KDA_ALPHA_CHANNEL) return 0;
    if ((dk != 64 && dk != 128) || (dv != 64 && dv != 128)) return 0;
    // the widest slice that still gives one workgroup per CU: a chain's
    // chunk time grows with its columns, the total work shrinks
    if (BH * (dv / 64) >= 256) return 64;
    if (BH * (dv / 32) >= 256) return 32;
    return 16;
}

hipError_t launch_inter_wide(InterParams prm, int dk, int nv, hipStream_t stream) {
    if (prm.BH == 0) return hipSuccess;
    if (nv <= 0 || prm.DV % nv) return hipErrorInvalidValue;
    prm.n_slices = prm.DV / nv;
    // (columns, compute waves, chunks in flight): every compute wave owns 16
    // or 32 columns; the data waves keep as many chunks in flight as their
    // registers hold
    if (dk == 128 && nv == 16) return launch_quad_cfg<128, KDA_QUAD_NSET>(prm, stream);
    if (dk == 128 && nv == 32) return launch_wide_cfg<128, 32, 2, KDA_WIDE_NSET32>(prm, stream);
    if (dk == 128 && nv == 64) return launch_wide_cfg<128, 64, 2, KDA_WIDE_NSET64>(prm, stream);
    if (dk == 64 && nv == 16) return launch_quad_cfg<64, KDA_QUAD_NSET>(prm, stream);
    if (dk == 64 && nv == 32) return launch_wide_cfg<64, 32, 2, KDA_WIDE_NSET32>(prm, stream);
    if (dk == 64 && nv == 64) return launch_wide_cfg<64, 64, 2, KDA_WIDE_NSET64>(prm, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_inter_wide_scan(InterParams prm, int dk, int nv, hipStream_t stream) {
    if (prm.BH == 0) return hipSuccess;
    if (nv <= 0 || prm.DV % nv || !prm.S_all || !prm.u_all || prm.scan_shift < 0 ||
        prm.scan_shift > 4)
        return hipErrorInvalidValue;
    prm.n_slices = prm.DV / nv;
    // (32 columns only: the 64-column scan form would spill registers)
    if (prm.rev) {
        if (dk == 128 && nv == 32) return launch_wide_cfg<128, 32, 2, KDA_WIDE_NSET32, true, true>(prm, stream);
        if (dk == 64 && nv == 32) return launch_wide_cfg<64, 32, 2, KDA_WIDE_NSET32, true, true>(prm, stream);
        return hipErrorInvalidValue;
    }
    if (dk == 128 && nv == 32) return launch_wide_cfg<128, 32, 2, KDA_WIDE_NSET32, true>(prm, stream);
    if (dk == 64 && nv == 32) return launch_wide_cfg<64, 32, 2, KDA_WIDE_NSET32, true>(prm, stream);
    return hipErrorInvalidValue;
}

}  // namespace kda
