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
// One workgroup (8 waves) owns one (b, h) head and a slice of NV state
// columns (columns of S evolve independently, so slices never talk) and walks
// the chunks in order.  Its fp32 state slice lives in registers as 16x16
// blocks spread over the waves, with a transposed operand copy in LDS.  Every
// other operand comes straight from HBM into registers in MFMA order (the
// records are laid out for exactly these loads), one chunk ahead: a chunk
// costs two barriers.
//   phase A  u tiles: u = U - W S        (then u, and e^{g_n-g} u, to LDS)
//            o tiles: o = (Q S) e^g      (kept in registers)
//   phase B  S tiles: S = e^{g_n} S + K^T u  (new operand copy to LDS)
//            o tiles: o += P u, to an LDS tile
// and the o tile goes to HBM at the start of the next chunk, through a buffer
// resource bounded by the sequence end (the ragged last chunk needs no
// branch).  o tiles are computed transposed (lane = one token, four adjacent
// columns).  On gfx9 loads and stores share one wait counter, so the loop is
// ordered to never wait on a store it has just issued.
#include <type_traits>

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
    static constexpr int PADE = 32 / ESZ;
    static constexpr int PK = DK + PADE;   // S^T operand copy [NV][DK]
    static constexpr int PC = C + PADE;    // u^T [NV][C]
    static constexpr int NW = 8, NT = 64 * NW;
    // Phase-A items: (role, R, column group) with role u (u = U - W S) or o
    // (o = Q S ...), R a 16-token block, and the NVB column blocks of the
    // slice split into NG groups of VG blocks, so one wave loads a W or Q row
    // block once and uses it for every column block of its group.
    static constexpr int NG = (2 * NB >= NW || NVB == 1) ? 1 : (NW / (2 * NB) < NVB ? NW / (2 * NB) : NVB);
    static constexpr int VG = NVB / NG;
    static constexpr int NIA = 2 * NB * NG;
    // State items: (cb, column group): K^T row block cb for SG column blocks.
    static constexpr int NGS = (NCB >= NW || NVB == 1) ? 1 : (NW / NCB < NVB ? NW / NCB : NVB);
    static constexpr int SG = NVB / NGS;
    static constexpr int NIS = NCB * NGS;
    static_assert(NIA <= NW && NIS <= NW, "one phase-A item and one state item per wave");
    static_assert(VG * NG == NVB && SG * NGS == NVB, "column groups");
    static constexpr int O_ST = 0;
    static constexpr int O_UT = O_ST + NV * PK * ESZ;
    static constexpr int O_UHT = O_UT + NV * PC * ESZ;
    static constexpr int PO = NV + PADE;   // o tile [C][NV]
    static constexpr int O_O = O_UHT + (KDA ? 0 : NV * PC * ESZ);
    static constexpr int LDS_BYTES = O_O + C * PO * ESZ;
    static_assert(DK % 32 == 0 && NV % 16 == 0 && (C == 32 || C == 64), "tile shape");
};

template <class Cfg>
__global__ void __launch_bounds__(Cfg::NT) kda_inter_kernel(InterParams prm) {
    typedef typename Cfg::E E;
    typedef Frag<E> F;
    typedef typename F::T FT;
    constexpr int DK = Cfg::DK, NV = Cfg::NV, C = Cfg::C, NB = Cfg::NB;
    constexpr bool KDA = Cfg::KDA;
    constexpr int PK = Cfg::PK, PC = Cfg::PC, NCB = Cfg::NCB, NVB = Cfg::NVB;
    constexpr int NW = Cfg::NW, NG = Cfg::NG, VG = Cfg::VG, NIA = Cfg::NIA;
    constexpr int NGS = Cfg::NGS, SG = Cfg::SG, NIS = Cfg::NIS;
    constexpr int ESZ = Cfg::ESZ, W = F::W, KS = F::KS;
    constexpr int NKA = DK / KS;  // k steps over key channels
    constexpr int NKP = C / KS;   // k steps over the chunk's tokens

    __shared__ __attribute__((aligned(16))) char smem[Cfg::LDS_BYTES];
    E* sST = (E*)(smem + Cfg::O_ST);
    E* sUT = (E*)(smem + Cfg::O_UT);
    E* sUHT = (E*)(smem + Cfg::O_UHT);
    E* sO = (E*)(smem + Cfg::O_O);
    constexpr int PO = Cfg::PO;

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63;
    const int lr = l & 15, lq = l >> 4;

    // ---- which (head, column slice) this workgroup owns --------------------
    // Dispatch places workgroup i on XCD i % 8; give all slices of a head the
    // same XCD so their shared operand reads hit one L2.
    const int total = prm.BH * prm.n_slices;
    int pidx = blockIdx.x;
    if ((total & 7) == 0) pidx = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
    const int bh = pidx / prm.n_slices;
    const int slice = pidx - bh * prm.n_slices;
    const int v0 = slice * NV;
    const int64_t L = prm.L;
    const int DV = prm.DV;
    const RecLayout rl = rec_layout(DK, DV, C, ESZ, KDA);

    const char* recs = (const char*)prm.ws + (int64_t)bh * prm.ncs * rl.bytes;
    // o of this head as a buffer: stores past token L are dropped
    const __amdgpu_buffer_rsrc_t orsrc =
        make_rsrc((const char*)prm.o + (int64_t)bh * L * DV * ESZ, (uint32_t)(L * DV * ESZ));

    // ---- this wave's items -----------------------------------------------------
    // phase A: item w < NIA is (role, R, group): role u for w < NB*NG, else o.
    // state: item w < NIS is (cb, group).  Waves without an item load the
    // first item's operands (valid addresses) and skip the arithmetic.
    const bool aval = w < NIA;
    const int ai = aval ? w : 0;
    const bool isU = ai < NB * NG;
    const int aR = (isU ? ai : ai - NB * NG) / NG;
    const int avb0 = ((isU ? ai : ai - NB * NG) % NG) * VG;  // first column block
    const bool sval = w < NIS;
    const int si = sval ? w : 0;
    const int scb = si / NGS;
    const int svb0 = (si % NGS) * SG;

    // ---- one chunk's operands, in registers ---------------------------------
    // The u and o roles share register slots: b[] holds P rows for an o wave,
    // U blocks (and e^{g_n-g}) for a u wave.  Both roles issue the same
    // loads from role-dependent addresses (a role with fewer slots re-reads a
    // valid one), so the instruction stream is one straight line.
    constexpr int PF = 16 / (4 * ESZ);                 // U blocks per 16-byte lane piece
    constexpr int UP = (VG + PF - 1) / PF;             // slots holding U
    constexpr int RU = KDA ? 0 : 1;                    // slot holding e^{g_n - g}
    constexpr int NBS = (NKP > UP + RU) ? NKP : UP + RU;
    struct Set {
        FT a[NKA];       // u role: W rows aR; o role: Q rows aR
        uint4 b[NBS];    // o role: P rows aR; u role: U blocks, then e^{g_n - g}
        float rq;        // scalar decay: e^{g_r} of row 16aR + lr (o role)
        FT kt[NKP];      // K^T rows of block scb
        floatx4 gm;      // KDA: e^{g_n} of rows 16scb + 4lq + e
        float gn;        // scalar decay: e^{g_n}
    };
    const int gvb0 = slice * NVB + avb0;               // first global column block
    const int uhalf = gvb0 % PF;                       // bf16, VG = 1: half of the piece
    // Loads only (no arithmetic on the loaded values, so nothing waits for
    // them here); the last chunk's record is re-read past the end.
    auto load = [&](Set& s, int cs) {
        cs = cs < prm.ncs ? cs : prm.ncs - 1;
        const char* rec = recs + (int64_t)cs * rl.bytes;
        const int R = aR;
        const char* ab = rec + (isU ? rl.w : rl.qt);
#pragma unroll
        for (int kk = 0; kk < NKA; ++kk) s.a[kk] = ldg<FT>(ab, ((R * NKA + kk) * 64 + l) * 16);
#pragma unroll
        for (int j = 0; j < NBS; ++j) {
            const int jp = j < NKP ? j : NKP - 1;
            const int ju = j < UP ? j : 0;
            const uint32_t uoff = ((R * (DV / (16 * PF)) + gvb0 / PF + ju) * 64 + l) * 16;
            const uint32_t roff = (C + 16 * R + 4 * lq) * 4;
            const char* bb = isU ? rec + ((RU && j == UP) ? rl.rs : rl.ut) : rec + rl.p;
            const uint32_t bo = isU ? ((RU && j == UP) ? roff : uoff)
                                    : (uint32_t)(((R * NKP + jp) * 64 + l) * 16);
            s.b[j] = ldg<uint4>(bb, bo);
        }
        if constexpr (!KDA) s.rq = ldg<float>(rec + rl.rs, (16 * R + lr) * 4);
#pragma unroll
        for (int kk = 0; kk < NKP; ++kk) s.kt[kk] = ldg<FT>(rec + rl.kt, ((scb * NKP + kk) * 64 + l) * 16);
        if constexpr (KDA) s.gm = ldg<floatx4>(rec + rl.gam, (16 * scb + 4 * lq) * 4);
        else s.gn = ldg<float>(rec + rl.rs, 2 * C * 4);
    };
    // U block g of a u wave, as fp32
    auto ut_f32 = [&](const Set& s, int g) -> floatx4 {
        if constexpr (ESZ == 2) {
            const int h = VG == 1 ? uhalf : g % 2;
            const uint4 q4 = s.b[VG == 1 ? 0 : g / 2];
            const uint32_t x = h == 0 ? q4.x : q4.z, y = h == 0 ? q4.y : q4.w;
            return floatx4{__uint_as_float(x << 16), __uint_as_float(x & 0xffff0000u),
                           __uint_as_float(y << 16), __uint_as_float(y & 0xffff0000u)};
        } else {
            const uint4 u = s.b[g];
            return floatx4{__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z),
                           __uint_as_float(u.w)};
        }
    };

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

    floatx4 oacc[VG];
    auto step = [&](const Set& s) {
        // ---------------- phase A ----------------
        if (aval) {
            const int R = aR;
            if (isU) {
                // u[16R + 4lq + e][16vb + lr] = U - sum_c W[r][c] S[c][v]
#pragma unroll
                for (int g = 0; g < VG; ++g) {
                    const int vb = avb0 + g;
                    const E* pst = sST + (16 * vb + lr) * PK + W * lq;
                    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kk = 0; kk < NKA; ++kk) acc = F::mma(acc, s.a[kk], F::load(pst + KS * kk));
                    const floatx4 u = ut_f32(s, g) - acc;
                    store_acc_transposed<E>(sUT + (16 * vb) * PC + 16 * R, PC, u);
                    if constexpr (!KDA)
                        store_acc_transposed<E>(sUHT + (16 * vb) * PC + 16 * R, PC,
                                                u * __builtin_bit_cast(floatx4, s.b[UP]));
                }
            } else {
                // transposed: lane holds (Q S)[r = 16R + lr][v = 16vb + 4lq + e]
#pragma unroll
                for (int g = 0; g < VG; ++g) {
                    const int vb = avb0 + g;
                    const E* pst = sST + (16 * vb + lr) * PK + W * lq;
                    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kk = 0; kk < NKA; ++kk) acc = F::mma(acc, F::load(pst + KS * kk), s.a[kk]);
                    if constexpr (!KDA) acc *= s.rq;
                    oacc[g] = acc;
                }
            }
        }
        __syncthreads();
        // ---------------- phase B ----------------
        if (sval) {
            const E* ub = KDA ? sUT : sUHT;
#pragma unroll
            for (int g = 0; g < SG; ++g) {
                const int vb = svb0 + g;
                floatx4 acc;
                if constexpr (KDA) acc = Sreg[g] * s.gm;
                else acc = Sreg[g] * s.gn;
                const E* pu = ub + (16 * vb + lr) * PC + W * lq;
#pragma unroll
                for (int kk = 0; kk < NKP; ++kk) acc = F::mma(acc, s.kt[kk], F::load(pu + KS * kk));
                Sreg[g] = acc;
                store_acc_transposed<E>(sST + (16 * vb) * PK + 16 * scb, PK, acc);
            }
        }
        if (aval && !isU) {
            const int R = aR;
#pragma unroll
            for (int g = 0; g < VG; ++g) {
                const int vb = avb0 + g;
                floatx4 acc = oacc[g];
                const E* pu = sUT + (16 * vb + lr) * PC + W * lq;
#pragma unroll
                for (int kk = 0; kk < NKP; ++kk)
                    if (KS * kk < 16 * (R + 1))
                        acc = F::mma(acc, F::load(pu + KS * kk), __builtin_bit_cast(FT, s.b[kk]));
                st4<E>(sO + (16 * R + lr) * PO + 16 * vb + 4 * lq, acc);
            }
        }
        __syncthreads();
    };
    // o tile of chunk cs, LDS -> HBM in 16-byte pieces; rows past the
    // sequence end fall outside the buffer and are dropped.
    auto store_o = [&](int cs) {
        const int64_t t0 = (prm.c0 + cs) * C;
        constexpr int PPR = NV * ESZ / 16, NPIECE = C * PPR;
        for (int i = tid; i < NPIECE; i += Cfg::NT) {
            const int r = i / PPR, cc = (i % PPR) * (16 / ESZ);
            const uint4 val = *(const uint4*)(sO + r * PO + cc);
            typedef int v4i __attribute__((ext_vector_type(4)));
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i, val), orsrc,
                                                   (int)(((t0 + r) * DV + v0 + cc) * ESZ), 0, 0);
        }
    };
    // Per chunk: wait for this chunk's operands (everything older is one
    // chunk old by now), store the previous chunk's o, fetch the next
    // chunk's operands, compute.  The waits never cover a fresh store.
    auto vm_wait_all = []() { __builtin_amdgcn_s_waitcnt(0x0f70); };  // vmcnt(0)

    Set s0, s1;
    if (prm.ncs > 0) load(s0, 0);
    for (int cs = 0; cs < prm.ncs; cs += 2) {
        vm_wait_all();
        if (cs > 0) store_o(cs - 1);
        load(s1, cs + 1);
        step(s0);
        if (cs + 1 >= prm.ncs) break;
        vm_wait_all();
        store_o(cs);
        load(s0, cs + 2);
        step(s1);
    }
    if (prm.ncs > 0) store_o(prm.ncs - 1);

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
