// The reverse record of one chunk, built from its forward record (wide
// order) and dJ/do, for the reverse scan of the chunkwise gradients.  Used by
// the intra-chunk kernel's gradient form right after it writes the forward
// record.
#pragma once

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

// Operand (m, 8 consecutive wide-order positions) of 16-byte piece pc of a
// wide-order operand with K columns: row m and the k of position e.
__device__ __forceinline__ void wide_piece(int pc, int K, int& m, int& kbase) {
    const int lane = pc & 63, blk = pc >> 6;
    const int kk = blk % (K >> 5), mb = blk / (K >> 5);
    m = 16 * mb + (lane & 15);
    kbase = 32 * kk + 4 * (lane >> 4);  // positions 0-3: kbase + e, 4-7: kbase + 16 + e - 4
}
__device__ __forceinline__ int wide_piece_k(int kbase, int e) { return kbase + (e & 3) + 16 * (e >> 2); }

template <int DK, int DV>
struct RevCfg {
    static constexpr int C = 64, NT = 512;
    static constexpr RecLayout RL = rec_layout(DK, DV, C, 2, true);
    static constexpr int PDO = DV + 16, PPT = C + 16;  // bf16 pitches
    static constexpr int O_W = 0, O_KT = O_W + C * DK * 2, O_QT = O_KT + DK * C * 2;
    static constexpr int O_P = O_QT + C * DK * 2, O_DO = O_P + C * C * 2;
    // P^T takes the space of W and K^T once both have been transposed, so
    // that two workgroups share a CU (at d_k = d_v = 128: 74 KiB each)
    static constexpr int O_PT = O_W;
    static constexpr int LDS_BYTES = O_DO + C * PDO * 2;
    static_assert(C * PPT * 2 <= O_QT, "P^T fits over W and K^T");
    static_assert(LDS_BYTES <= 80 * 1024 || DV > 128, "two workgroups per CU");
};

// Chunk c of head bh: reads the forward record (W negated, K^T, Q~, P) and
// the chunk's rows of dJ/do, writes reverse record nc - 1 - c.  Every thread
// of the workgroup (RevCfg::NT) calls it; smem holds RevCfg::LDS_BYTES.
template <int DK, int DV>
__device__ __forceinline__ void build_rev_record(const void* recs, void* rrecs, const void* dout,
                                                 int64_t L, int nc, int bh, int c, char* smem) {
    typedef RevCfg<DK, DV> Cfg;
    constexpr int C = Cfg::C, NT = Cfg::NT, PDO = Cfg::PDO, PPT = Cfg::PPT;
    constexpr RecLayout RL = Cfg::RL;
    const bf16* sW = (const bf16*)(smem + Cfg::O_W);
    const bf16* sKt = (const bf16*)(smem + Cfg::O_KT);
    const bf16* sQt = (const bf16*)(smem + Cfg::O_QT);
    const bf16* sP = (const bf16*)(smem + Cfg::O_P);
    bf16* sDO = (bf16*)(smem + Cfg::O_DO);
    bf16* sPT = (bf16*)(smem + Cfg::O_PT);

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63;
    const int64_t t0 = (int64_t)c * C;
    const int n = (int)(L - t0 < C ? L - t0 : C);
    const char* src = (const char*)recs + ((int64_t)bh * nc + c) * RL.bytes;
    char* dst = (char*)rrecs + ((int64_t)bh * nc + (nc - 1 - c)) * rev_rec_bytes(DK, DV);

    // the forward record's W (negated), K^T, Q~ and P as stored; dO by rows
    auto copy_in = [&](uint32_t goff, int loff, int bytes) {
        for (int i = tid * 16; i < bytes; i += NT * 16)
            *(uint4*)(smem + loff + i) = *(const uint4*)(src + goff + i);
    };
    copy_in(RL.w, Cfg::O_W, C * DK * 2);
    copy_in(RL.kt, Cfg::O_KT, DK * C * 2);
    copy_in(RL.qt, Cfg::O_QT, C * DK * 2);
    copy_in(RL.p, Cfg::O_P, C * C * 2);
    const bf16* gdo = (const bf16*)dout + ((int64_t)bh * L + t0) * DV;
    for (int i = tid; i < C * DV / 8; i += NT) {
        const int r = i / (DV / 8), c8 = (i % (DV / 8)) * 8;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (r < n) v = *(const uint4*)(gdo + (int64_t)r * DV + c8);
        *(uint4*)(sDO + r * PDO + c8) = v;
    }
    __syncthreads();

    // W <- K e^{g_n - g} (the transpose of the stored K^T), K^T <- -W^T (the
    // stored W is already negated), K2^T <- (Q e^g)^T in the Q~ section
    {
        bf16* aw = (bf16*)(dst + RL.w);
        bf16* akt = (bf16*)(dst + RL.kt);
        bf16* bkt = (bf16*)(dst + RL.qt);
        for (int pc = tid; pc < C * DK / 8; pc += NT) {
            int m, kb;
            wide_piece(pc, DK, m, kb);  // m: token, k: channel
            bf16x8 v;
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = sKt[wide_elem(wide_piece_k(kb, e), m, C)];
            *(bf16x8*)(aw + pc * 8) = v;
        }
        for (int pc = tid; pc < DK * C / 8; pc += NT) {
            int m, kb;
            wide_piece(pc, C, m, kb);  // m: channel, k: token
            bf16x8 va, vb;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int r = wide_piece_k(kb, e);
                va[e] = sW[wide_elem(r, m, DK)];
                vb[e] = sQt[wide_elem(r, m, DK)];
            }
            *(bf16x8*)(akt + pc * 8) = va;
            *(bf16x8*)(bkt + pc * 8) = vb;
        }
        // the decay e^{g_n}, copied
        const float* sgam = (const float*)(src + RL.gam);
        for (int i = tid; i < DK; i += NT) ((float*)(dst + RL.gam))[i] = sgam[i];
        // U2 = dO in accumulator order, after the record's own sections:
        // element (16R + 4(l/16) + i, 16vb + l%16) at
        // ((R * DV/32 + vb/2) * 64 + l) * 8 + (vb % 2) * 4 + i
        bf16* but = (bf16*)(dst + RL.bytes);
        for (int t = w; t < 4 * (DV / 16); t += NT / 64) {
            const int R = t / (DV / 16), vb = t % (DV / 16);
            bf16x4 v;
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = sDO[(16 * R + 4 * (l >> 4) + i) * PDO + 16 * vb + (l & 15)];
            *(bf16x4*)(but + ((R * (DV / 32) + vb / 2) * 64 + l) * 8 + (vb % 2) * 4) = v;
        }
    }
    __syncthreads();
    // P^T by rows for the product P^T dO (over W and K^T, now read)
    for (int i = tid; i < C * C; i += NT) {
        const int j = i / C, r = i - j * C;
        sPT[j * PPT + r] = sP[wide_elem(r, j, C)];
    }
    __syncthreads();
    // U = P^T dO (MFMA), stored in accumulator order
    bf16* aut = (bf16*)(dst + RL.ut);
    for (int t = w; t < 4 * (DV / 16); t += NT / 64) {
        const int jb = t / (DV / 16), vb = t % (DV / 16);
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = mma_block_bt<bf16>(acc, sPT + 16 * jb * PPT, PPT, sDO, PDO, 16 * vb, C);
        st4<bf16>(aut + ((jb * (DV / 32) + vb / 2) * 64 + l) * 8 + (vb % 2) * 4, acc);
    }
}

}  // namespace kda
