// kda_decode.hip -- one decode step of the KDA / gated delta rule on gfx950.
//
// Per (b, h), for one token ("22,580: From GPT-2 to Kimi K3"
// (yichencityu.github.io) section 5.2 with section 08's decay; "22580: From
// GPT-2 to Kimi3, Explained" (zharfai.com), "Gated DeltaNet adds controlled
// forgetting"):
//     S~ = diag(alpha) S;  r_k = k S~;  r_q = q S~
//     u  = beta (v - r_k);  o = r_q + (q . k) u;  S = S~ + k^T u
// o = q (S~ + k^T u) = r_q + (q . k) u, so the state is read once and written
// once.  The step is bound by that 8 dk dv bytes of HBM traffic per head.
//
// One 256-thread workgroup per head (per (sequence, head) in slot mode, where
// the state comes from a pool through the sequence's slot index).  Thread (row group rg, column group cg)
// holds RPT rows x 4 columns of S in registers (float4 loads: each row of a
// wave's access is 512 contiguous bytes), forms partial r_k / r_q over its
// rows, and the row groups are summed through LDS.  The new state is written
// with non-temporal stores: nothing reads it back before the next step, and
// on MI355X keeping those lines out of the caches lifts the read-modify-write
// stream from about 5.0 to about 6.5 TB/s (256 x 32 heads, d = 128).
//
// LA instance: one step of normalized linear attention with phi = elu + 1
// ("22,580: From GPT-2 to Kimi K3", section 04): S += phi(k)^T v,
// z += phi(k), o = phi(q) S / (phi(q) . z), so o = (phi(q) S_old +
// (phi(q) . phi(k)) v) / (phi(q) . z_old + phi(q) . phi(k)), again one read
// and one write of S.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

template <int DK, int DV, typename E, bool LA>
__global__ void __launch_bounds__(256) kda_decode_kernel(DecodeParams p) {
    constexpr int NCG = DV / 4;      // float4 column groups
    constexpr int NRG = 256 / NCG;   // row groups
    constexpr int RPT = DK / NRG;    // rows per thread
    static_assert(NCG * NRG == 256 && RPT * NRG == DK, "decode tiling");

    __shared__ __attribute__((aligned(16))) float red_k[NRG][DV];
    __shared__ __attribute__((aligned(16))) float red_q[NRG][DV];
    __shared__ float red_qk[NRG], red_qz[NRG];
    __shared__ float sq[DK], sk[DK], sa[DK], sz[DK];
    __shared__ float snorm[2];

    const int tid = threadIdx.x;
    const int cg = tid % NCG, rg = tid / NCG;
    const int64_t bh = blockIdx.x;
    const bool gbf = p.gate_bf16 != 0;

    float* S = p.S + bh * DK * DV;
    if (p.slots) {
        // state pool: (slot, h) of sequence b; an idle sequence writes o = 0
        const int64_t b = bh / p.H, h = bh - b * p.H;
        const int64_t slot = p.slots[b];
        if (slot < 0 || slot >= p.n_slots) {
            if (tid < DV / 4) {
                E* po = (E*)p.o + bh * DV + 4 * tid;
#pragma unroll
                for (int e = 0; e < 4; ++e) po[e] = from_f32<E>(0.f);
            }
            return;
        }
        S = p.S + (slot * p.H + h) * DK * DV;
    }

    if (tid < DK) {
        sq[tid] = to_f32(((const E*)p.q)[bh * DK + tid]);
        sk[tid] = to_f32(((const E*)p.k)[bh * DK + tid]);
        if constexpr (LA) {
            sq[tid] = elu1(sq[tid]);
            sk[tid] = elu1(sk[tid]);
            sz[tid] = p.z[bh * DK + tid];
        }
        float la = 0.f;
        if (p.alpha_mode == KDA_ALPHA_CHANNEL)
            la = gbf ? (float)((const bf16*)p.log_alpha)[bh * DK + tid]
                     : ((const float*)p.log_alpha)[bh * DK + tid];
        else if (p.alpha_mode == KDA_ALPHA_HEAD)
            la = gbf ? (float)((const bf16*)p.log_alpha)[bh] : ((const float*)p.log_alpha)[bh];
        if (p.flags & KDA_IN_GATE_RAW) la = log_alpha_of_raw(la);
        sa[tid] = (p.alpha_mode == KDA_ALPHA_NONE) ? 1.f : __expf(la);
    }
    float beta = 1.f;
    if constexpr (!LA) {
        beta = gbf ? (float)((const bf16*)p.beta)[bh] : ((const float*)p.beta)[bh];
        if (p.flags & KDA_IN_BETA_LOGIT) beta = sigmoid(beta);
    }

    floatx4 s[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i)
        s[i] = *(const floatx4*)(S + (int64_t)(rg * RPT + i) * DV + 4 * cg);
    __syncthreads();
    if (p.flags & KDA_IN_NORM_QK) {
        // q / |q| and k / |k| (the state loads above are already in flight)
        if (tid < 64) {
            float a = 0.f, b = 0.f;
            for (int i = tid; i < DK; i += 64) {
                a += sq[i] * sq[i];
                b += sk[i] * sk[i];
            }
            a = group_sum<64>(a);
            b = group_sum<64>(b);
            if (tid == 0) {
                snorm[0] = inv_norm(a);
                snorm[1] = inv_norm(b);
            }
        }
        __syncthreads();
        if (tid < DK) {
            sq[tid] *= snorm[0];
            sk[tid] *= snorm[1];
        }
        __syncthreads();
    }

    floatx4 pk = {0.f, 0.f, 0.f, 0.f}, pq = {0.f, 0.f, 0.f, 0.f};
    float pqk = 0.f, pqz = 0.f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int row = rg * RPT + i;
        if constexpr (!LA) {
            s[i] = s[i] * sa[row];
            pk += sk[row] * s[i];
        } else {
            pqz += sq[row] * sz[row];
        }
        pq += sq[row] * s[i];
        pqk += sq[row] * sk[row];
    }
    if constexpr (!LA) *(floatx4*)&red_k[rg][4 * cg] = pk;
    *(floatx4*)&red_q[rg][4 * cg] = pq;
    if (cg == 0) {
        red_qk[rg] = pqk;
        red_qz[rg] = pqz;
    }
    __syncthreads();

    floatx4 rk = {0.f, 0.f, 0.f, 0.f}, rq = {0.f, 0.f, 0.f, 0.f};
    float qk = 0.f, qz = 0.f;
#pragma unroll
    for (int g = 0; g < NRG; ++g) {
        if constexpr (!LA) rk += *(const floatx4*)&red_k[g][4 * cg];
        rq += *(const floatx4*)&red_q[g][4 * cg];
        qk += red_qk[g];
        if constexpr (LA) qz += red_qz[g];
    }
    floatx4 vv;
#pragma unroll
    for (int e = 0; e < 4; ++e) vv[e] = to_f32(((const E*)p.v)[bh * DV + 4 * cg + e]);
    // linear attention: no delta term (u = v)
    const floatx4 u = LA ? vv : beta * (vv - rk);
    if constexpr (LA) {
        if (tid < DK) p.z[bh * DK + tid] = sz[tid] + sk[tid];
    }
    if (rg == 0) {
        floatx4 o = rq + qk * u;
        if constexpr (LA) o = o * (1.f / (qz + qk));
        E* po = (E*)p.o + bh * DV + 4 * cg;
#pragma unroll
        for (int e = 0; e < 4; ++e) po[e] = from_f32<E>(o[e]);
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int row = rg * RPT + i;
        __builtin_nontemporal_store(s[i] + sk[row] * u, (floatx4*)(S + (int64_t)row * DV + 4 * cg));
    }
}

hipError_t launch_decode(const DecodeParams& prm, int dk, int dv, int qkv_bf16,
                         hipStream_t stream) {
    if (prm.BH == 0) return hipSuccess;
#define KDA_CASE(DK_, DV_, E_)                                                           \
    if (dk == DK_ && dv == DV_ && (qkv_bf16 != 0) == (sizeof(E_) == 2)) {               \
        if (prm.linear_attn)                                                            \
            hipLaunchKernelGGL((kda_decode_kernel<DK_, DV_, E_, true>), dim3(prm.BH),   \
                               dim3(256), 0, stream, prm);                              \
        else                                                                            \
            hipLaunchKernelGGL((kda_decode_kernel<DK_, DV_, E_, false>), dim3(prm.BH),  \
                               dim3(256), 0, stream, prm);                              \
        return hipGetLastError();                                                       \
    }
    KDA_CASE(128, 128, bf16)
    KDA_CASE(128, 64, bf16)
    KDA_CASE(64, 128, bf16)
    KDA_CASE(64, 64, bf16)
    KDA_CASE(128, 128, float)
    KDA_CASE(128, 64, float)
    KDA_CASE(64, 128, float)
    KDA_CASE(64, 64, float)
#undef KDA_CASE
    return hipErrorInvalidValue;
}

}  // namespace kda
