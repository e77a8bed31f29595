// kda_feature.hip -- the feature map phi(x) = elu(x) + 1 of normalized linear
// attention ("22,580: From GPT-2 to Kimi K3" (yichencityu.github.io), section
// 04: applied to q and k separately, before they meet) on q, written once per
// call for the state pass to read (k gets phi inside the state pass).
//
// Elementwise and HBM-bound: each thread moves 16-byte pieces (grid-stride),
// storing phi rounded to the input type.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

template <typename E>
__global__ void __launch_bounds__(256) kda_feature_map_kernel(FeatureParams p) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < p.n16; i += stride) {
        const uint4 u = ((const uint4*)p.q)[i];
        uint4 r;
        if constexpr (sizeof(E) == 2)
            r = __builtin_bit_cast(uint4, elu1(__builtin_bit_cast(bf16x8, u)));
        else
            r = __builtin_bit_cast(uint4, elu1(__builtin_bit_cast(floatx4, u)));
        ((uint4*)p.fq)[i] = r;
    }
}

hipError_t launch_feature_map(const FeatureParams& prm, int qkv_bf16, hipStream_t stream) {
    if (prm.n16 == 0) return hipSuccess;
    int64_t blocks = (prm.n16 + 255) / 256;
    if (blocks > 8192) blocks = 8192;  // 32 workgroups per CU, then grid-stride
    if (qkv_bf16)
        hipLaunchKernelGGL((kda_feature_map_kernel<bf16>), dim3((unsigned)blocks), dim3(256), 0,
                           stream, prm);
    else
        hipLaunchKernelGGL((kda_feature_map_kernel<float>), dim3((unsigned)blocks), dim3(256), 0,
                           stream, prm);
    return hipGetLastError();
}

}  // namespace kda
