// kda_internal.h -- launch interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda.h"

namespace kda {

// Arguments of the fused chunkwise prefill kernel (one (b,h) per BH index).
struct ChunkParams {
    const void* q;          // [BH, L, DK]  qkv type
    const void* k;          // [BH, L, DK]
    const void* v;          // [BH, L, DV]
    const void* log_alpha;  // [BH, L, DK] | [BH, L] | unused, gate type
    const void* beta;       // [BH, L] gate type
    const float* S0;        // [BH, DK, DV] or null
    void* o;                // [BH, L, DV]  qkv type
    float* S_final;         // [BH, DK, DV] or null
    int64_t L;
    int BH;
    int DV;
    int n_slices;           // DV / slice width (set by launch_chunk)
    int gate_bf16;
    int alpha_mode;
};

// Arguments of the decode step kernel.
struct DecodeParams {
    const void* q;          // [BH, DK]
    const void* k;          // [BH, DK]
    const void* v;          // [BH, DV]
    const void* log_alpha;  // [BH, DK] | [BH] | unused
    const void* beta;       // [BH]
    float* S;               // [BH, DK, DV], updated in place
    void* o;                // [BH, DV]
    int BH;
    int gate_bf16;
    int alpha_mode;
};

// State-column slice width the prefill kernel uses for this problem.
int chunk_slice_width(int dk, int dv, int qkv_bf16, int64_t BH);

hipError_t launch_chunk(ChunkParams prm, int dk, int qkv_bf16, int nv, hipStream_t stream);
hipError_t launch_decode(const DecodeParams& prm, int dk, int dv, int qkv_bf16,
                         hipStream_t stream);

}  // namespace kda
