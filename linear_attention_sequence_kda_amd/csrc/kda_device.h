// kda_device.h -- device helpers shared by the gfx950 KDA kernels.
//
// MFMA fragment conventions (checked on gfx950):
//   v_mfma_f32_16x16x32_bf16: lane l supplies A[l%16][8(l/16) .. 8(l/16)+7]
//     and B[8(l/16) .. +7][l%16]; it receives D[4(l/16)+i][l%16], i = 0..3.
//   v_mfma_f32_16x16x4_f32:   lane l supplies A[l%16][l/16], B[l/16][l%16],
//     and receives D[4(l/16)+i][l%16].
// A "fragment" below is what one lane supplies for KS consecutive k:
//   bf16: 8 bf16 at k offset 8(l/16) of a 32-wide k step  (one MFMA)
//   fp32: 4 floats at k offset 4(l/16) of a 16-wide k step (four MFMAs; the
//         s-th MFMA takes element s, which permutes k consistently for both
//         operands, so the sum over the four covers all 16 k).
// Both operands are given "k-contiguous": A as [m][k], B as [n][k].
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// ---- scalar conversions ---------------------------------------------------
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
template <typename E> __device__ __forceinline__ E from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// ---- MFMA fragments -------------------------------------------------------
template <typename E> struct Frag;

template <> struct Frag<bf16> {
    typedef bf16x8 T;
    static constexpr int W = 8;    // k elements per lane
    static constexpr int KS = 32;  // k per step
    static __device__ __forceinline__ T load(const bf16* p) { return *(const bf16x8*)p; }
    // p[0..7] * s[0..7], rounded back to bf16
    static __device__ __forceinline__ T load_scaled(const bf16* p, const float* s) {
        bf16x8 v = *(const bf16x8*)p;
        floatx4 s0 = *(const floatx4*)s;
        floatx4 s1 = *(const floatx4*)(s + 4);
        bf16x8 r;
        r[0] = (bf16)((float)v[0] * s0[0]);
        r[1] = (bf16)((float)v[1] * s0[1]);
        r[2] = (bf16)((float)v[2] * s0[2]);
        r[3] = (bf16)((float)v[3] * s0[3]);
        r[4] = (bf16)((float)v[4] * s1[0]);
        r[5] = (bf16)((float)v[5] * s1[1]);
        r[6] = (bf16)((float)v[6] * s1[2]);
        r[7] = (bf16)((float)v[7] * s1[3]);
        return r;
    }
    // p[0..7] * (s0, s1), rounded back to bf16
    static __device__ __forceinline__ T load_scaled_v(const bf16* p, floatx4 s0, floatx4 s1) {
        bf16x8 v = *(const bf16x8*)p;
        bf16x8 r;
        r[0] = (bf16)((float)v[0] * s0[0]);
        r[1] = (bf16)((float)v[1] * s0[1]);
        r[2] = (bf16)((float)v[2] * s0[2]);
        r[3] = (bf16)((float)v[3] * s0[3]);
        r[4] = (bf16)((float)v[4] * s1[0]);
        r[5] = (bf16)((float)v[5] * s1[1]);
        r[6] = (bf16)((float)v[6] * s1[2]);
        r[7] = (bf16)((float)v[7] * s1[3]);
        return r;
    }
    static __device__ __forceinline__ T load_scaled_neg(const bf16* p, const float* s) {
        bf16x8 v = *(const bf16x8*)p;
        floatx4 s0 = *(const floatx4*)s;
        floatx4 s1 = *(const floatx4*)(s + 4);
        bf16x8 r;
        r[0] = (bf16)(-(float)v[0] * s0[0]);
        r[1] = (bf16)(-(float)v[1] * s0[1]);
        r[2] = (bf16)(-(float)v[2] * s0[2]);
        r[3] = (bf16)(-(float)v[3] * s0[3]);
        r[4] = (bf16)(-(float)v[4] * s1[0]);
        r[5] = (bf16)(-(float)v[5] * s1[1]);
        r[6] = (bf16)(-(float)v[6] * s1[2]);
        r[7] = (bf16)(-(float)v[7] * s1[3]);
        return r;
    }
    static __device__ __forceinline__ floatx4 mma(floatx4 acc, T a, T b) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
    }
};

template <> struct Frag<float> {
    typedef floatx4 T;
    static constexpr int W = 4;
    static constexpr int KS = 16;
    static __device__ __forceinline__ T load(const float* p) { return *(const floatx4*)p; }
    static __device__ __forceinline__ T load_scaled(const float* p, const float* s) {
        return *(const floatx4*)p * *(const floatx4*)s;
    }
    static __device__ __forceinline__ T load_scaled_v(const float* p, floatx4 s0, floatx4) {
        return *(const floatx4*)p * s0;
    }
    static __device__ __forceinline__ T load_scaled_neg(const float* p, const float* s) {
        return -(*(const floatx4*)p * *(const floatx4*)s);
    }
    static __device__ __forceinline__ floatx4 mma(floatx4 acc, T a, T b) {
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], acc, 0, 0, 0);
        return acc;
    }
};

// acc(16x16) += A[16 x K] * B[16 x K]^T; A, B point at row 0 / k 0 of the
// operand tiles (k-contiguous, pitches lda / ldb in elements).  K % KS == 0.
template <typename E>
__device__ __forceinline__ floatx4 mma_block(floatx4 acc, const E* A, int lda, const E* B,
                                             int ldb, int K) {
    const int l = lane_id();
    const int r = l & 15, q = l >> 4;
    typedef Frag<E> F;
    const E* pa = A + r * lda + F::W * q;
    const E* pb = B + r * ldb + F::W * q;
#pragma unroll
    for (int kk = 0; kk < K; kk += F::KS)
        acc = F::mma(acc, F::load(pa + kk), F::load(pb + kk));
    return acc;
}

// Same, with the A operand scaled per k by s[k] (s indexed from k = 0).
template <typename E, bool NEG>
__device__ __forceinline__ floatx4 mma_block_scaled_a(floatx4 acc, const E* A, int lda,
                                                      const float* s, const E* B, int ldb,
                                                      int K) {
    const int l = lane_id();
    const int r = l & 15, q = l >> 4;
    typedef Frag<E> F;
    const E* pa = A + r * lda + F::W * q;
    const E* pb = B + r * ldb + F::W * q;
    const float* ps = s + F::W * q;
#pragma unroll
    for (int kk = 0; kk < K; kk += F::KS) {
        typename F::T a = NEG ? F::load_scaled_neg(pa + kk, ps + kk) : F::load_scaled(pa + kk, ps + kk);
        acc = F::mma(acc, a, F::load(pb + kk));
    }
    return acc;
}

// Write the four accumulator values of a lane, D[4q+i][r], transposed into a
// k-contiguous tile: dst[r * ld + 4q + i].
template <typename E>
__device__ __forceinline__ void store_acc_transposed(E* dst, int ld, floatx4 acc) {
    const int l = lane_id();
    const int r = l & 15, q = l >> 4;
    E* p = dst + r * ld + 4 * q;
    if constexpr (sizeof(E) == 2) {
        bf16x4 v;
        v[0] = (bf16)acc[0];
        v[1] = (bf16)acc[1];
        v[2] = (bf16)acc[2];
        v[3] = (bf16)acc[3];
        *(bf16x4*)p = v;
    } else {
        *(floatx4*)p = acc;
    }
}

// A operand fragment of K^T-like products read from a row-major [k][m] tile
// (m contiguous, pitch ld): lane (m = l%16, q = l/16) receives
// A[m][k0 + W q .. + W - 1] = T[k0 + W q + i][m0 + m].
//   bf16: two ds_read_b64_tr_b16.  Within a 16-lane group that instruction
//   hands output lane l element e of source lane (4e + l/4)'s 8 bytes, element
//   l%4; pointing source lane i at row i/4, column 4(i%4) of a 4-row slab
//   therefore delivers 4 consecutive rows of column l.
//   fp32: four scalar reads down the column.
__device__ __forceinline__ bf16x8 load_frag_tr(const bf16* T, int ld, int k0, int m0) {
    typedef short v4s __attribute__((ext_vector_type(4)));
    const int l = lane_id();
    const int q = l >> 4, i = l & 15;
    const bf16* p = T + (k0 + 8 * q + (i >> 2)) * ld + m0 + 4 * (i & 3);
    v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)p);
    v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4s*)(p + 4 * ld));
    // repack as whole 32-bit words (per-element bf16 casts were miscompiled)
    typedef int v2i __attribute__((ext_vector_type(2)));
    typedef int v4i __attribute__((ext_vector_type(4)));
    const v2i a = __builtin_bit_cast(v2i, lo), b = __builtin_bit_cast(v2i, hi);
    const v4i c = {a[0], a[1], b[0], b[1]};
    return __builtin_bit_cast(bf16x8, c);
}
__device__ __forceinline__ floatx4 load_frag_tr(const float* T, int ld, int k0, int m0) {
    const int l = lane_id();
    const int q = l >> 4, m = l & 15;
    const float* p = T + (k0 + 4 * q) * ld + m0 + m;
    floatx4 r = {p[0], p[ld], p[2 * ld], p[3 * ld]};
    return r;
}

// acc(16x16) += A * B^T where A[m][k] = T[k][m0 + m] comes from a row-major
// [k][m] tile (read transposed) and B is k-contiguous ([n][k], pitch ldb).
template <typename E>
__device__ __forceinline__ floatx4 mma_block_at(floatx4 acc, const E* T, int ldt, int m0,
                                                const E* B, int ldb, int K) {
    const int l = lane_id();
    const int r = l & 15, q = l >> 4;
    typedef Frag<E> F;
    const E* pb = B + r * ldb + F::W * q;
#pragma unroll
    for (int kk = 0; kk < K; kk += F::KS)
        acc = F::mma(acc, load_frag_tr(T, ldt, kk, m0), F::load(pb + kk));
    return acc;
}

// acc(16x16) += A * B^T where A is k-contiguous ([m][k], pitch lda) and
// B[n][k] = T[k][n0 + n] comes from a row-major [k][n] tile read transposed.
template <typename E>
__device__ __forceinline__ floatx4 mma_block_bt(floatx4 acc, const E* A, int lda, const E* T,
                                                int ldt, int n0, int K) {
    const int l = lane_id();
    const int r = l & 15, q = l >> 4;
    typedef Frag<E> F;
    const E* pa = A + r * lda + F::W * q;
#pragma unroll
    for (int kk = 0; kk < K; kk += F::KS)
        acc = F::mma(acc, F::load(pa + kk), load_frag_tr(T, ldt, kk, n0));
    return acc;
}

// ---- operand records ("fragment order") -----------------------------------
// Element offset of operand element (m, k) of an operand with K columns, in
// the order a 16x16 MFMA tile loop reads it: 16-byte pieces of W consecutive
// k, piece ((m/16) * (K/KS) + k/KS) * 64 + ((k % KS) / W) * 16 + m % 16.
template <typename E>
__device__ __forceinline__ uint32_t frag_elem(int m, int k, int K) {
    constexpr int W = Frag<E>::W, KS = Frag<E>::KS;
    return (uint32_t)((((m >> 4) * (K / KS) + k / KS) * 64 + ((k % KS) / W) * 16 + (m & 15)) * W +
                      k % W);
}

// ---- "wide" operand records -----------------------------------------------------
// Element offset of bf16 operand element (m, k) of an operand with K columns
// in the order the wide state pass reads it: 16-byte pieces of 8 values,
// piece ((m/16) * (K/32) + k/32) * 64 + lane, lane = 16 ((k % 16) / 4) + m % 16,
// position (k % 4) + 4 ((k % 32) / 16).  Within a 32-wide k step a lane's
// 8 values are k = 32kk + 4q .. +3 and 32kk + 16 + 4q .. +3 (q = lane / 16):
// exactly the rows a lane holds of two 16-row MFMA accumulator blocks, so an
// accumulator pair is an MFMA operand as it is (both operands of a product
// take the contraction index in this same order, which leaves the sum as it
// is).  Four consecutive k (a multiple of 4) are four consecutive positions.
__device__ __forceinline__ uint32_t wide_elem(int m, int k, int K) {
    const int kp = k & 31;
    return (uint32_t)(((((m >> 4) * (K >> 5) + (k >> 5)) * 64 + ((kp & 15) >> 2) * 16 + (m & 15)) * 8) +
                      (kp & 3) + 4 * (kp >> 4));
}

// ---- small stores and loads --------------------------------------------------
template <typename E>
__device__ __forceinline__ void st4(E* p, floatx4 v) {
    if constexpr (sizeof(E) == 2) {
        bf16x4 t;
        t[0] = (bf16)v[0];
        t[1] = (bf16)v[1];
        t[2] = (bf16)v[2];
        t[3] = (bf16)v[3];
        *(bf16x4*)p = t;
    } else {
        *(floatx4*)p = v;
    }
}

// v if keep, else zero (an explicit mask: a select of 16-byte values can be
// lowered into a select of stack addresses)
__device__ __forceinline__ uint4 keep_or_zero(uint4 v, bool keep) {
    const uint32_t m = keep ? 0xffffffffu : 0u;
    return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m);
}

// Load through a uniform base pointer plus a 32-bit byte offset (saddr form).
template <typename T>
__device__ __forceinline__ T ldg(const void* base, uint32_t byte_off) {
    return *(const T*)((const char*)base + byte_off);
}
// The same load with the non-temporal hint: for inputs read once, which then
// do not displace data that is read again soon (a prefill span's records in
// the memory-side cache) from the caches.
template <typename T>
__device__ __forceinline__ T ldg_stream(const void* base, uint32_t byte_off) {
    const char* p = (const char*)base + byte_off;
    if constexpr (sizeof(T) == 16) {
        typedef unsigned v4u __attribute__((ext_vector_type(4)));
        return __builtin_bit_cast(T, __builtin_nontemporal_load((const v4u*)p));
    } else if constexpr (sizeof(T) == 4) {
        return __builtin_bit_cast(T, __builtin_nontemporal_load((const uint32_t*)p));
    } else {
        static_assert(sizeof(T) == 2, "16-, 4- or 2-byte loads");
        return __builtin_bit_cast(T, __builtin_nontemporal_load((const uint16_t*)p));
    }
}

// Buffer resource over [base, base + bytes): loads past the end return zero
// and stores past the end are dropped by the hardware.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, 0x00020000);
}
// Store four values (converted to E) at byte offset off of a buffer.
template <typename E>
__device__ __forceinline__ void buf_st4(__amdgpu_buffer_rsrc_t r, uint32_t off, floatx4 v) {
    typedef int v2i __attribute__((ext_vector_type(2)));
    typedef int v4i __attribute__((ext_vector_type(4)));
    if constexpr (sizeof(E) == 2) {
        bf16x4 t;
        t[0] = (bf16)v[0];
        t[1] = (bf16)v[1];
        t[2] = (bf16)v[2];
        t[3] = (bf16)v[3];
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(v2i, t), r, (int)off, 0, 0);
    } else {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i, v), r, (int)off, 0, 0);
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

// ---- cross-lane moves (DPP) -------------------------------------------------
// Value of lane 4*(l/4) + so (so a compile-time constant after unrolling): a
// quad_perm broadcast inside every group of four lanes.
__device__ __forceinline__ float quad_bcast(float x, int so) {
    int v = __float_as_int(x);
    switch (so) {
        case 0: v = __builtin_amdgcn_mov_dpp(v, 0x00, 0xf, 0xf, false); break;
        case 1: v = __builtin_amdgcn_mov_dpp(v, 0x55, 0xf, 0xf, false); break;
        case 2: v = __builtin_amdgcn_mov_dpp(v, 0xaa, 0xf, 0xf, false); break;
        default: v = __builtin_amdgcn_mov_dpp(v, 0xff, 0xf, 0xf, false); break;
    }
    return __int_as_float(v);
}

// Inclusive prefix sum over the 64 lanes of a wave: shifts by 1, 2, 4, 8
// inside each row of 16 lanes, then the last lane of row 0 (row 2) is added
// to row 1 (row 3) and the last lane of row 1 to rows 2 and 3.  Lanes with no
// source add the "old" operand, 0.
__device__ __forceinline__ float wave_inclusive_sum(float x) {
#define KDA_DPP_ADD(ctrl, rmask)                                                              \
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), ctrl, rmask, 0xf, \
                                                    false))
    KDA_DPP_ADD(0x111, 0xf);  // row_shr:1
    KDA_DPP_ADD(0x112, 0xf);  // row_shr:2
    KDA_DPP_ADD(0x114, 0xf);  // row_shr:4
    KDA_DPP_ADD(0x118, 0xf);  // row_shr:8
    KDA_DPP_ADD(0x142, 0xa);  // row_bcast:15 into rows 1 and 3
    KDA_DPP_ADD(0x143, 0xc);  // row_bcast:31 into rows 2 and 3
#undef KDA_DPP_ADD
    return x;
}

__device__ __forceinline__ float read_lane(float x, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

// ---- fast exp for decay factors (inputs <= 0) -----------------------------
__device__ __forceinline__ float exp_neg(float x) { return __expf(x); }

// ---- input preprocessing (kda_input_flags) ---------------------------------
// sum of x over each aligned group of G lanes (G a power of two <= 64),
// returned in every lane of the group
template <int G>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
    for (int o = 1; o < G; o <<= 1) x += __shfl_xor(x, o);
    return x;
}
// sum of x over lanes l, l ^ 16, l ^ 32, l ^ 48
__device__ __forceinline__ float sum_over_lq(float x) {
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
    return x;
}
// sum of squares of one MFMA operand fragment
__device__ __forceinline__ float frag_sumsq(bf16x8 v) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) s += (float)v[i] * (float)v[i];
    return s;
}
__device__ __forceinline__ float frag_sumsq(floatx4 v) {
    return v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
}
// 1 / max(|x|, 1e-12) from the sum of squares (a zero row normalizes to zero)
__device__ __forceinline__ float inv_norm(float ss) { return 1.f / fmaxf(sqrtf(ss), 1e-12f); }
__device__ __forceinline__ float sigmoid(float x) { return 1.f / (1.f + __expf(-x)); }
// ln(alpha) from the raw gate g: -exp(g)
__device__ __forceinline__ float log_alpha_of_raw(float g) { return -__expf(g); }
// sum of squares of a 16-byte piece of E elements
__device__ __forceinline__ float sumsq16(uint4 u, bf16) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float a = __uint_as_float(w[i] << 16), b = __uint_as_float(w[i] & 0xffff0000u);
        s += a * a + b * b;
    }
    return s;
}
__device__ __forceinline__ float sumsq16(uint4 u, float) {
    const float a = __uint_as_float(u.x), b = __uint_as_float(u.y), c = __uint_as_float(u.z),
                d = __uint_as_float(u.w);
    return a * a + b * b + c * c + d * d;
}

// ---- linear attention feature map phi(x) = elu(x) + 1 (positive) ----------
__device__ __forceinline__ float elu1(float x) { return x > 0.f ? x + 1.f : __expf(x); }
__device__ __forceinline__ bf16x8 elu1(bf16x8 v) {
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = (bf16)elu1((float)v[i]);
    return r;
}
__device__ __forceinline__ floatx4 elu1(floatx4 v) {
    floatx4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = elu1(v[i]);
    return r;
}
// MFMA B operand of ones over tokens kk KS + W (lane/16) .. + W - 1 that are
// below n (zeros for padded tokens)
template <typename E>
__device__ __forceinline__ typename Frag<E>::T ones_below(int first, int n) {
    typename Frag<E>::T r;
#pragma unroll
    for (int i = 0; i < Frag<E>::W; ++i) r[i] = from_f32<E>(first + i < n ? 1.f : 0.f);
    return r;
}

}  // namespace kda
