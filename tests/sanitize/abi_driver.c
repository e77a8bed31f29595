/*
 * Sanitizer driver for the host side of the C ABI (test infrastructure).
 * tests/test_sanitizers.py builds the ABI layer (kda_api.cpp) with
 * -fsanitize=address,undefined on the host, links it with the kernels'
 * objects and this driver, and runs it on a machine that may have no GPU:
 * every call below is rejected by the host checks, or is an empty problem,
 * or is a size query, so no kernel is launched.  Pointers are fake aligned
 * addresses that are never dereferenced.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "kda.h"

static int fails = 0;
#define EXPECT(call, code)                                                         \
    do {                                                                           \
        int rc_ = (call);                                                          \
        if (rc_ != (code)) {                                                       \
            fprintf(stderr, "line %d: %s returned %d, expected %d\n", __LINE__,    \
                    #call, rc_, (code));                                           \
            ++fails;                                                               \
        }                                                                          \
    } while (0)

#define P(i) ((void*)(uintptr_t)(0x7F0000000000ull + (uint64_t)(i) * (64ull << 20)))

static kda_shape shp(int64_t B, int64_t H, int64_t L, int64_t dk, int64_t dv, int qd, int gd,
                     int mode) {
    kda_shape s;
    s.B = B, s.H = H, s.L = L, s.dk = dk, s.dv = dv;
    s.qkv_dtype = qd, s.gate_dtype = gd, s.alpha_mode = mode;
    return s;
}

int main(void) {
    kda_shape s = shp(2, 3, 100, 128, 128, KDA_BF16, KDA_F32, KDA_ALPHA_CHANNEL);
    const size_t ws = kda_chunk_fwd_workspace_bytes(&s);
    if (ws == 0 || ws % 256) ++fails;
    kda_shape z = s;
    z.B = 0;
    if (kda_chunk_fwd_workspace_bytes(&z) != 0) ++fails;
    if (kda_chunk_fwd_workspace_bytes(NULL) != 0) ++fails;
    for (int64_t L = 1; L < 1 << 20; L = L * 3 + 1) {
        kda_shape t = s;
        t.L = L;
        t.alpha_mode = (int)(L % 3);
        t.qkv_dtype = (int)(L & 1);
        (void)kda_chunk_fwd_workspace_bytes(&t);
        (void)kda_chunk_fwd_varlen_workspace_bytes(&t, L / 2);
        (void)kda_recurrence_bwd_workspace_bytes(&t);
        (void)kda_recurrence_bwd_ex_workspace_bytes(&t, 7);
        (void)kda_linear_attn_fwd_workspace_bytes(&t);
    }
    /* prefill: null shape, bad sizes, null pointer, misalignment, overlap,
       small workspace, empty problem */
    EXPECT(kda_chunk_fwd(NULL, P(0), P(1), P(2), P(3), P(4), P(5), P(6), P(7), P(8), ws, NULL), KDA_ERR_NULL);
    kda_shape bad = s;
    bad.dk = 96;
    EXPECT(kda_chunk_fwd(&bad, P(0), P(1), P(2), P(3), P(4), P(5), P(6), P(7), P(8), ws, NULL), KDA_ERR_SHAPE);
    bad = s;
    bad.qkv_dtype = 5;
    EXPECT(kda_chunk_fwd(&bad, P(0), P(1), P(2), P(3), P(4), P(5), P(6), P(7), P(8), ws, NULL), KDA_ERR_DTYPE);
    bad = s;
    bad.alpha_mode = 3;
    EXPECT(kda_chunk_fwd(&bad, P(0), P(1), P(2), P(3), P(4), P(5), P(6), P(7), P(8), ws, NULL), KDA_ERR_ALPHA_MODE);
    bad = s;
    bad.L = -1;
    EXPECT(kda_chunk_fwd(&bad, P(0), P(1), P(2), P(3), P(4), P(5), P(6), P(7), P(8), ws, NULL), KDA_ERR_SHAPE);
    bad = s;
    bad.B = INT64_MAX / 2;
    EXPECT(kda_chunk_fwd(&bad, P(0), P(1), P(2), P(3), P(4), P(5), P(6), P(7), P(8), ws, NULL), KDA_ERR_SHAPE);
    EXPECT(kda_chunk_fwd(&s, NULL, P(1), P(2), P(3), P(4), P(5), P(6), P(7), P(8), ws, NULL), KDA_ERR_NULL);
    EXPECT(kda_chunk_fwd(&s, P(0), P(1), P(2), P(3), (char*)P(4) + 8, P(5), P(6), P(7), P(8), ws, NULL), KDA_ERR_ALIGN);
    EXPECT(kda_chunk_fwd(&s, P(0), P(1), P(2), P(3), P(4), P(5), (char*)P(0) + 1024, P(7), P(8), ws, NULL), KDA_ERR_ALIAS);
    EXPECT(kda_chunk_fwd(&s, P(0), P(1), P(2), P(3), P(4), P(5), P(6), P(7), P(8), ws - 1, NULL), KDA_ERR_WORKSPACE);
    EXPECT(kda_chunk_fwd_ex(&s, 8u, P(0), P(1), P(2), P(3), P(4), P(5), P(6), P(7), P(8), ws, NULL), KDA_ERR_FLAGS);
    EXPECT(kda_chunk_fwd(&z, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL), KDA_OK);
    /* packed sequences */
    EXPECT(kda_chunk_fwd_varlen(&s, 0u, NULL, 64, P(0), P(1), P(2), P(3), P(4), P(5), P(6), P(7), P(8), ws, NULL), KDA_ERR_NULL);
    EXPECT(kda_chunk_fwd_varlen(&s, 0u, (const int32_t*)P(9), -1, P(0), P(1), P(2), P(3), P(4), P(5), P(6), P(7), P(8), ws, NULL), KDA_ERR_SHAPE);
    /* decode */
    kda_shape d = shp(4, 8, 1, 128, 64, KDA_BF16, KDA_F32, KDA_ALPHA_HEAD);
    EXPECT(kda_decode_step(&d, P(0), P(1), (char*)P(2) + 4, P(3), P(4), (float*)P(5), P(6), NULL), KDA_ERR_ALIGN);
    kda_shape d2 = d;
    d2.L = 2;
    EXPECT(kda_decode_step(&d2, P(0), P(1), P(2), P(3), P(4), (float*)P(5), P(6), NULL), KDA_ERR_SHAPE);
    EXPECT(kda_decode_step(&d, P(0), P(1), P(2), P(3), P(4), (float*)P(5), (char*)P(5) + 64, NULL), KDA_ERR_ALIAS);
    EXPECT(kda_decode_step_slots(&d, P(0), P(1), P(2), P(3), P(4), (float*)P(5), 4, NULL, P(6), NULL), KDA_ERR_NULL);
    EXPECT(kda_decode_step_slots(&d, P(0), P(1), P(2), P(3), P(4), (float*)P(5), -1, (const int32_t*)P(7), P(6), NULL), KDA_ERR_SHAPE);
    EXPECT(kda_decode_step_ex(&d, 16u, P(0), P(1), P(2), P(3), P(4), (float*)P(5), P(6), NULL), KDA_ERR_FLAGS);
    /* linear attention */
    kda_shape la = shp(2, 2, 50, 64, 64, KDA_F32, KDA_F32, KDA_ALPHA_HEAD);
    EXPECT(kda_linear_attn_fwd(&la, P(0), P(1), P(2), NULL, NULL, P(6), NULL, NULL, P(8), 1 << 20, NULL), KDA_ERR_ALPHA_MODE);
    la.alpha_mode = KDA_ALPHA_NONE;
    EXPECT(kda_linear_attn_decode_step(&la, P(0), P(1), P(2), (float*)P(5), (float*)P(7), P(6), NULL), KDA_ERR_SHAPE);
    /* gradients */
    const size_t bws = kda_recurrence_bwd_workspace_bytes(&s);
    float* f = (float*)P(20);
    EXPECT(kda_recurrence_bwd(&s, P(0), P(1), P(2), P(3), P(4), NULL, P(5), NULL, (float*)P(6), (float*)P(7), (float*)P(8), (float*)P(9), (float*)P(10), NULL, f, bws - 1, NULL), KDA_ERR_WORKSPACE);
    EXPECT(kda_recurrence_bwd(&s, P(0), P(1), P(2), P(3), P(4), NULL, P(5), NULL, (float*)P(6), (float*)P(6), (float*)P(8), (float*)P(9), (float*)P(10), NULL, f, bws, NULL), KDA_ERR_ALIAS);
    const size_t bxs = kda_recurrence_bwd_ex_workspace_bytes(&s, 7u);
    EXPECT(kda_recurrence_bwd_ex(&s, 7u, P(0), P(1), P(2), P(3), P(4), NULL, P(5), NULL, (float*)P(6), (float*)((char*)f + bxs - 4096), (float*)P(8), (float*)P(9), (float*)P(10), NULL, f, bxs, NULL), KDA_ERR_ALIAS);
    EXPECT(kda_recurrence_bwd_ex(&s, 7u, P(0), P(1), P(2), P(3), P(4), NULL, P(5), NULL, (float*)P(6), (float*)P(7), (float*)P(8), (float*)P(9), (float*)P(10), NULL, f, bxs - 1, NULL), KDA_ERR_WORKSPACE);
    /* strings and timing without launches */
    for (int c = 0; c < 12; ++c)
        if (!kda_strerror(c) || !strlen(kda_strerror(c))) ++fails;
    if (kda_abi_version() != KDA_ABI_VERSION) ++fails;
    int64_t n = -1;
    double ms = -1.0;
    EXPECT(kda_timing_read("kda_intra_kernel", &n, &ms), KDA_OK);
    if (n != 0) ++fails;
    EXPECT(kda_timing_read("nope", &n, &ms), KDA_ERR_SHAPE);
    EXPECT(kda_timing_reset(), KDA_OK);
    if (fails) {
        fprintf(stderr, "%d checks failed\n", fails);
        return 1;
    }
    printf("abi sanitizer driver: ok\n");
    return 0;
}
