/*
 * kda_oracle.h -- plain fp64 CPU oracle of the KDA / gated delta rule.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the CPU
 * baseline leg of the benchmark may call this library; the product path never
 * links or loads it.  It shares no code, header or constant with the HIP
 * library.
 *
 * What it computes (per (b, h) head, row-vector convention, S is d_k x d_v):
 *
 *   S <- S0 (zero when absent)
 *   for t = 0 .. L-1:
 *       a   = exp(log_alpha_t)           per key channel / per head / 1
 *       S~  = diag(a) S                  decay acts on the d_k (row) axis
 *       u   = beta_t (v_t - k_t S~)      delta correction against the decayed state
 *       S   = S~ + k_t^T u
 *       o_t = q_t S                      read after the write
 *
 * Sources: "22580: From GPT-2 to Kimi3, Explained" (zharfai.com), sections
 * "The delta rule turns writing into editing" (the delta update and the read
 * q S), "Gated DeltaNet adds controlled forgetting" (the transition
 * alpha_t (I - beta_t k_t^T k_t) S + beta_t k_t^T v_t) and "Kimi Delta
 * Attention makes forgetting finer" (per-channel decay); "22,580: From GPT-2 to
 * Kimi K3" (yichencityu.github.io) section 6.1 (token loop: write, then read
 * q S) and section 9.1 (per-channel alpha).  The order "decay, then correct
 * against the decayed state" is the reading under which exact replacement of
 * a unit key's value holds for per-channel alpha; it coincides with the
 * printed scalar-gate formula.
 *
 * Inputs are read in their stored type (fp32, or bf16 bit patterns) and
 * widened exactly to fp64.  Columns of S evolve independently, so a caller may
 * ask for a column range only; outputs then hold those columns.
 */
#ifndef KDA_ORACLE_H
#define KDA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1, ORACLE_F64 = 2 };
enum { ORACLE_ALPHA_NONE = 0, ORACLE_ALPHA_HEAD = 1, ORACLE_ALPHA_CHANNEL = 2 };

/*
 * q, k:       [B,H,L,dk] in qkv_dtype       v: [B,H,L,dv] in qkv_dtype
 * log_alpha:  [B,H,L,dk] (channel) | [B,H,L] (head) | ignored (none), gate_dtype
 * beta:       [B,H,L] in gate_dtype
 * S0:         [B,H,dk,dv] fp64, or NULL for a zero state
 * col0,ncols: the d_v columns to compute, [col0, col0 + ncols)
 * delta:      1 = delta rule; 0 = additive write u = beta v (a diagnostic mode)
 * o:          [B,H,L,ncols] fp64 (may be NULL)
 * S_final:    [B,H,dk,ncols] fp64 (may be NULL)
 * nthreads:   worker threads (<= 0: 1).  Results do not depend on it.
 * Returns 0, or -1 on a bad argument.
 */
int kda_oracle_forward(int64_t B, int64_t H, int64_t L, int64_t dk, int64_t dv,
                       int qkv_dtype, int gate_dtype, int alpha_mode,
                       const void* q, const void* k, const void* v,
                       const void* log_alpha, const void* beta,
                       const double* S0, int64_t col0, int64_t ncols, int delta,
                       double* o, double* S_final, int nthreads);

#ifdef __cplusplus
}
#endif
#endif
