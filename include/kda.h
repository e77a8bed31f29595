/*
 * kda.h -- C ABI of the MI355X (gfx950) KDA / gated delta rule library.
 *
 * The operation (per batch b and head h; row vectors; S is d_k x d_v):
 *
 *     S~  = diag(alpha_t) S             decay, one factor per key channel
 *     u   = beta_t (v_t - k_t S~)       delta-rule correction
 *     S   = S~ + k_t^T u                write
 *     o_t = q_t S                       read (after the write)
 *
 * i.e. S_t = (I - beta_t k_t^T k_t) diag(alpha_t) S_(t-1) + beta_t k_t^T v_t,
 * o_t = q_t S_t.  Sources: "22580: From GPT-2 to Kimi3, Explained"
 * (zharfai.com), sections "The delta rule turns writing into editing",
 * "Gated DeltaNet adds controlled forgetting" and "Kimi Delta Attention makes
 * forgetting finer"; "22,580: From GPT-2 to Kimi K3" (yichencityu.github.io),
 * sections 5.2 (delta update), 6.1 (token loop: write then read), 6.3 (the
 * chunkwise WY form) and 9.1 (per-channel alpha).  The decay is applied before
 * the correction, so a unit key written with beta = 1 reads back its value
 * exactly for any per-channel alpha.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensors are dense, row-major, contiguous device buffers owned by the
 *   caller.  q, k: [B,H,L,dk]; v, o: [B,H,L,dv]; beta: [B,H,L];
 *   log_alpha: [B,H,L,dk] (KDA_ALPHA_CHANNEL) or [B,H,L] (KDA_ALPHA_HEAD) or
 *   unused (KDA_ALPHA_NONE, alpha = 1; may be NULL).  States are fp32
 *   [B,H,dk,dv] with d_v contiguous.  Decode drops the L axis (L must be 1).
 * - log_alpha holds ln(alpha_t), which must be finite and <= 0; any such
 *   value is supported (alpha may underflow to 0, which wipes the channel).
 *   The prefill kernels split each per-channel decay factor at 16-token
 *   sub-block boundaries so that no intermediate leaves the float range; a
 *   sub-block whose summed ln(alpha) falls below -69 in some channel has its
 *   diagonal blocks summed directly (slower, same result).  beta should be
 *   in [0, 1].  Neither is checked; NaN or Inf stays inside its own (b, h).
 * - q, k, v and o share qkv_dtype; log_alpha and beta share gate_dtype.
 *   Arithmetic: fp32 inputs are computed entirely in fp32 (fp32 MFMA); bf16
 *   inputs use bf16 MFMA operands with fp32 accumulation, and the state is
 *   fp32 throughout.  o is rounded to its dtype with round-to-nearest-even.
 * - Supported sizes: dk, dv in {64, 128}; B, H, L >= 0 (any L: a ragged last
 *   chunk is handled in the kernel).  Every pointer must be 16-byte aligned.
 * - Calls are asynchronous on hip_stream (a hipStream_t; NULL = the null
 *   stream).  Outputs are valid once that stream has been synchronized.  The
 *   library allocates no device memory, keeps no per-call state and is safe
 *   to call from several host threads.
 * - Return value: KDA_OK (0) or a kda_status code.  Every check except
 *   KDA_ERR_HIP is made on the host before any HIP call, so a rejected call
 *   touches neither the device nor any buffer.  A fault inside a kernel is
 *   reported by the stream, not here.
 * - Diagnostics: with the environment variable KDA_LOG set to anything but
 *   "" or "0" (read once per process), every call writes to stderr one line
 *   with its shape and flags, the prefill calls one more with their plan
 *   (chunks, spans, record and workspace bytes, the state pass and its slice
 *   width), and any call that does not return KDA_OK one with its status (and
 *   HIP's message for KDA_ERR_HIP); each line starts with "[kda] ".  Every
 *   call is also one roctx range (rocprofiler-sdk) named after the entry
 *   point, which `rocprofv3 --marker-trace` records around the kernels the
 *   call launched.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 1

enum kda_dtype { KDA_F32 = 0, KDA_BF16 = 1 };

enum kda_alpha_mode {
    KDA_ALPHA_NONE = 0,    /* alpha = 1: DeltaNet                          */
    KDA_ALPHA_HEAD = 1,    /* one decay per token and head: Gated DeltaNet */
    KDA_ALPHA_CHANNEL = 2  /* one decay per token, head and key channel: KDA */
};

enum kda_status {
    KDA_OK = 0,
    KDA_ERR_NULL = 1,       /* a required pointer is NULL                     */
    KDA_ERR_SHAPE = 2,      /* negative size, unsupported dk/dv, size overflow,
                               or L != 1 for decode                           */
    KDA_ERR_DTYPE = 3,      /* qkv_dtype or gate_dtype not a kda_dtype        */
    KDA_ERR_ALPHA_MODE = 4, /* alpha_mode not a kda_alpha_mode                */
    KDA_ERR_ALIGN = 5,      /* a pointer is not 16-byte aligned               */
    KDA_ERR_WORKSPACE = 6,  /* workspace smaller than the size query returns  */
    KDA_ERR_ALIAS = 7,      /* an output overlaps an input, or S_final only
                               partly overlaps S0                             */
    KDA_ERR_HIP = 8,        /* a HIP launch failed; kda_last_error() has text */
    KDA_ERR_FLAGS = 9,      /* an unknown kda_input_flags bit                 */
    KDA_ERR_SCRATCH = 10    /* kda_chunk_fwd_noalloc: the problem needs more
                               work memory than its static buffer holds       */
};

/*
 * Input preprocessing fused into the kernels' loads (kda_chunk_fwd_ex,
 * kda_decode_step_ex, kda_decode_step_slots_ex).  The token mixer's layer feeds the recurrence with
 * L2-normalized q and k, beta = sigmoid(x W_beta) and alpha = exp(-exp(g))
 * ("22,580: From GPT-2 to Kimi K3" (yichencityu.github.io), section 5.2: the
 * DeltaNet layer normalizes q and k, which makes reading a written key exact,
 * and squashes beta with a sigmoid; "22580: From GPT-2 to Kimi K3, Explained"
 * (lukebest.github.io), "Key code and formulas", "KDA (per-channel alpha)":
 * alpha = exp(-exp(g))).
 * With these bits the caller passes the raw values and the kernels apply the
 * step as they load them, so no preprocessed copy goes through memory:
 *   KDA_IN_NORM_QK     q, k are raw: the op uses q / max(|q|, 1e-12) and the
 *                      same for k (L2 over d_k, per token and head)
 *   KDA_IN_BETA_LOGIT  beta holds logits: the op uses sigmoid(beta)
 *   KDA_IN_GATE_RAW    log_alpha holds g: the op uses ln(alpha) = -exp(g)
 *                      (ignored with KDA_ALPHA_NONE)
 */
enum kda_input_flags {
    KDA_IN_NORM_QK = 1,
    KDA_IN_BETA_LOGIT = 2,
    KDA_IN_GATE_RAW = 4
};

typedef struct kda_shape {
    int64_t B, H, L, dk, dv; /* L = 1 for decode */
    int32_t qkv_dtype;       /* enum kda_dtype: q, k, v and o                 */
    int32_t gate_dtype;      /* enum kda_dtype: log_alpha and beta            */
    int32_t alpha_mode;      /* enum kda_alpha_mode                           */
} kda_shape;

/*
 * Chunkwise-parallel prefill ("22,580: From GPT-2 to Kimi K3", section 6.3:
 * chunks of C = 64 tokens; inside a chunk the delta corrections are solved at
 * once through the WY factors T = (I + A)^-1 found by forward substitution,
 * and one state is carried from chunk to chunk).  Per (b, h) it runs the
 * recurrence above over all L tokens, starting from S0.
 *
 *   S0       [B,H,dk,dv] fp32 initial state, or NULL for a zero state.
 *   o        [B,H,L,dv] output in qkv_dtype.  Must not overlap any input or
 *            S_final.
 *   S_final  [B,H,dk,dv] fp32 final state, or NULL to skip it.  May be the
 *            same buffer as S0 (in-place update); any other overlap with S0
 *            or with an input is an error.
 *   workspace, workspace_bytes: device scratch of at least
 *            kda_chunk_fwd_workspace_bytes(shape) bytes (may be NULL when that
 *            is 0).  The library does not keep it after the call's kernels end.
 */
int kda_chunk_fwd(const kda_shape* shape, const void* q, const void* k, const void* v,
                  const void* log_alpha, const void* beta, const float* S0, void* o,
                  float* S_final, void* workspace, size_t workspace_bytes,
                  void* hip_stream);

/* kda_chunk_fwd on raw inputs: flags is a set of kda_input_flags (0 gives
 * kda_chunk_fwd exactly); KDA_ERR_FLAGS for an unknown bit.  Same workspace. */
int kda_chunk_fwd_ex(const kda_shape* shape, uint32_t flags, const void* q, const void* k,
                     const void* v, const void* log_alpha, const void* beta, const float* S0,
                     void* o, float* S_final, void* workspace, size_t workspace_bytes,
                     void* hip_stream);

/* Bytes of device workspace kda_chunk_fwd needs for this shape (0 for a
 * shape the call would reject). */
size_t kda_chunk_fwd_workspace_bytes(const kda_shape* shape);

/*
 * kda_chunk_fwd_ex without a workspace argument and without any device
 * allocation, for callers that cannot allocate: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The work
 * memory (the per-chunk records of one span of chunks, and with several spans
 * and no S_final the state carried between them) is a static device buffer of
 * KDA_NOALLOC_SCRATCH_BYTES inside the library: one per GPU, at its own
 * address, held until the process ends.  The span plan is shortened so that
 * it fits (results equal kda_chunk_fwd_ex's bit for bit).  The buffer of the
 * calling thread's current device is used, so hip_stream must belong to that
 * device.
 *   Arguments, layouts and checks: as kda_chunk_fwd_ex, without workspace.
 *   Errors: as kda_chunk_fwd_ex, plus KDA_ERR_SCRATCH when one chunk of every
 *   head (and the state area) does not fit in the buffer (e.g. more than 896
 *   heads with per-channel decay at dk = dv = 128 in bf16); that check runs
 *   on the host before any HIP call.  KDA_ERR_HIP if the buffer's device
 *   address cannot be looked up.
 *   Concurrency: every call on a GPU shares that GPU's buffer, which keeps the
 *   last call's contents (nothing in it needs to start at zero).  Calls that
 *   overlap in time on one GPU (other streams, other host threads) race on
 *   it; serialize them.  No event is recorded even with kda_timing_enable.
 */
#define KDA_NOALLOC_SCRATCH_BYTES (64ll << 20)
int kda_chunk_fwd_noalloc(const kda_shape* shape, uint32_t flags, const void* q, const void* k,
                          const void* v, const void* log_alpha, const void* beta,
                          const float* S0, void* o, float* S_final, void* hip_stream);

/*
 * One decode step for every (b, h): the recurrence above for a single token,
 * updating S in place ("22,580: From GPT-2 to Kimi K3", section 5.2 and
 * section 08's gate; "22580: From GPT-2 to Kimi3, Explained", "Gated DeltaNet
 * adds controlled forgetting").  shape->L must be 1.
 *
 *   q, k     [B,H,dk]; v, o: [B,H,dv]; log_alpha [B,H,dk] | [B,H] | unused;
 *   beta     [B,H].
 *   S        [B,H,dk,dv] fp32, read and overwritten with the new state.
 *   o        must not overlap S or any input.
 */
int kda_decode_step(const kda_shape* shape, const void* q, const void* k, const void* v,
                    const void* log_alpha, const void* beta, float* S, void* o,
                    void* hip_stream);

/*
 * Decode step over a pool of states, for serving: sequence b of this step
 * (shape->B sequences, shape->L == 1) reads and updates state slot slots[b]
 * of S_pool, so a server keeps one state per live request and steps any
 * subset of them without gathering or scattering states ("22,580: From GPT-2
 * to Kimi K3", section 5.2: the fixed-size state is the whole per-request
 * cache).  Same recurrence and the same q, k, v, log_alpha, beta, o layouts
 * as kda_decode_step.
 *
 *   S_pool   [n_slots,H,dk,dv] fp32, updated in place at the used slots only.
 *   n_slots  number of states in the pool (>= 0).
 *   slots    device int32 [B]: the slot of each sequence.  A value outside
 *            [0, n_slots) marks an idle sequence: its o is written as zeros
 *            and no state is read or written.  Two sequences of one call must
 *            not share a slot (their updates would race); this is not checked,
 *            since slots lives in device memory.  4-byte aligned.
 * Errors as kda_decode_step, plus KDA_ERR_NULL for slots == NULL (B*H > 0)
 * and KDA_ERR_SHAPE for n_slots < 0.  slots must not overlap o or S_pool.
 */
int kda_decode_step_slots(const kda_shape* shape, const void* q, const void* k, const void* v,
                          const void* log_alpha, const void* beta, float* S_pool,
                          int64_t n_slots, const int32_t* slots, void* o, void* hip_stream);

/*
 * Prefill of a batch of packed variable-length sequences, for serving: each
 * sequence runs the recurrence of kda_chunk_fwd over its own tokens from its
 * own initial state, chunks never cross a sequence boundary, and no padding
 * is stored or computed ("22,580: From GPT-2 to Kimi K3", section 6.3 for the
 * chunk algorithm; section 5.2 for the per-sequence state the decode steps
 * then continue).
 *   shape       B = number of sequences N, L = T = total tokens, H, dk, dv,
 *               dtypes and alpha_mode as for kda_chunk_fwd.
 *   cu_seqlens  device int32 [N + 1]: sequence i owns tokens cu_seqlens[i] ..
 *               cu_seqlens[i+1] - 1.  Must be nondecreasing with
 *               cu_seqlens[0] = 0 and cu_seqlens[N] = T; the kernels clamp it
 *               to [0, T] (a malformed table gives undefined results but no
 *               access outside the tensors).  4-byte aligned; an input.
 *   max_seqlen  host: >= every sequence length (the chunk plan and the
 *               workspace follow min(max_seqlen, T)); tokens of a longer
 *               sequence beyond it are not processed.
 *   q, k        [H, T, dk]; v, o [H, T, dv]; log_alpha [H, T, dk] | [H, T];
 *               beta [H, T]  (sequence i of head h at rows h T + cu_seqlens[i]..)
 *   S0, S_final [N, H, dk, dv] fp32, per sequence (NULL as for kda_chunk_fwd).
 *   flags       kda_input_flags, as for kda_chunk_fwd_ex.
 *   workspace   >= kda_chunk_fwd_varlen_workspace_bytes(shape, max_seqlen).
 * Errors as for kda_chunk_fwd_ex, plus KDA_ERR_SHAPE for max_seqlen < 0 and
 * KDA_ERR_NULL for a NULL cu_seqlens with N > 0.
 */
int kda_chunk_fwd_varlen(const kda_shape* shape, uint32_t flags, const int32_t* cu_seqlens,
                         int64_t max_seqlen, const void* q, const void* k, const void* v,
                         const void* log_alpha, const void* beta, const float* S0, void* o,
                         float* S_final, void* workspace, size_t workspace_bytes,
                         void* hip_stream);
/* Device workspace bytes kda_chunk_fwd_varlen needs (0 if it would reject the
 * shape or max_seqlen). */
size_t kda_chunk_fwd_varlen_workspace_bytes(const kda_shape* shape, int64_t max_seqlen);

/*
 * Normalized linear attention with the feature map phi(x) = elu(x) + 1, the
 * recurrent mixer the delta rule improves on ("22,580: From GPT-2 to Kimi K3"
 * (yichencityu.github.io), section 04; "22,580: GPT-2 to Kimi K3, explained"
 * (zharfai.com), "Linear attention collapses history into a fixed state").
 * Per (b, h), with phi applied to the raw q_t and k_t:
 *     S_t = S_{t-1} + phi(k_t)^T v_t      z_t = z_{t-1} + phi(k_t)
 *     o_t = phi(q_t) S_t / (phi(q_t) . z_t)
 * (read after the write, as for kda_chunk_fwd), computed chunkwise with the
 * same state pass as kda_chunk_fwd's one-decay path, without the delta term.
 *   shape      alpha_mode must be KDA_ALPHA_NONE (else KDA_ERR_ALPHA_MODE);
 *              gate_dtype is not used.
 *   q, k       [B,H,L,dk] raw (before phi); v, o [B,H,L,dv] in qkv_dtype.
 *   S0, z0     [B,H,dk,dv] and [B,H,dk] fp32 initial state and normalizer,
 *              or NULL for zero.  With S0 = z0 = 0 the first token gives
 *              o_1 = v_1.
 *   S_final, z_final  [B,H,dk,dv], [B,H,dk] fp32 outputs or NULL; each may be
 *              the same buffer as S0 / z0 (in place).
 *   workspace  device scratch of kda_linear_attn_fwd_workspace_bytes(shape)
 *              bytes: phi(q) in qkv_dtype, written once per call and read by
 *              the state pass; not kept after the call.
 * Errors and checks as for kda_chunk_fwd.
 */
int kda_linear_attn_fwd(const kda_shape* shape, const void* q, const void* k, const void* v,
                        const float* S0, const float* z0, void* o, float* S_final,
                        float* z_final, void* workspace, size_t workspace_bytes,
                        void* hip_stream);
/* Workspace bytes kda_linear_attn_fwd needs (0 if it would reject the shape). */
size_t kda_linear_attn_fwd_workspace_bytes(const kda_shape* shape);

/*
 * One decode step of the same normalized linear attention for every (b, h):
 * S += phi(k)^T v and z += phi(k) in place, o = phi(q) S / (phi(q) . z).
 *   shape   L = 1, alpha_mode KDA_ALPHA_NONE (else KDA_ERR_SHAPE /
 *           KDA_ERR_ALPHA_MODE); gate_dtype is not used.
 *   q, k    [B,H,dk] raw; v, o [B,H,dv] in qkv_dtype.
 *   S, z    [B,H,dk,dv] and [B,H,dk] fp32, read and updated in place (the
 *           S_final / z_final of kda_linear_attn_fwd continue here).
 * Outputs overlap no input and each other (KDA_ERR_ALIAS).
 */
int kda_linear_attn_decode_step(const kda_shape* shape, const void* q, const void* k,
                                const void* v, float* S, float* z, void* o, void* hip_stream);

/*
 * Kernel timing, for measurement tools (not part of the computation).  While
 * timing is on, every kernel that kda_chunk_fwd or kda_decode_step launches is
 * bracketed by two HIP events recorded on the call's stream; the event pairs
 * are kept until kda_timing_reset.  The events add a few microseconds of
 * stream work per launch and nothing else changes.
 *
 *   kda_timing_enable(on)   on != 0 starts recording for later calls, 0 stops.
 *   kda_timing_reset()      destroys every kept event pair.  KDA_ERR_HIP if a
 *                           destroy failed.
 *   kda_timing_read(name, &launches, &total_ms)
 *                           waits for the kept launches of the kernel `name`
 *                           ("kda_intra_kernel", "kda_inter_kernel",
 *                           "kda_inter_scalar_kernel", "kda_inter_wide_kernel",
 *                           "kda_inter_quad_kernel",
 *                           "kda_decode_kernel",
 *                           "kda_feature_map_kernel" or "kda_bwd_kernel")
 *                           and returns how many there were and their summed
 *                           duration in milliseconds.  KDA_ERR_NULL for a NULL
 *                           argument, KDA_ERR_SHAPE for an unknown name,
 *                           KDA_ERR_HIP if an event query failed.
 *
 * The three calls share one process-wide record; use them from one thread.
 */
int kda_timing_enable(int on);
int kda_timing_reset(void);
int kda_timing_read(const char* kernel, int64_t* launches, double* total_ms);

/* kda_decode_step and kda_decode_step_slots on raw inputs: flags is a set of
 * kda_input_flags, as for kda_chunk_fwd_ex (0 gives the plain call exactly;
 * KDA_ERR_FLAGS for an unknown bit, checked after the shape).  Every other
 * argument, its layout, ownership and check is that of the plain call; the
 * raw q and k are normalized per (b, h) over d_k, so no copy is written. */
int kda_decode_step_ex(const kda_shape* shape, uint32_t flags, const void* q, const void* k,
                       const void* v, const void* log_alpha, const void* beta, float* S, void* o,
                       void* hip_stream);
int kda_decode_step_slots_ex(const kda_shape* shape, uint32_t flags, const void* q,
                             const void* k, const void* v, const void* log_alpha,
                             const void* beta, float* S_pool, int64_t n_slots,
                             const int32_t* slots, void* o, void* hip_stream);

/*
 * Gradients of the recurrence above through all L tokens of every (b, h), for
 * training: given dJ/do and dJ/dS_final, the reverse sweep of the step (its
 * chain rule; the forward step is the one of "22,580: From GPT-2 to Kimi K3",
 * section 5.2 with section 08's decay) gives dJ/dq, dJ/dk, dJ/dv,
 * dJ/dln(alpha), dJ/dbeta and dJ/dS0.  It runs token by token (the state is
 * recomputed from checkpoints taken every 8 tokens), not in chunkwise form.
 *
 *   q, k, v, log_alpha, beta, S0: the inputs of kda_chunk_fwd (preprocessed
 *            values: no kda_input_flags), same layouts and dtypes.
 *   dout     [B,H,L,dv] in qkv_dtype: dJ/do.
 *   dS_final [B,H,dk,dv] fp32 dJ/dS_final, or NULL for zero.
 *   dq, dk   [B,H,L,dk] fp32;  dv [B,H,L,dv] fp32;  dbeta [B,H,L] fp32.
 *   dlog_alpha  fp32 with log_alpha's layout ([B,H,L,dk] or [B,H,L]);
 *            unused (may be NULL) with KDA_ALPHA_NONE.
 *   dS0      [B,H,dk,dv] fp32, or NULL to skip it (with S0 NULL it is the
 *            gradient with respect to a zero initial state).
 *   workspace, workspace_bytes: device scratch of at least
 *            kda_recurrence_bwd_workspace_bytes(shape) bytes
 *            (B*H*ceil(L/8)*dk*dv*4); not kept after the call's kernels end.
 * The outputs are written in full (dq, dk, dlog_alpha and dbeta are zeroed on
 * the stream first, then accumulated with float atomics, so their last bits
 * may differ between runs).  Outputs must not overlap each other, the
 * workspace or any input (KDA_ERR_ALIAS).  All pointers 16-byte aligned.
 * Errors as for kda_chunk_fwd; KDA_ERR_NULL for a missing required gradient.
 */
int kda_recurrence_bwd(const kda_shape* shape, const void* q, const void* k, const void* v,
                       const void* log_alpha, const void* beta, const float* S0,
                       const void* dout, const float* dS_final, float* dq, float* dk,
                       float* dv, float* dlog_alpha, float* dbeta, float* dS0, void* workspace,
                       size_t workspace_bytes, void* hip_stream);

/* Bytes of device workspace kda_recurrence_bwd needs (0 for a rejected shape). */
size_t kda_recurrence_bwd_workspace_bytes(const kda_shape* shape);

/*
 * The same gradients as kda_recurrence_bwd, in chunkwise form: the chunk form
 * of "22,580: From GPT-2 to Kimi K3" (yichencityu.github.io), section 6.3 with
 * section 9.1's per-channel decay, differentiated, which is what "Chunkwise
 * DeltaNet makes the recurrence trainable on GPUs" ("22580: From GPT-2 to
 * Kimi3, Explained", zharfai.com) asks of it.  The forward's intra-chunk
 * kernel writes every chunk's factors (and T^T); a scan of the forward state
 * pass keeps the state entering each chunk; the reverse recursion of dJ/dS,
 * dJ/dS_in = diag(e^{g_n}) dJ/dS_out + (Q e^g)^T dO - W^T du with
 * du = P^T dO + (K e^{g_n-g}) dJ/dS_out, runs as the same state pass over
 * records rebuilt from the forward ones; every chunk's gradients then follow
 * independently on the matrix cores.
 *
 *   Arguments, layouts, ownership and errors as for kda_recurrence_bwd, except:
 *   qkv_dtype must be KDA_BF16 (q, k, v and dout bf16; KDA_ERR_DTYPE
 *            otherwise); every decay mode and gate dtype is accepted.
 *   workspace_bytes >= kda_chunk_bwd_workspace_bytes(shape): the forward's
 *            chunk records of the whole sequence, one reverse record per
 *            chunk, T^T and four states per chunk (about 5.3 KiB per token
 *            and head at d_k = d_v = 128); not kept after the call's
 *            kernels end.
 *   Arithmetic: bf16 operands on the matrix cores with fp32 accumulation, as
 *            the forward's chunked prefill; every output is written once (no
 *            atomics), so repeated calls give the same bits.
 */
int kda_chunk_bwd(const kda_shape* shape, const void* q, const void* k, const void* v,
                  const void* log_alpha, const void* beta, const float* S0, const void* dout,
                  const float* dS_final, float* dq, float* dk, float* dv, float* dlog_alpha,
                  float* dbeta, float* dS0, void* workspace, size_t workspace_bytes,
                  void* hip_stream);

/* Bytes of device workspace kda_chunk_bwd needs (0 for a rejected shape or L = 0). */
size_t kda_chunk_bwd_workspace_bytes(const kda_shape* shape);

/*
 * kda_recurrence_bwd on raw inputs: flags is a set of kda_input_flags, as for
 * kda_chunk_fwd_ex, and the gradients are with respect to the raw values the
 * caller passes (through the q/k normalization, the beta sigmoid and
 * ln alpha = -exp(g)).  The inputs are preprocessed into fp32 copies in the
 * workspace, the gradient kernel runs on them, and the chain rule of each
 * flagged step is applied to its outputs in place.  workspace_bytes >=
 * kda_recurrence_bwd_ex_workspace_bytes(shape, flags) (0 for L = 0, where
 * the call is kda_recurrence_bwd's).  Arguments, layouts, ownership and
 * errors as for kda_recurrence_bwd; KDA_ERR_FLAGS for an unknown bit.
 */
int kda_recurrence_bwd_ex(const kda_shape* shape, uint32_t flags, const void* q, const void* k,
                          const void* v, const void* log_alpha, const void* beta,
                          const float* S0, const void* dout, const float* dS_final, float* dq,
                          float* dk, float* dv, float* dlog_alpha, float* dbeta, float* dS0,
                          void* workspace, size_t workspace_bytes, void* hip_stream);
size_t kda_recurrence_bwd_ex_workspace_bytes(const kda_shape* shape, uint32_t flags);

/* Static text for a kda_status code. */
const char* kda_strerror(int status);

/* Text of the last KDA_ERR_HIP seen on the calling thread ("" if none). */
const char* kda_last_error(void);

/* KDA_ABI_VERSION of the loaded library. */
int kda_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* KDA_H */
