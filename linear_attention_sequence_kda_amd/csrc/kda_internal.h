// kda_internal.h -- launch interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda.h"

namespace kda {

// ---- two-kernel prefill --------------------------------------------------
// The intra-chunk kernel writes, per (b,h) head and chunk, one record of the
// chunk's state-independent factors; the inter-chunk kernel walks the chunks
// in order and carries the state.  With per-channel decay (KDA) the record
// holds every operand of the state pass; its sections (byte offsets, each
// 256-byte aligned), C = chunk length, E = the q/k/v element type:
//   w    W   = T diag(beta e^g) K     [C][DK]  E, fragment order (rows = token)
//   ut   U   = T diag(beta) V         [C][DV]  E, accumulator order
//   p    P   (decayed causal Q K^T)   [C][C]   E, fragment order (rows = token)
//   kt   K^T (KDA: (K e^{g_n-g})^T)   [DK][C]  E, fragment order (rows = channel)
//   qt   Q (KDA: Q e^g)               [C][DK]  E, fragment order (rows = token)
//   gam  KDA only: e^{g_n} per key channel, DK floats (section of >= 1 KiB)
//   rs   scalar decay only: e^{g_r} [C], e^{g_n-g_r} [C], e^{g_n}, fp32
//        (section of >= 1 KiB)
// "Fragment order" stores an operand with rows m and contraction index k the
// way a 16x16 MFMA tile loop consumes it: 16-byte pieces (W = 16/sizeof(E)
// consecutive k) of row m, piece index ((m/16) * (K/KS) + k/KS) * 64 + lane,
// lane = ((k % KS) / W) * 16 + m % 16, KS = 4 W, so each lane of a wave reads
// its operand for one k step of one 16-row block with one 16-byte load and the
// 64 lanes read 1 KiB of contiguous memory.  "Accumulator order" stores the
// 16x16 blocks (R, vb) of U as lane-major quads, PF = 16 / (4 sizeof(E))
// column blocks side by side in each lane's 16 bytes: element
// (16R + 4(l/16) + i, 16vb + l%16) at
// ((R * DV/(16 PF) + vb/PF) * 64 + l) * 4 PF + (vb % PF) * 4 + i.
struct RecLayout {
    uint32_t w, ut, p, kt, qt, gam, rs, tb, bytes;
};
__host__ __device__ constexpr uint32_t rec_align(uint32_t x) { return (x + 255u) & ~255u; }
__host__ __device__ constexpr RecLayout rec_layout(int dk, int dv, int c, int esz, bool kda) {
    RecLayout r{0, 0, 0, 0, 0, 0, 0, 0, 0};
    uint32_t o = 0;
    r.w = o;
    o = rec_align(o + (uint32_t)(c * dk * esz));
    r.ut = o;
    o = rec_align(o + (uint32_t)(c * dv * esz));
    r.p = o;
    o = rec_align(o + (uint32_t)(c * c * esz));
    r.kt = o;
    o = rec_align(o + (uint32_t)(dk * c * esz));
    r.qt = o;
    o = rec_align(o + (uint32_t)(c * dk * esz));
    // the decay scalars take one whole 1 KiB piece (the inter-chunk kernel
    // copies records in 1 KiB pieces)
    r.gam = o;
    if (kda) o = rec_align(o + (uint32_t)(dk * 4 > 1024 ? dk * 4 : 1024));
    r.rs = o;
    if (!kda) o = rec_align(o + (uint32_t)((2 * c + 4) * 4 > 1024 ? (2 * c + 4) * 4 : 1024));
    r.bytes = o;
    return r;
}

// Record of the scalar-decay path ("thin": the inter-chunk kernel reads q, k
// and v itself and only needs the solved triangle and the decay scalars):
//   tb   T diag(beta)                 [C][C]   E, row-major, zero above the diagonal
//   rs   g_r [C], e^{g_r} [C], e^{g_n-g_r} [C], and with KDA_IN_NORM_QK
//        1/|k_r| [C] (0 past the sequence end); fp32, 1 KiB section.
//        e^{g_n} is e^{g_r} at r = C-1 (padded tokens keep g).
__host__ __device__ constexpr RecLayout rec_layout_thin(int c, int esz) {
    RecLayout r{0, 0, 0, 0, 0, 0, 0, 0, 0};
    r.tb = 0;
    r.rs = rec_align((uint32_t)(c * c * esz));
    r.bytes = r.rs + rec_align((uint32_t)(4 * c * 4 > 1024 ? 4 * c * 4 : 1024));
    return r;
}

// Chunk length of the prefill kernels: 64 tokens with bf16 operands, 32 in fp32.
constexpr int chunk_len(int qkv_bf16) { return qkv_bf16 ? 64 : 32; }

// Token range of workgroup head bh in the [*, d] input rows: rows base ..
// base + len - 1.  Dense layout ([BH, L, d]): base = bh L, len = L.  Packed
// sequences (cu != null, L = T total tokens, [H, T, d] tensors): bh = i H + h
// is head h of sequence i, which owns tokens cu[i] .. cu[i+1] - 1; the table
// is clamped to [0, T], so a malformed one cannot move an access outside the
// tensors.
struct SeqRange {
    int64_t base, len;
};
__device__ __forceinline__ SeqRange seq_range(const int32_t* cu, int64_t L, int H, int bh) {
    if (!cu) return SeqRange{(int64_t)bh * L, L};
    const int i = bh / H, h = bh - i * H;
    int64_t s = cu[i], e = cu[i + 1];
    s = s < 0 ? 0 : (s > L ? L : s);
    e = e < s ? s : (e > L ? L : e);
    return SeqRange{(int64_t)h * L + s, e - s};
}

struct IntraParams {
    const void* q;          // [BH, L, DK]  qkv type
    const void* k;          // [BH, L, DK]
    const void* v;          // [BH, L, DV]
    const void* log_alpha;  // [BH, L, DK] | [BH, L] | unused, gate type
    const void* beta;       // [BH, L] gate type
    void* ws;               // records [BH][ncs]
    int64_t L;
    int64_t c0;             // first chunk of this span
    int ncs;                // chunks in this span
    int BH;
    int gate_bf16;
    uint32_t flags = 0;     // kda_input_flags
    const int32_t* cu = nullptr;  // packed sequences: [B + 1] token offsets
    int H = 1;              // heads per sequence (packed sequences)
    // per-channel decay, bf16: write the record in the wide state pass's
    // order (W negated, W / Q~ / P / K^T in wide_elem order)
    int wide = 0;
    // per-channel decay: also write T^T = ((I + A)^-1)^T of every chunk,
    // fp32 [BH][ncs][C][C] row-major (chunkwise gradients), or null
    float* tt = nullptr;
    // per-channel decay computed from one ln(alpha) per token ([BH, L]), which
    // every channel reads (chunkwise gradients of a head gate)
    int la_head = 0;
    // chunkwise gradients: also build each chunk's reverse record (reverse
    // chunk order, rev_rec_bytes each) from the record just written and
    // dJ/do ([BH, L, DV] bf16); requires the wide order, c0 = 0, ncs = all chunks
    void* rrecs = nullptr;
    const void* dout = nullptr;
};

struct InterParams {
    const void* q;          // [BH, L, DK]  (scalar-decay kernel)
    const void* k;          // [BH, L, DK]  (scalar-decay kernel)
    const void* v;          // [BH, L, DV]  (scalar-decay kernel)
    const void* ws;         // records [BH][ncs] written by the intra-chunk kernel
    const float* S_in;      // [BH, DK, DV] or null (zero state)
    float* S_out;           // [BH, DK, DV] or null; may equal S_in
    void* o;                // [BH, L, DV]  qkv type
    int64_t L;
    int64_t c0;
    int ncs;
    int BH;
    int DV;
    int n_slices;           // DV / slice width (set by launch_inter)
    uint32_t flags = 0;     // kda_input_flags (the scalar kernel normalizes q, k)
    const int32_t* cu = nullptr;  // packed sequences, as in IntraParams
    int H = 1;
    // normalized linear attention (scalar kernel only): no records; the
    // normalizer z [BH, DK] fp32 in (null: zero) and out (null: not written)
    int linear_attn = 0;
    const float* z_in = nullptr;
    float* z_out = nullptr;
    // scan form of the wide state pass (launch_inter_wide_scan): no o; the
    // state entering chunk x (fp32) and that chunk's u = U - W S (bf16) are
    // written for every chunk x with x % 2^scan_shift == 0, as entry
    // x >> scan_shift of S_all [BH][n_store][DK][DV] and u_all [BH][n_store][C][DV]
    float* S_all = nullptr;
    void* u_all = nullptr;
    int scan_shift = 0;
    int n_store = 0;
    // scan form over reverse records (rev_rec_bytes each): every step also
    // adds a second product, S += K2^T U2, K2^T in the record's Q~ section
    // (in K^T's order) and U2 in an extra section (in U's order)
    int rev = 0;
};

// Bytes of one reverse record: the forward record's sections, then U2 (bf16
// [C][DV] in accumulator order).
__host__ __device__ constexpr uint32_t rev_rec_bytes(int dk, int dv) {
    return rec_layout(dk, dv, 64, 2, true).bytes + rec_align((uint32_t)(64 * dv * 2));
}

// Device address of the calling thread's current device's static buffer of
// kda_chunk_fwd_noalloc (KDA_NOALLOC_SCRATCH_BYTES), looked up once per device.
hipError_t scratch_address(void** out);

hipError_t launch_intra(const IntraParams& prm, int dk, int dv, int qkv_bf16, int alpha_mode,
                        hipStream_t stream);
hipError_t launch_inter(InterParams prm, int dk, int qkv_bf16, int alpha_mode, int nv,
                        hipStream_t stream);
hipError_t launch_inter_scalar(InterParams prm, int dk, int qkv_bf16, int nv, hipStream_t stream);
// State pass for per-channel decay with bf16 operands over wide column slices
// (nv = 64 or 128 state columns per workgroup; dk, nv in {64, 128}); reads
// records written with IntraParams::wide.
hipError_t launch_inter_wide(InterParams prm, int dk, int nv, hipStream_t stream);
// Slice width of launch_inter_wide for this problem, or 0 where that pass
// does not apply (the other state passes run instead).
int wide_slice_width(int dk, int dv, int qkv_bf16, int alpha_mode, int64_t BH);
// The wide state pass in scan form (InterParams::S_all / u_all; no o), 32
// columns per workgroup.
hipError_t launch_inter_wide_scan(InterParams prm, int dk, int nv, hipStream_t stream);

// Arguments of the decode step kernel.
struct DecodeParams {
    const void* q;          // [BH, DK]
    const void* k;          // [BH, DK]
    const void* v;          // [BH, DV]
    const void* log_alpha;  // [BH, DK] | [BH] | unused
    const void* beta;       // [BH]
    float* S;               // [BH, DK, DV] (or a pool, see slots), updated in place
    void* o;                // [BH, DV]
    int BH;
    int gate_bf16;
    int alpha_mode;
    // slot mode: sequence b's state is S + (slots[b] * H + h) * DK * DV, a
    // pool of n_slots states; a slot outside [0, n_slots) marks an idle
    // sequence (o = 0, no state touched).  slots == nullptr: S is [BH, ...].
    const int32_t* slots = nullptr;
    int64_t n_slots = 0;
    int H = 1;
    uint32_t flags = 0;     // kda_input_flags
    // normalized linear attention step: z [BH, DK] fp32 normalizer, in place
    int linear_attn = 0;
    float* z = nullptr;
};

// phi(q) of normalized linear attention: n16 16-byte pieces.
struct FeatureParams {
    const void* q;
    void* fq;
    int64_t n16;
};
hipError_t launch_feature_map(const FeatureParams& prm, int qkv_bf16, hipStream_t stream);

// State-column slice width the inter-chunk kernel uses for this problem.
int chunk_slice_width(int dk, int dv, int qkv_bf16, int64_t BH);

hipError_t launch_decode(const DecodeParams& prm, int dk, int dv, int qkv_bf16,
                         hipStream_t stream);

// Arguments of the gradient kernel (reverse sweep of the recurrence).
struct BwdParams {
    const void* q;          // [BH, L, DK] qkv type
    const void* k;          // [BH, L, DK]
    const void* v;          // [BH, L, DV]
    const void* log_alpha;  // [BH, L, DK] | [BH, L] | unused; gate type
    const void* beta;       // [BH, L] gate type
    const void* dout;       // [BH, L, DV] qkv type: dJ/do
    const float* S0;        // [BH, DK, DV] or null (zero state)
    const float* dS_final;  // [BH, DK, DV] or null (zero)
    float* dq;              // [BH, L, DK]
    float* dk;              // [BH, L, DK]
    float* dv_out;          // [BH, L, DV]
    float* dlog_alpha;      // like log_alpha, fp32; unused without a decay
    float* dbeta;           // [BH, L]
    float* dS0;             // [BH, DK, DV] or null
    float* ckpt;            // bwd_workspace_bytes of scratch
    int64_t BH;
    int64_t L;
    int dv;
    int gate_bf16;
    int alpha_mode;
};
int64_t bwd_workspace_bytes(int64_t bh, int64_t L, int dk, int dv);
// zero the outputs the gradient kernel accumulates into (dq, dk, dlog_alpha, dbeta)
hipError_t zero_bwd_outputs(const BwdParams& prm, int dk, hipStream_t stream);
hipError_t launch_bwd(const BwdParams& prm, int dk, int qkv_bf16, hipStream_t stream);

// Raw-input gradients: the preprocessed fp32 copies the gradient kernel reads,
// and the chain rule applied to its outputs in place afterwards.
struct BwdPrep {
    const void *q, *k, *v, *dout, *log_alpha, *beta;  // raw inputs
    float *qn, *kn, *v32, *do32, *la32, *b32;          // [rows, dk|dv] / [rows]
    float *nq, *nk;                                    // |q|, |k| per row
    float *dq, *dk, *dlog_alpha, *dbeta;               // gradients (post, in place)
    int64_t rows;                                      // B * H * L
    int DK, DV;
    int alpha_mode;
    uint32_t flags;
};
hipError_t launch_bwd_prep(const BwdPrep& prm, int qkv_bf16, int gate_bf16, hipStream_t stream);
hipError_t launch_bwd_post(const BwdPrep& prm, hipStream_t stream);

// ---- chunkwise gradients (bf16 q/k/v/do, per-channel records) ------------------
// One decay per token (or none) widened to fp32 per-channel ln(alpha) and an
// fp32 beta, so the per-channel kernels serve every decay mode.
struct GateWiden {
    const void* log_alpha;  // [rows] | unused (alpha = 1); gate type
    const void* beta;       // [rows] gate type
    float* la;              // [rows, DK] out
    float* b;               // [rows] out
    int64_t rows;
    int DK;
    int gate_bf16;
};
hipError_t launch_gate_widen(const GateWiden& prm, hipStream_t stream);

// Chunk-parallel gradients from the two scans' per-chunk states.
struct ChunkGradParams {
    const void* q;          // [BH, L, DK] bf16
    const void* k;
    const void* v;          // [BH, L, DV] bf16
    const void* dout;       // [BH, L, DV] bf16
    const void* la;         // [BH, L, DK] per-channel ln(alpha), or one per token, gate type
    const void* beta;       // [BH, L] gate type
    const float* tt;        // [BH][nc][C][C] T^T, fp32
    const float* S_all;     // [BH][nc][DK][DV] state entering each chunk, fp32
    const void* u_all;      // [BH][nc][C][DV] u of each chunk, bf16
    const float* G_all;     // [BH][nc][DK][DV] dJ/dS leaving each chunk, fp32
    const void* du_all;     // [BH][nc][C][DV] dJ/du of each chunk, bf16
    float* dq;              // [BH, L, DK]
    float* dk;
    float* dv_out;          // [BH, L, DV]
    float* dbeta;           // [BH, L]
    float* dla;             // [BH, L, DK] (dla_mode 2), [BH, L] (1), unused (0)
    int64_t L;
    int nc;
    int BH;
    int gate_bf16;
    int dla_mode;
    int la_rs;              // elements between rows of la (DK per channel, 1 per token)
};
hipError_t launch_chunk_grad(const ChunkGradParams& prm, int dk, int dv, hipStream_t stream);

}  // namespace kda
