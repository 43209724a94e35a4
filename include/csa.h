/*
 * csa.h - C ABI of the MI355X (gfx950) library for DeepSeek-V4 Compressed
 * Sparse Attention (CSA) and Heavily Compressed Attention (HCA).
 *
 * Sources (web pages, cited by title and section):
 *   [P1] "DeepSeek V4 Inside: One Token Through Every Block"
 *   [P2] "DeepSeek-v4 Beyond Basics: A Practical Guide to mHC, CSA, HCA, and Muon"
 *   [P3] "07 The Model" (DS4 course, Phase 1 Module 1)
 *   [P4] Hugging Face transformers documentation "DeepSeek-V4"
 *
 * Conventions shared by every call
 *   - Tensors are device memory, contiguous and row-major, 16-byte aligned,
 *     owned by the caller.  The library never allocates, frees or
 *     synchronises; it launches only on the given stream (a hipStream_t
 *     passed as void*, NULL = the null stream).
 *   - `dt` is the storage type of activations, pools and outputs
 *     (CSA_F32 or CSA_BF16).  Small parameter vectors (biases, gains, head
 *     weights, sinks) are always float32.  bf16 outputs are rounded once,
 *     round-to-nearest-even, from float32 results.
 *   - Positions are absolute, 0-based token positions (int64, device).
 *   - Return value: CSA_OK or a negative csa_status.  Argument and shape
 *     errors are reported before anything is launched.  CSA_ERR_HIP means a
 *     launch failed.  Faults of running kernels surface at the caller's next
 *     synchronisation.  Nothing is printed.
 *   - Kernels clamp every index they read (pool index, window position) to
 *     the buffers described by the arguments; data that violates a stated
 *     precondition gives unspecified values, never an out-of-bounds access.
 *   - The library is stateless and re-entrant; results are deterministic
 *     (same inputs, same bits).  The one exception is
 *     csa_decode_index_topk_noalloc, which works in a scratch array the
 *     library holds on each device.
 */
#ifndef CSA_H
#define CSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CSA_OK = 0,
  CSA_ERR_ARG = -1,         /* null pointer, negative size, inconsistent sizes */
  CSA_ERR_UNSUPPORTED = -2, /* shape outside what the kernels implement      */
  CSA_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required     */
  CSA_ERR_HIP = -4,         /* a kernel launch failed                          */
  CSA_ERR_SCRATCH = -5      /* the call needs more than the library's scratch  */
} csa_status;

typedef enum { CSA_F32 = 0, CSA_BF16 = 1 } csa_dtype;

/* ---------------------------------------------------------------------------
 * csa_compress - token-level compressor.
 *
 * [P2] section 3.2.2 (eqs. 9-12): two token streams C^a, C^b and logits Z^a,
 * Z^b; each block of m tokens becomes one entry, a per-channel softmax over
 * the rows of both streams (plus position biases B^a, B^b) weighting the
 * rows.  Adjacent blocks overlap.  [P2] section 3.3 (eqs. 20-23): HCA uses one
 * stream, m' = 128, no overlap.  [P2] section 3.3 (quoting section 2.3.3):
 * RMSNorm on the compressed KV head and RoPE on its last 64 channels.  [P3]
 * "The indexer: a learned retrieval mechanism" and [P2] section 3.2.2: the
 * indexer keys are produced by the same operation on their own streams
 * (no norm, no RoPE).  With m = 1, no overlap, RMSNorm and RoPE, the call
 * produces the uncompressed sliding-window rows.
 *
 * Entry i of the call pools tokens pos0[b] + m*i .. + m-1 of stream a
 * (c_a/z_a rows m*i .. m*i+m-1; a partial last block pools the rows that
 * exist) and, if overlap != 0, the previous block's m rows of stream b:
 * c_b/z_b rows m*(i-1) .. for i >= 1, prev_c_b/prev_z_b for i == 0 (when
 * prev_c_b is NULL, or the block starts before token m so no block precedes
 * it, entry 0 has no b rows, as at the start of a sequence).
 * Logit of a row = z + bias[offset in block].  Then, if gain != NULL,
 * y = y / sqrt(mean(y^2) + eps) * gain; then, if rope_dims > 0, RoPE with
 * interleaved pairs on the last rope_dims channels at position pos0[b] + m*i
 * (angles pos * rope_base^(-2j/rope_dims) in float64).
 *
 *   c_a, z_a        [B, T, D]   (z_a may be NULL: all logits zero)
 *   c_b, z_b        [B, T, D]   required iff overlap != 0, else NULL
 *   prev_c_b/_z_b   [B, m, D]   optional iff overlap != 0, else NULL
 *   bias_a, bias_b  [m, D] f32  (NULL = zero)
 *   gain            [D] f32     (NULL = no RMSNorm)
 *   pos0            [B] int64   device; required if rope_dims > 0
 *   out             [B, ceil(T/m), D] with batch stride out_bstride elements
 *                   (0 = contiguous); may point into a larger pool buffer
 *   ws              optional device workspace of csa_compress_ws_bytes(...)
 *                   bytes (NULL allowed).  A call with few entries spreads
 *                   each entry over several workgroups; with a gain that
 *                   needs the workspace, without one it runs one workgroup
 *                   per entry.  A non-NULL ws smaller than the query gives
 *                   CSA_ERR_WORKSPACE.  Calls sharing a workspace must not
 *                   overlap in time.
 * Supported: 1 <= m <= 1024, D a power of two with 8 <= D <= 1024 (bf16) or
 * 4 <= D <= 1024 (f32), rope_dims even and <= D.
 * ------------------------------------------------------------------------- */
int csa_compress(int dt, int B, int T, int D, int m, int overlap,
                 const void* c_a, const void* z_a, const void* c_b, const void* z_b,
                 const void* prev_c_b, const void* prev_z_b,
                 const float* bias_a, const float* bias_b,
                 const float* gain, float eps,
                 int rope_dims, double rope_base, const int64_t* pos0,
                 void* out, int64_t out_bstride, void* ws, size_t ws_bytes, void* stream);

/* Workspace (bytes) csa_compress can use for this shape (overlap as in the
 * call); 0 when it needs none.  Returns 0 for invalid sizes. */
size_t csa_compress_ws_bytes(int dt, int B, int T, int D, int m, int overlap);

/* ---------------------------------------------------------------------------
 * Mixed BF16 / FP8 storage of the KV entries.
 *
 * [P1] "What does HCA change?" (quoting the paper's section 2.3.4): the KV
 * cache keeps the RoPE channels in BF16 and the other channels in FP8; the
 * pages give no format.  Format here (the OCP Microscaling FP8 format,
 * converted in hardware on gfx950): per entry of D = 512 channels with R
 * RoPE channels (R a multiple of 32), one packed row of
 * csa_kv_fp8_row_bytes(D, R) bytes (592 for R = 64):
 *   bytes [0, D-R)       E4M3 codes of channels 0 .. D-R-1: bit 7 the sign,
 *                        bits 3-6 the exponent field (bias 7), bits 0-2 the
 *                        mantissa; field 0 is subnormal (m * 2^-9); largest
 *                        finite magnitude 0x7E = 448
 *   bytes [D-R, D+R)     the R RoPE channels in bfloat16
 *   bytes [D+R, ...)     one E8M0 scale byte per 32 code channels, value
 *                        2^(s-127), zero-padded to a multiple of 16 bytes
 * Quantization: per 32-channel block s = floor(log2(max |x|)) - 8 + 127
 * clamped to [0, 254] (0 for an all-zero block); each element is
 * |x| / 2^(s-127) rounded to the nearest E4M3 magnitude, ties to the even
 * code, saturating at 448; sign bit set for x < 0.  The RoPE channels are
 * rounded to bfloat16 (nearest even).  Window rows stay bf16.
 * ------------------------------------------------------------------------- */

/* Bytes of one packed row; 0 for a shape the format does not cover (D must
 * be 512, R a multiple of 32 in [0, D]). */
size_t csa_kv_fp8_row_bytes(int D, int rope_dims);

/* rows x D values (dt f32 or bf16, finite) -> packed rows [rows, row_bytes]
 * uint8 (device, caller-owned).  Errors: CSA_ERR_ARG for a bad dt, rows < 0
 * or NULL pointers with rows > 0; CSA_ERR_UNSUPPORTED for another shape or
 * past rows * D = 2^39. */
int csa_quantize_kv_fp8(int dt, int64_t rows, int D, int rope_dims, const void* x, void* out,
                        void* stream);

/* Packed rows -> their exact values as bf16 [rows, D] (an E4M3 value times
 * a power of two is exact in bf16 for scale bytes 9..246), with the same
 * hardware conversion the attention uses.  Errors as csa_quantize_kv_fp8. */
int csa_dequantize_kv_fp8(int64_t rows, int D, int rope_dims, const void* rows_in, void* out,
                          void* stream);

/* csa_compress_kvfp8 - csa_compress writing each entry as a packed row
 * (pooled, normalised and rotated in float32 exactly as csa_compress does,
 * then quantized as csa_quantize_kv_fp8).  out [B, n_out rows] of
 * csa_kv_fp8_row_bytes(D, rope_dims) bytes, batch stride out_bstride bytes
 * (0: n_out rows).  Other arguments, workspace and errors as csa_compress;
 * CSA_ERR_UNSUPPORTED for a shape the row format does not cover. */
int csa_compress_kvfp8(int dt, int B, int T, int D, int m, int overlap,
                       const void* c_a, const void* z_a, const void* c_b, const void* z_b,
                       const void* prev_c_b, const void* prev_z_b,
                       const float* bias_a, const float* bias_b,
                       const float* gain, float eps,
                       int rope_dims, double rope_base, const int64_t* pos0,
                       void* out, int64_t out_bstride, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * csa_compress_batch - up to two compressors over the same token block in
 * one launch.
 *
 * The same operation as csa_compress, once per job, for jobs that share the
 * block shape and positions: [P2] section 3.2.2 runs the KV compressor and
 * the indexer-key compressor over the same tokens, so a decode step
 * compresses its closing block twice.  Each job is what csa_compress takes
 * after its shared arguments (streams of [B, T, job.D], optional biases,
 * gain, rope, out with batch stride).  One workgroup per entry and job (no
 * channel split, no workspace).
 *
 *   dt, B, T, m, overlap, pos0   shared by the jobs, as in csa_compress
 *   jobs[n_jobs], 1 <= n_jobs <= 2
 * Each job is checked as csa_compress checks its arguments; the first
 * failing job's status is returned and nothing is launched.
 * ------------------------------------------------------------------------- */
typedef struct csa_compress_job {
  int D;
  const void* c_a;
  const void* z_a;
  const void* c_b;
  const void* z_b;
  const void* prev_c_b;
  const void* prev_z_b;
  const float* bias_a;
  const float* bias_b;
  const float* gain;
  float eps;
  int rope_dims;
  double rope_base;
  void* out;
  int64_t out_bstride;
  /* 0: out holds entries of dt.  1: out holds packed mixed BF16 / FP8 rows
   * (csa_kv_fp8_row_bytes(D, rope_dims) bytes each, see csa_compress_kvfp8)
   * and out_bstride counts bytes; D = 512 only, and in the decode calls only
   * for the KV job jobs[1]. */
  int out_kv_fp8;
} csa_compress_job;

int csa_compress_batch(int dt, int B, int T, int m, int overlap, const int64_t* pos0,
                       const csa_compress_job* jobs, int n_jobs, void* stream);

/* ---------------------------------------------------------------------------
 * csa_index_topk - lightning indexer scores and top-K selection.
 *
 * [P2] section 3.2.2 (eqs. 13-17) and [P3] "The indexer: a learned retrieval
 * mechanism": I[t,s] = sum_h w[t,h] * ReLU(q[t,h] . K[s]); the K entries with
 * the highest scores are kept.  [P1] "How does CSA compress 8 tokens into 4
 * KV entries?": only causally closed entries may be chosen (mask first, then
 * rank).  [P3] (same section): when no more than K entries are visible,
 * all of them are kept.  [P4] "Tata letak attention mask": empty slots
 * carry -1.
 *
 * Query t of sequence b sits at position q_pos0[b] + t and sees entries
 * s < min(n_entries[b], (q_pos0[b] + t + 1) / m).  Scores are float32 (bf16
 * products accumulated in float32); ties go to the lower entry index.
 *
 *   q_idx      [B, Tq, Hi, Di]     dt
 *   w_idx      [B, Tq, Hi]         f32
 *   k_idx      [B, N_cap, Di]      dt (compressed indexer keys)
 *   n_entries  [B] int32 device    live entries, <= N_cap
 *   q_pos0     [B] int64 device
 *   idx_out    [B, Tq, K] int32    chosen entries in ascending order, then -1
 *   score_out  [B, Tq, K] f32      score of each chosen entry, -inf on -1
 *                                  slots (may be NULL)
 *   all_scores [B, Tq, N_cap] f32  every score of the visible entries;
 *                                  later columns unspecified (may be NULL)
 *   ws         workspace of csa_index_topk_ws_bytes(B, Tq, Hi, N_cap, K)
 * Supported: Hi <= 64, Di <= 256, Hi * Di <= 8192, 1 <= K <= 4096,
 * N_cap <= 2^26.
 * ------------------------------------------------------------------------- */
int csa_index_topk(int dt, int B, int Tq, int Hi, int Di, int N_cap, int K, int m,
                   const void* q_idx, const float* w_idx, const void* k_idx,
                   const int32_t* n_entries, const int64_t* q_pos0,
                   int32_t* idx_out, float* score_out, float* all_scores,
                   void* ws, size_t ws_bytes, void* stream);
size_t csa_index_topk_ws_bytes(int B, int Tq, int Hi, int N_cap, int K);

/* ---------------------------------------------------------------------------
 * csa_decode_index_topk - a decode step's compressors and indexer in one call.
 *
 * [P2] section 3.2.2 (eqs. 9-12, then 13-17): the block of m tokens that
 * closes at this step becomes a new compressed entry, which the indexer
 * ranks with the older ones.  For each sequence b the entry goes to row
 * r_b = min(n_entries[b], N_cap) - 1 (nothing when that is negative) of
 * each job's pool; jobs[0] is the indexer-key compressor and its pool is
 * the indexer's k_idx.  Then exactly csa_index_topk over k_idx.  The same
 * results as csa_compress_batch (one entry, written at row r_b) followed by
 * csa_index_topk; for bf16 with Hi = 64, Di = 128, Tq < 8, job D <= 512
 * and at most 8 pooled rows the compressors run inside the indexer launch
 * (one launch fewer, the fresh key scored by the workgroup that built it),
 * else as a launch of their own.
 *
 *   jobs[n_jobs]   n_jobs 1 to 3.  jobs[2], if given, is the step token's
 *                  window row (Tq = 1; the compressor with m = 1, as
 *                  csa_window_row): c_a = kv [B, 1, D], gain, rope, no b
 *                  streams; out = the window ring [B, L_win, D] with
 *                  out_bstride = L_win * D; the row goes to slot
 *                  q_pos0[b] % L_win (it runs inside the same launch).
 *                  jobs[0..1] as for csa_compress_batch with T = m:
 *                  c_a, z_a [B, m, D]; prev_c_b, prev_z_b [B, m, D] or NULL
 *                  (overlap: the previous block's second stream; c_b, z_b
 *                  must be given and are not read); bias_a, bias_b [m, D];
 *                  out = the pool base [B, N_cap, D], out_bstride 0 or
 *                  N_cap * D.  jobs[0].D == Di.
 *   block_pos0 [B] int64 device  position of the closing block's first token
 *   other arguments as csa_index_topk (ws of csa_index_topk_ws_bytes).
 * Errors: as csa_compress_batch and csa_index_topk; CSA_ERR_ARG also for
 * N_cap == 0, jobs[0].D != Di or another out_bstride.
 * ------------------------------------------------------------------------- */
int csa_decode_index_topk(int dt, int B, int Tq, int Hi, int Di, int N_cap, int K, int m,
                          int overlap, const int64_t* block_pos0, const csa_compress_job* jobs,
                          int n_jobs, const void* q_idx, const float* w_idx,
                          const int32_t* n_entries, const int64_t* q_pos0, int32_t* idx_out,
                          float* score_out, float* all_scores, void* ws, size_t ws_bytes,
                          void* stream);

/* ---------------------------------------------------------------------------
 * csa_index_scores - the lightning indexer scores alone (the scoring half
 * of csa_index_topk, same kernels, no selection).
 *
 * [P2] section 3.2.2 (eqs. 13-16): I[t,s] = sum_h w[t,h] * ReLU(q[t,h] .
 * K[s]) for every entry s visible to query t (visibility as in
 * csa_index_topk).  Arguments as csa_index_topk; scores [B, Tq, N_cap] f32
 * receives the visible columns of every row, later columns are left
 * untouched.  No workspace.  Supported shapes as csa_index_topk.
 * ------------------------------------------------------------------------- */
int csa_index_scores(int dt, int B, int Tq, int Hi, int Di, int N_cap, int m,
                     const void* q_idx, const float* w_idx, const void* k_idx,
                     const int32_t* n_entries, const int64_t* q_pos0, float* scores,
                     void* stream);

/* ---------------------------------------------------------------------------
 * MX FP4 indexer keys.
 *
 * [P1] "What does HCA change?": the cache holds the indexer's keys in FP4
 * (and the attention entries in mixed BF16/FP8); the pages give no format.
 * Format here (the OCP Microscaling FP4 format, converted in hardware on
 * gfx950): each key of Di channels (Di a multiple of 32) is Di/2 code bytes,
 * channel 2i in the low nibble of byte i, plus Di/32 scale bytes.  A code is
 * E2M1: bit 3 the sign, bits 0-2 a magnitude index into {0, 0.5, 1, 1.5, 2,
 * 3, 4, 6}.  Scale byte s of a 32-channel block multiplies its elements by
 * 2^(s - 127).
 *
 *   k_codes   [B, N_cap, Di/2]  uint8
 *   k_scales  [B, N_cap, Di/32] uint8
 * ------------------------------------------------------------------------- */

/* csa_quantize_mxfp4 - rows x D values to MX FP4.  Per 32-channel block,
 * s = floor(log2(max |x|)) - 2 + 127 clamped to [0, 254] (0 for an all-zero
 * block); each element is |x| / 2^(s-127) rounded to the nearest magnitude,
 * ties to the even index (values in [6, 8) give 6), sign bit set for x < 0.
 *   x       [rows, D] dt, finite
 *   codes   [rows, D/2] uint8; scales [rows, D/32] uint8 (device, caller-owned)
 * Errors: CSA_ERR_ARG for a bad dt, rows < 0, D <= 0 or D % 32 != 0, NULL
 * pointers with rows > 0; CSA_ERR_UNSUPPORTED past rows * D = 2^39. */
int csa_quantize_mxfp4(int dt, int64_t rows, int D, const void* x, uint8_t* codes,
                       uint8_t* scales, void* stream);

/* csa_index_topk_mxfp4 / csa_index_scores_mxfp4 - csa_index_topk and
 * csa_index_scores with the keys in MX FP4 (dt is bf16: q_idx bf16, w_idx
 * f32).  Each key value is its code's magnitude times its block's scale
 * (exact in bf16 for scale bytes 2..253), so the results are those of the
 * bf16 calls on the dequantized keys.  Same shapes, workspace and errors as
 * those calls; CSA_ERR_ARG also for Di % 32 != 0 or a NULL k_scales. */
int csa_index_topk_mxfp4(int B, int Tq, int Hi, int Di, int N_cap, int K, int m,
                         const void* q_idx, const float* w_idx, const uint8_t* k_codes,
                         const uint8_t* k_scales, const int32_t* n_entries,
                         const int64_t* q_pos0, int32_t* idx_out, float* score_out,
                         float* all_scores, void* ws, size_t ws_bytes, void* stream);
int csa_index_scores_mxfp4(int B, int Tq, int Hi, int Di, int N_cap, int m,
                           const void* q_idx, const float* w_idx, const uint8_t* k_codes,
                           const uint8_t* k_scales, const int32_t* n_entries,
                           const int64_t* q_pos0, float* scores, void* stream);

/* csa_decode_index_topk_mxfp4 - csa_decode_index_topk with the indexer keys
 * in MX FP4: the key job's fresh entry (pooled in float32 as the compressor
 * does) is quantized as csa_quantize_mxfp4 and written to row r_b of k_codes
 * and k_scales; the indexer then reads the FP4 keys (the fresh one scored
 * from its quantized value).  jobs[0].out must be NULL and its out_bstride
 * 0; jobs[1] (the KV compressor, if given) writes bf16 as before.  Only the
 * fused launch writes FP4: bf16 streams, Hi = 64, Di = 128, Tq < 8, job
 * D <= 512 and at most 8 pooled rows, else CSA_ERR_UNSUPPORTED before any
 * launch.  Other arguments and errors as csa_decode_index_topk (dt bf16). */
int csa_decode_index_topk_mxfp4(int B, int Tq, int Hi, int Di, int N_cap, int K, int m,
                                int overlap, const int64_t* block_pos0,
                                const csa_compress_job* jobs, int n_jobs, const void* q_idx,
                                const float* w_idx, uint8_t* k_codes, uint8_t* k_scales,
                                const int32_t* n_entries, const int64_t* q_pos0,
                                int32_t* idx_out, float* score_out, float* all_scores,
                                void* ws, size_t ws_bytes, void* stream);

/* csa_decode_index_topk_noalloc - csa_decode_index_topk for callers that
 * cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  The workspace is not an
 * argument: the call works in a scratch array of CSA_NOALLOC_SCRATCH_BYTES
 * that the library holds on each device (a static device array, present
 * while the library is loaded; its address is looked up once per device,
 * on the first call there, with that device current).  The call allocates
 * and frees nothing.  Calls that overlap in time on one device share that
 * device's array and race: order them on one stream.  The array keeps the
 * last call's contents; nothing in it needs to start at zero (the scores
 * the selection reads are written by the same call).  Arguments, results
 * and errors as csa_decode_index_topk without ws / ws_bytes; CSA_ERR_SCRATCH
 * when csa_index_topk_ws_bytes(B, Tq, Hi, N_cap, K) exceeds the scratch
 * (decode of 8 sequences at 1,048,576 tokens needs 8.9 MB). */
#define CSA_NOALLOC_SCRATCH_BYTES (32u << 20)
int csa_decode_index_topk_noalloc(int dt, int B, int Tq, int Hi, int Di, int N_cap, int K, int m,
                                  int overlap, const int64_t* block_pos0,
                                  const csa_compress_job* jobs, int n_jobs, const void* q_idx,
                                  const float* w_idx, const int32_t* n_entries,
                                  const int64_t* q_pos0, int32_t* idx_out, float* score_out,
                                  float* all_scores, void* stream);

/* csa_decode_index_scores(_mxfp4) - the scoring half of
 * csa_decode_index_topk(_mxfp4): the closing block's fresh entries are
 * written exactly as there (the same launch: for the shapes listed there the
 * compressors run inside the indexer launch), then every visible entry is
 * scored into scores [B, Tq, N_cap] f32 (later columns unspecified); no
 * selection, no workspace.  [P2] section 3.2.2 (eqs. 9-16).  A caller that
 * selects elsewhere uses it: a pool split over several devices scores each
 * slice and merges the per-slice winners; it also times the fused launch on
 * its own.  Arguments and errors as csa_decode_index_topk(_mxfp4) without
 * K, idx_out, score_out and the workspace; CSA_ERR_ARG for a NULL scores. */
int csa_decode_index_scores(int dt, int B, int Tq, int Hi, int Di, int N_cap, int m, int overlap,
                            const int64_t* block_pos0, const csa_compress_job* jobs, int n_jobs,
                            const void* q_idx, const float* w_idx, const int32_t* n_entries,
                            const int64_t* q_pos0, float* scores, void* stream);
int csa_decode_index_scores_mxfp4(int B, int Tq, int Hi, int Di, int N_cap, int m, int overlap,
                                  const int64_t* block_pos0, const csa_compress_job* jobs,
                                  int n_jobs, const void* q_idx, const float* w_idx,
                                  uint8_t* k_codes, uint8_t* k_scales,
                                  const int32_t* n_entries, const int64_t* q_pos0,
                                  float* scores, void* stream);

/* ---------------------------------------------------------------------------
 * Streaming decode state.
 *
 * [P4] "Lapisan cache" (the per-layer caches, DeepseekV4CSACache and
 * DeepseekV4HCACache, keep the raw sliding window and, for the compressor
 * and the indexer, the pending tokens, the pool, the entry count and the
 * overlap state) and [P1]
 * "How does CSA compress 8 tokens into 4 KV entries?" (an entry exists once
 * its block of m tokens has closed).  A decode loop keeps every count on
 * the device, so steps can be captured in a HIP graph and replayed with no
 * host round trip:
 *
 *   - the window is a ring: row p % L_win of win holds token p; pass
 *     win_pos0 = NULL to csa_sparse_attn / hca_attn for it (L_win >= W);
 *   - csa_window_row writes the new token's window row into the ring;
 *   - csa_decode_advance moves q_pos, n_entries and block_pos0 to the next
 *     token; a block_pos0[b] of -1 tells csa_compress_batch,
 *     csa_decode_index_topk(_mxfp4) that no block closes for sequence b at
 *     this step (its caches are left untouched and the indexer ranks the
 *     entries already stored).
 * ------------------------------------------------------------------------- */

/* csa_window_row - the window row of each sequence's new token, written into
 * the ring: win[b, pos[b] % L_win] = RoPE(RMSNorm(kv[b]) * gain, pos[b])
 * (the compressor with m = 1).
 *   kv   [B, 1, D] dt;  gain [D] f32 or NULL (no RMSNorm);  pos [B] int64 device
 *   win  [B, L_win, D] dt (ring)
 * Errors as csa_compress; CSA_ERR_ARG also for L_win <= 0 or a NULL pos. */
int csa_window_row(int dt, int B, int D, const void* kv, const float* gain, float eps,
                   int rope_dims, double rope_base, const int64_t* pos, void* win, int L_win,
                   void* stream);

/* csa_decode_advance - one token forward for every sequence (device only):
 * q_pos[b] += 1; with t the new q_pos[b], n_entries[b] = min((t + 1) / m,
 * N_cap) and block_pos0[b] = t + 1 - m when the block closes at t
 * ((t + 1) % m == 0), else -1.  Start a sequence at q_pos = -1.  N_cap
 * must cover the whole context: once n_entries reaches it, a closing step
 * writes its entry over row N_cap - 1.
 *   q_pos, block_pos0 [B] int64;  n_entries [B] int32 (device, in place)
 * CSA_ERR_ARG for B < 0, m <= 0, N_cap < 0 or NULL pointers. */
int csa_decode_advance(int B, int m, int N_cap, int64_t* q_pos, int32_t* n_entries,
                       int64_t* block_pos0, void* stream);

/* ---------------------------------------------------------------------------
 * csa_output_proj - grouped low-rank output projection of T tokens.
 *
 * [P2] section 3.3 (after eq. 26): the concatenated head outputs are split
 * into G groups, each group projected to an intermediate of r channels, and
 * the G intermediates, concatenated, projected to the final attention output.
 * [P1] "What does layer 0 sliding-window attention do to p?" (grouped W_O,
 * Flash: 64 heads in 8 groups); [P4] "Arsitektur" (groups -> a low rank per
 * group -> hidden size).  Group j holds heads j*H/G .. (j+1)*H/G - 1.
 *
 *   mid[t, j*r + n] = sum_k o[t, j*H/G*D + k] * w_a[j, n, k]   (rounded to bf16)
 *   out[t, e]       = sum_c mid[t, c] * w_b[e, c]
 *
 *   o    [T, H, D] bf16 (attention outputs)
 *   w_a  [G, r, (H/G)*D] bf16
 *   w_b  [d_model, G*r] bf16
 *   mid  [T, G*r] bf16   caller-owned intermediates (written)
 *   out  [T, d_model] bf16
 * float32 accumulation; two launches.  Supported: T <= 16 (decode batches,
 * the weights streamed once) with (H/G)*D a multiple of 512, G*r a multiple
 * of 1024, r and d_model multiples of 16; or 16 < T <= 2^22 (a tiled GEMM)
 * with (H/G)*D and G*r multiples of 64, r and d_model multiples of 128; else
 * CSA_ERR_UNSUPPORTED.  CSA_ERR_ARG for nonpositive sizes, H % G != 0 or NULL
 * pointers (T = 0 does nothing).
 * ------------------------------------------------------------------------- */
int csa_output_proj(int T, int H, int D, int G, int r, int d_model, const void* o,
                    const void* w_a, const void* w_b, void* mid, void* out, void* stream);

/* ---------------------------------------------------------------------------
 * csa_sparse_attn - shared-K=V multi-query attention with a per-head sink
 * over the selected pool rows and the sliding-window rows.
 *
 * [P2] section 3.2.2 (eq. 19) and [P4] "Arsitektur": the selected entries are
 * both key and value of a multi-query attention with one KV head; the
 * window's uncompressed rows are concatenated with them.  [P1] "What does
 * layer 0 sliding-window attention do to p?" (eq. 27): a per-head sink
 * logit sits in the softmax denominator only.  [P1] "How does CSA compress 8
 * tokens into 4 KV entries?" and [P4] "Arsitektur": the query's rope slice
 * is rotated at its position t and the output's rope slice by -t.
 *
 * For query t (position q_pos0[b] + t) and head h:
 *   rows  = pool[b, idx[b,t,j]] for every idx >= 0 (no de-duplication),
 *           then win[b, p - win_pos0[b]] for p in [max(0, t-W+1), t] that
 *           lie inside the window buffer;
 *   q'    = RoPE(q[b,t,h], t);  z_j = scale * q' . row_j;
 *   lse   = log(sum_j exp z_j + exp sink[h]);
 *   out   = RoPE(sum_j exp(z_j - lse) row_j, -t).
 * With no rows, out = 0 and lse = sink[h].
 *
 *   q       [B, Tq, H, D] dt (RMS-normalised, not rotated)
 *   pool    [B, N_cap, D] dt;  idx [B, Tq, K] int32 (-1 = empty slot)
 *   win     [B, L_win, D] dt;  win_pos0 [B] int64 device, or NULL for a
 *           ring (row p % L_win holds token p; requires L_win >= W)
 *   sink    [H] f32; q_pos0 [B] int64 device
 *   out     [B, Tq, H, D] dt;  lse [B, Tq, H] f32 natural log (may be NULL)
 *   ws      workspace of csa_attn_ws_bytes(B, Tq, H, D, K + W)
 * Supported: D <= 1024, H <= 128, rope_dims even and <= D; in bf16 with
 * H = 64 or 128 (Flash, Pro) and D = 512 (the MFMA path), K + W <= 524288
 * (else CSA_ERR_UNSUPPORTED).
 * ------------------------------------------------------------------------- */
int csa_sparse_attn(int dt, int B, int Tq, int H, int D, int rope_dims, double rope_base,
                    float scale, const void* q, const void* pool, int N_cap,
                    const int32_t* idx, int K, const void* win, int L_win,
                    const int64_t* win_pos0, int W, const float* sink,
                    const int64_t* q_pos0, void* out, float* lse,
                    void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * hca_attn - the same attention with every visible compressed entry as a
 * key (no indexer).
 *
 * [P2] section 3.3 (eqs. 24-26) and [P1] "What does HCA change?": no top-k,
 * dense attention over the heavily compressed entries plus the window.
 * [P4] "Tata letak attention mask": entry w is visible to t iff
 * w < (t + 1) / m.
 *
 * rows = pool[b, w] for w < min(n_entries[b], (q_pos0[b] + t + 1) / m), then
 * the window rows as in csa_sparse_attn.  Other arguments as there.
 *   ws      workspace of csa_attn_ws_bytes(B, Tq, H, D, N_cap + W)
 * ------------------------------------------------------------------------- */
int hca_attn(int dt, int B, int Tq, int H, int D, int rope_dims, double rope_base,
             float scale, const void* q, const void* pool, int N_cap,
             const int32_t* n_entries, int m, const void* win, int L_win,
             const int64_t* win_pos0, int W, const float* sink,
             const int64_t* q_pos0, void* out, float* lse,
             void* ws, size_t ws_bytes, void* stream);

/* csa_sparse_attn_kvfp8 / hca_attn_kvfp8 - csa_sparse_attn and hca_attn
 * over a pool of packed mixed BF16 / FP8 rows (see csa_kv_fp8_row_bytes):
 * pool [B, N_cap, row_bytes] uint8.  q, the window and out are bf16 (no dt
 * argument); each pool row's values are its exact dequantization, so the
 * result is that of the bf16 call on the dequantized pool.  Other arguments,
 * workspace and errors as those calls; CSA_ERR_UNSUPPORTED outside the
 * bf16 MFMA shape (H a multiple of 64 up to 128, D = 512, R a multiple of
 * 32). */
int csa_sparse_attn_kvfp8(int B, int Tq, int H, int D, int rope_dims, double rope_base,
                          float scale, const void* q, const void* pool, int N_cap,
                          const int32_t* idx, int K, const void* win, int L_win,
                          const int64_t* win_pos0, int W, const float* sink,
                          const int64_t* q_pos0, void* out, float* lse,
                          void* ws, size_t ws_bytes, void* stream);
int hca_attn_kvfp8(int B, int Tq, int H, int D, int rope_dims, double rope_base,
                   float scale, const void* q, const void* pool, int N_cap,
                   const int32_t* n_entries, int m, const void* win, int L_win,
                   const int64_t* win_pos0, int W, const float* sink,
                   const int64_t* q_pos0, void* out, float* lse,
                   void* ws, size_t ws_bytes, void* stream);

/* Workspace (bytes) for csa_sparse_attn / hca_attn with at most
 * keys_per_query rows per query (K + W, or N_cap + W). */
size_t csa_attn_ws_bytes(int B, int Tq, int H, int D, int keys_per_query);

/* ---------------------------------------------------------------------------
 * hca_decode_attn - one HCA decode step in one call: the closing block's
 * entry is pooled, stored and attended together with the entries already in
 * the pool.  The result is that of csa_compress (HCA: m-row blocks, no
 * overlap, one block per sequence, entry to row min(n_entries[b], N_cap) - 1
 * of pool) followed by hca_attn with Tq = 1, up to rounding order.
 *
 * [P2] section 3.3 (eqs. 20-23): the new entry is the softmax-weighted pool
 * of the block's m rows per channel (logits z + bias), then RMSNorm with
 * gain and RoPE at the block's first position block_pos0[b]; [P2] section
 * 3.3 (eqs. 24-26) and [P4] "Tata letak attention mask": the query at t
 * attends to every entry w < min(n_entries[b], (t + 1) / m), the new one
 * included, and to its window.
 *
 *   c, z        [B, m, D] bf16: the block's rows and logits (z may be NULL:
 *               logits from the bias alone)
 *   bias        [m, D] f32 or NULL (zero);  gain [D] f32 or NULL (no RMSNorm)
 *   block_pos0  [B] int64 device: the closing block's first position, or -1
 *               when no block closes for sequence b (nothing is pooled or
 *               stored, and the call is hca_attn)
 *   pool        [B, N_cap, D] bf16, written at the new entry's row only;
 *               n_entries[b] counts the entries including the new one
 *   q [B, 1, H, D], q_pos0 [B] (the query's position), out [B, 1, H, D]:
 *   bf16; rope_dims applies to the query, the output and the new entry.
 *   Other arguments as hca_attn (dt = bf16, Tq = 1).
 *   ws          workspace of hca_decode_attn_ws_bytes(B, H, D, N_cap + W)
 * The last key-range split of each query computes the entry (its workgroup
 * pools the rows while the other splits stream the pool) and the others
 * leave its row out, so no launch waits for the compressor.
 * CSA_ERR_UNSUPPORTED outside the bf16 MFMA shape (H a multiple of 64 up to
 * 128, D = 512, even rope_dims) or for m > 1024; CSA_ERR_ARG for m <= 0 or
 * NULL c, n_entries, block_pos0; otherwise errors as hca_attn.
 * ------------------------------------------------------------------------- */
int hca_decode_attn(int B, int H, int D, int rope_dims, double rope_base, float scale,
                    const void* q, void* pool, int N_cap, const int32_t* n_entries, int m,
                    const void* c, const void* z, const float* bias, const float* gain,
                    float eps, const int64_t* block_pos0, const void* win, int L_win,
                    const int64_t* win_pos0, int W, const float* sink, const int64_t* q_pos0,
                    void* out, float* lse, void* ws, size_t ws_bytes, void* stream);

/* hca_decode_attn_kvfp8 - hca_decode_attn over a pool of packed mixed
 * BF16 / FP8 rows (see csa_kv_fp8_row_bytes): pool [B, N_cap, row_bytes]
 * uint8.  The new entry is stored as a packed row (as csa_compress_kvfp8
 * stores it) and attended as the values read back from that row, so the
 * result is that of csa_compress_kvfp8 followed by hca_attn_kvfp8 with
 * Tq = 1, up to rounding order.  Other arguments, workspace and errors as
 * hca_decode_attn; CSA_ERR_UNSUPPORTED also for rope_dims not a multiple of
 * 32. */
int hca_decode_attn_kvfp8(int B, int H, int D, int rope_dims, double rope_base, float scale,
                          const void* q, void* pool, int N_cap, const int32_t* n_entries, int m,
                          const void* c, const void* z, const float* bias, const float* gain,
                          float eps, const int64_t* block_pos0, const void* win, int L_win,
                          const int64_t* win_pos0, int W, const float* sink,
                          const int64_t* q_pos0, void* out, float* lse, void* ws,
                          size_t ws_bytes, void* stream);

/* Workspace (bytes) for hca_decode_attn(_kvfp8) with at most keys_per_query
 * rows per query (N_cap + W); 0 for shapes it does not take. */
size_t hca_decode_attn_ws_bytes(int B, int H, int D, int keys_per_query);

/* ---------------------------------------------------------------------------
 * swa_decode_attn - one decode step of a sliding-window-only layer in one
 * call: the query token's window row is built and stored, and the query
 * attends to its window.  The result is that of csa_window_row (or
 * csa_compress with m = 1 into the window buffer) followed by
 * csa_sparse_attn with K = 0 and no pool, up to rounding order.
 *
 * [P3] "The per-layer pattern" and [P1] "What does layer 0 sliding-window
 * attention do to p?": the first layers attend to the raw window only, the
 * query's own token included, with the sink in the softmax (eq. 27 of
 * [P1]); [P2] section 3.2.2: the window holds the most recent uncompressed
 * tokens.  The window row of token t is built as csa_compress builds one
 * with m = 1: RMSNorm(kv) * gain, RoPE at t.
 *
 *   q [B, 1, H, D], out [B, 1, H, D], kv [B, 1, D]: bf16
 *   gain [D] f32 or NULL (no RMSNorm); q_pos0 [B] int64 device: the token's
 *   position t (the row's RoPE position too)
 *   win [B, L_win, D] bf16: a ring (win_pos0 NULL, L_win >= W; row
 *   t % L_win is written) or a linear buffer with win[b, r] the token at
 *   win_pos0[b] + r (row t - win_pos0[b] is written when it lies in the
 *   buffer; otherwise nothing is written and the window holds what the
 *   buffer holds).  Other arguments as csa_sparse_attn.
 *   ws          workspace of swa_decode_attn_ws_bytes(B, H, D, W)
 * The last key-range split of each query builds and stores the row and
 * attends to it alone; the others leave it out.
 * CSA_ERR_UNSUPPORTED outside the bf16 MFMA shape (H a multiple of 64 up to
 * 128, D = 512); CSA_ERR_ARG for NULL kv or win, L_win <= 0, W <= 0, a ring
 * shorter than W, odd or out-of-range rope_dims, a negative eps with a
 * gain; CSA_ERR_WORKSPACE as csa_sparse_attn.
 * ------------------------------------------------------------------------- */
int swa_decode_attn(int B, int H, int D, int rope_dims, double rope_base, float scale,
                    const void* q, const void* kv, const float* gain, float eps, void* win,
                    int L_win, const int64_t* win_pos0, int W, const float* sink,
                    const int64_t* q_pos0, void* out, float* lse, void* ws, size_t ws_bytes,
                    void* stream);

/* Workspace (bytes) for swa_decode_attn over a window of W rows; 0 for
 * shapes it does not take. */
size_t swa_decode_attn_ws_bytes(int B, int H, int D, int W);

/* Human-readable name of a csa_status value (static string). */
const char* csa_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* CSA_H */
