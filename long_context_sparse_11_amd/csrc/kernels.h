// Internal interface between the C ABI layer (abi.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.h"

namespace csa {

// ---------------------------------------------------------------- compressor
struct CompressArgs {
  int dt;  // 0 f32, 1 bf16
  int B, T, D, m, overlap, n_out;
  const void *c_a, *z_a, *c_b, *z_b, *prev_c_b, *prev_z_b;
  const float *bias_a, *bias_b, *gain;
  float eps;
  int rope_dims;
  double rope_theta1;   // rope_base^(-2/rope_dims), computed on the host
  const int64_t* pos0;
  void* out;
  int64_t out_bstride;
  int slices;           // channel slices per entry (set by the launcher)
  float* ws_y;          // [B, n_out, D] f32 pooled values when slices > 1 with a gain
  size_t ws_bytes;
  // when set (one entry per sequence): sequence b's entry goes to row
  // min(rows_at[b], rows_cap) - 1 of out (none when that is negative)
  const int32_t* rows_at;
  int rows_cap;
  // when set, entries are stored as MX FP4 (fused decode path only): out
  // holds the codes [B, rows, D/2] bytes and out_scales the scale bytes
  // [B, rows, D/32]; out_bstride still counts channels (rows * D)
  uint8_t* out_scales;
  // when > 0: entry i of sequence b goes to row (pos0[b] / m + i) % ring_len
  // of out (a ring of window rows, m = 1)
  int ring_len;
  // when > 0: entries are stored as packed mixed BF16 / FP8 rows of this
  // many bytes (D = 512, rope_dims a multiple of 32); out_bstride then counts
  // bytes
  int out_fp8_row;
};
// Row of out that entry i of sequence b goes to, or -1 for none: with
// rows_at, min(rows_at[b], rows_cap) - 1; a negative pos0[b] means no block
// closes for b at this step (decode); with ring_len, the ring slot.
__device__ __forceinline__ int64_t compress_out_row(const CompressArgs& a, int b, int i) {
  if (a.pos0 && a.pos0[b] < 0) return -1;
  if (a.rows_at) return (int64_t)min(a.rows_at[b], a.rows_cap) - 1;
  if (a.ring_len > 0) {
    const int64_t p = (a.pos0 ? a.pos0[b] / a.m : 0) + i;
    return p % a.ring_len;
  }
  return i;
}
// Stores one KV entry (D = 512) as a packed mixed BF16 / FP8 row from the 64
// lanes of a wave, lane l holding channels 8l .. 8l+7: the lanes of the
// D - R non-RoPE channels write 8 E4M3 codes each (the 4 lanes of a
// 32-channel block meet by lane swaps for its scale, the first writes the
// scale byte), the others their bf16 channels; lane 0 zeroes the padding.
__device__ __forceinline__ void store_kv_fp8_row(uint8_t* row, int lane, const float (&y)[8],
                                                 int R) {
  constexpr int D = 512;
  const int nc = (D - R) >> 3;
  const bool fp8 = lane < nc;
  float am = 0.f;
  if (fp8) {
#pragma unroll
    for (int e = 0; e < 8; ++e) am = fmaxf(am, fabsf(y[e]));
  }
  am = fmaxf(am, __shfl_xor(am, 1));
  am = fmaxf(am, __shfl_xor(am, 2));
  const uint32_t s = mx8_scale_byte(am);
  if (fp8) {
    uint2 w;
    w.x = e4m3_code(y[0], s) | (e4m3_code(y[1], s) << 8) | (e4m3_code(y[2], s) << 16) |
          (e4m3_code(y[3], s) << 24);
    w.y = e4m3_code(y[4], s) | (e4m3_code(y[5], s) << 8) | (e4m3_code(y[6], s) << 16) |
          (e4m3_code(y[7], s) << 24);
    *reinterpret_cast<uint2*>(row + 8 * lane) = w;
    if ((lane & 3) == 0) row[D + R + (lane >> 2)] = (uint8_t)s;
  } else {
    uint4 pk;
    pk.x = pack_bf16x2(y[0], y[1]);
    pk.y = pack_bf16x2(y[2], y[3]);
    pk.z = pack_bf16x2(y[4], y[5]);
    pk.w = pack_bf16x2(y[6], y[7]);
    *reinterpret_cast<uint4*>(row + (D - R) + 16 * (lane - nc)) = pk;
  }
  if (lane == 0) {
    for (int p = D + R + (D - R) / 32; p < D + R + kv_fp8_scale_pad(D, R); ++p) row[p] = 0;
  }
}
// The values a reader of that packed row gets back for the lane's 8
// channels, as bf16 pairs: the E4M3 codes times their block's scale (exact
// in bf16, converted as the attention converts a staged row), or the bf16
// RoPE channels.  All 64 lanes take part (the block scale's lane swaps).
__device__ __forceinline__ u32x4_t kv_fp8_row_values(int lane, const float (&y)[8], int R) {
  constexpr int D = 512;
  const bool fp8 = lane < ((D - R) >> 3);
  float am = 0.f;
  if (fp8) {
#pragma unroll
    for (int e = 0; e < 8; ++e) am = fmaxf(am, fabsf(y[e]));
  }
  am = fmaxf(am, __shfl_xor(am, 1));
  am = fmaxf(am, __shfl_xor(am, 2));
  const uint32_t s = mx8_scale_byte(am);
  u32x4_t v;
  if (fp8) {
    const uint32_t lo = e4m3_code(y[0], s) | (e4m3_code(y[1], s) << 8) |
                        (e4m3_code(y[2], s) << 16) | (e4m3_code(y[3], s) << 24);
    const uint32_t hi = e4m3_code(y[4], s) | (e4m3_code(y[5], s) << 8) |
                        (e4m3_code(y[6], s) << 16) | (e4m3_code(y[7], s) << 24);
    const float sc = mx_scale_value(s);
    v[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, sc, false));
    v[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, sc, true));
    v[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, sc, false));
    v[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, sc, true));
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = pack_bf16x2(y[2 * k], y[2 * k + 1]);
  }
  return v;
}
// Workspace the compressor uses for a call of this shape (0 = none); rows:
// rows pooled per entry (m, or 2m with overlap).
size_t compress_ws_bytes(int dt, int B, int n_out, int D, int rows);
hipError_t launch_compress(CompressArgs a, hipStream_t stream);
// n (1 or 2) compressors over the same token block (same dt, B, T, m,
// overlap, pos0) in one launch, one workgroup per entry and job.
hipError_t launch_compress_batch(const CompressArgs* jobs, int n, hipStream_t stream);

// ------------------------------------------------------------------- indexer
struct IndexArgs {
  int dt;
  int B, Tq, Hi, Di, N_cap, m;
  const void* q;        // [B, Tq, Hi, Di]
  const float* w;       // [B, Tq, Hi]
  const void* k;        // [B, N_cap, Di]
  const int32_t* n_entries;
  const int64_t* q_pos0;
  float* scores;        // [B*Tq, N_cap]
  // MX FP4 keys when set: k holds the codes [B, N_cap, Di/2] bytes and ks the
  // scale bytes [B, N_cap, Di/32]; q is bf16
  const uint8_t* ks;
};
// True when the MFMA kernels cover this shape (bf16, 64 heads x 128).
bool index_uses_mfma(const IndexArgs& a);
hipError_t launch_index_scores(const IndexArgs& a, hipStream_t stream);
// Decode step with fresh entries: the compressor jobs (bf16, one closing
// block per sequence, T = m) run in extra workgroups of the indexer launch
// and write row min(n_entries[b], N_cap) - 1 of their pools; job 0 is the
// indexer-key compressor, whose fresh entry those workgroups also score.
// Job 2, when present, is the step token's window row (m = 1, written to its
// ring slot, ring_len > 0).
struct FreshJobs {
  CompressArgs job[3];
  int n_jobs;
};
// True when launch_index_fresh covers this shape (otherwise the compressors
// and the indexer run as separate launches).
bool index_fresh_fused(const IndexArgs& a, const FreshJobs& f);
hipError_t launch_index_fresh(const IndexArgs& a, const FreshJobs& f, hipStream_t stream);

// ---------------------------------------------------------------- MX FP4 keys
// Decode-state advance: q_pos[b] += 1, then n_entries[b] = min((q_pos + 1)
// / m, N_cap) and block_pos0[b] = the closing block's first token, or -1.
hipError_t launch_decode_advance(int B, int m, int N_cap, int64_t* q_pos, int32_t* n_entries,
                                 int64_t* block_pos0, hipStream_t stream);

// rows x D values (f32 or bf16, D a multiple of 32) to MX FP4 codes
// [rows, D/2] and scale bytes [rows, D/32].
hipError_t launch_mxfp4_quantize(int dt, int64_t rows, int D, const void* x, uint8_t* codes,
                                 uint8_t* scales, hipStream_t stream);

// ------------------------------------------------- mixed BF16 / FP8 KV rows
int kv_fp8_row_bytes_host(int D, int R);
hipError_t launch_kv_fp8_quantize(int dt, int64_t rows, int D, int R, const void* x, void* out,
                                  hipStream_t stream);
hipError_t launch_kv_fp8_dequantize(int64_t rows, int D, int R, const void* in, void* out,
                                    hipStream_t stream);

// --------------------------------------------------------------------- top-k
// Largest score row that one workgroup selects from in LDS.
constexpr int kTopkCap = 16384;

struct TopkArgs {
  int mode;             // 0: direct rows, 1: chunk of a row, 2: merge of candidates
  int B, Tq, N_cap, m, K;
  int nchunks;          // chunks per query (mode 1); chunks merged (mode 2)
  int chunk;            // elements per chunk (mode 1)
  const float* scores;  // mode 0/1: [B*Tq, N_cap]; mode 2: candidates [B*Tq, nchunks*K]
  const int32_t* in_idx;  // mode 2: candidate indices [B*Tq, nchunks*K]
  const int32_t* n_entries;
  const int64_t* q_pos0;
  int32_t* out_idx;     // [segments, K]
  float* out_scores;    // [segments, K] or null
};
hipError_t launch_topk(const TopkArgs& a, int segments, hipStream_t stream);

// ----------------------------------------------------------------- attention
struct AttnArgs {
  int dt;
  int B, Tq, H, D, R;
  double rope_theta1;   // rope_base^(-2/R), computed on the host
  float scale;
  const void* q;        // [B, Tq, H, D]
  const void* pool;     // [B, N_cap, D]
  int N_cap;
  int csa;              // 1: rows = idx-selected pool rows; 0: visible prefix (HCA)
  const int32_t* idx;   // CSA: [B, Tq, K] (may be null when K == 0)
  int K;
  const int32_t* n_entries;  // HCA
  int m;                     // HCA
  const void* win;      // [B, L_win, D]
  int L_win;
  // row r of win holds token win_pos0[b] + r; null: a ring, row p % L_win
  // holds token p (L_win >= W)
  const int64_t* win_pos0;
  int W;
  const float* sink;    // [H]
  const int64_t* q_pos0;
  void* out;            // [B, Tq, H, D]
  float* lse;           // [B, Tq, H] or null
  // 0: pool rows are D elements of dt; > 0: packed mixed BF16 / FP8 rows of
  // this many bytes (kv_fp8_row_bytes; bf16 MFMA shape only)
  int pool_row_bytes;
  int splits;           // key-range splits per query (1 = no combine pass)
  float* part_ml;       // [B*Tq, splits, H, 2] when splits > 1: (max, sum)
  bf16_t* part_o;       // [B*Tq, splits, H, D] unnormalised split outputs
  // Decode steps with a new row (Tq = 1, the MFMA shape; the kernels without
  // selected indices): the last split of each query computes the row from
  // job fj and counts as a split of that one row, the other splits leave it
  // out.  fresh 1 (hca_decode_attn(_kvfp8)): the closing block's entry
  // (T = m, one entry per sequence), to pool row min(n_entries[b], N_cap) - 1
  // when fj.pos0[b] >= 0.  fresh 2 (swa_decode_attn): the query token's own
  // window row (m = 1, at fj.pos0[b] = q_pos0[b]), to its window buffer row.
  int fresh;
  CompressArgs fj;
};
bool attn_uses_mfma(int dt, int H, int D, int R);
int attn_splits(int dt, int B, int Tq, int H, int D, int keys_per_query);
// most selected + window rows per query the MFMA path takes (CSA)
int64_t attn_max_csa_keys();
size_t attn_ws_bytes(int dt, int B, int Tq, int H, int D, int keys_per_query);
int attn_fresh_splits(int B, int H, int D, int keys_per_query);
size_t attn_fresh_ws_bytes(int B, int H, int D, int keys_per_query);
hipError_t launch_attn(const AttnArgs& a, hipStream_t stream);

}  // namespace csa
