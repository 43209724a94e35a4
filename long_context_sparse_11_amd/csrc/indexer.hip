// Lightning-indexer scores I[t,s] = sum_h w[t,h] * ReLU(q[t,h] . K[s]) for
// every compressed key s visible to query t ("DeepSeek-v4 Beyond Basics"
// section 3.2.2, eq. 16; "07 The Model", "The indexer: a learned retrieval
// mechanism").  Scores are float32; bf16 products accumulate in float32.
//
// Three kernels:
//  * index_generic   any shape/dtype, one thread per (query, key), VALU.
//  * index_decode    bf16, 64 heads x 128, few queries: every wave streams its
//                    own 32-key tiles straight from HBM into MFMA operands;
//                    the query's 64x128 head matrix stays in registers.
//  * index_prefill   bf16, 64 heads x 128, many queries: 8 waves = 8 queries
//                    share 64-key tiles staged in LDS (double buffered).
//
// MX FP4 keys (IndexArgs::ks set): every kernel has a variant that reads the
// codes and scale bytes and turns them into the same bf16 operands (exact:
// an E2M1 value times a power of two has at most two significant bits).
//
// MFMA layout (v_mfma_f32_32x32x16_bf16, C[32x32] += A[32x16] B[16x32]):
// lane l feeds A row (l % 32) and B column (l % 32) with 8 consecutive K
// slots starting at 8 * (l / 32); accumulator element r of lane l is
// C[8*(r/4) + 4*(l/32) + r%4][l % 32].  Here A = query heads (M = 32 heads),
// B = keys (N = 32 keys) and the 128-long contraction runs in 8 steps; at
// step s the K slots of lane half g map to key channels 64*g + 8*s .. +7,
// the same map on both operands, so each lane reads 128 contiguous bytes of
// its key row.  After the 16 MFMAs of a tile a lane holds 32 of the 64 head
// dots of one key: ReLU, weight, sum, and one cross-half shuffle finish it.
#include "kernels.h"

namespace csa {

// ------------------------------------------------------------------ generic
template <typename T, bool FP4>
__global__ __launch_bounds__(256) void index_generic(IndexArgs a) {
  extern __shared__ float sq[];  // [Hi*Di] query, then [Hi] weights
  const int query = blockIdx.y;
  const int b = query / a.Tq;
  const int t = query - b * a.Tq;
  const int n_vis = visible_entries(a.q_pos0[b] + t, a.m, min(a.n_entries[b], a.N_cap));
  const int HD = a.Hi * a.Di;
  const T* qp = (const T*)a.q + (int64_t)query * HD;
  for (int e = threadIdx.x; e < HD; e += blockDim.x) sq[e] = Elem<T>::get(qp + e);
  for (int e = threadIdx.x; e < a.Hi; e += blockDim.x) sq[HD + e] = a.w[(int64_t)query * a.Hi + e];
  __syncthreads();
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= n_vis) return;
  const int64_t krow = (int64_t)b * a.N_cap + s;
  const T* kp = (const T*)a.k + krow * a.Di;
  auto key = [&](int c) -> float {
    if constexpr (FP4) {
      const uint32_t byte = ((const uint8_t*)a.k)[krow * (a.Di / 2) + (c >> 1)];
      return e2m1_value((c & 1) ? byte >> 4 : byte & 15u, a.ks[krow * (a.Di / 32) + (c >> 5)]);
    } else {
      return Elem<T>::get(kp + c);
    }
  };
  float score = 0.f;
  for (int h = 0; h < a.Hi; ++h) {
    float dot = 0.f;
    for (int c = 0; c < a.Di; ++c) dot += sq[h * a.Di + c] * key(c);
    score += sq[HD + h] * fmaxf(dot, 0.f);
  }
  a.scores[(int64_t)query * a.N_cap + s] = score;
}

// --------------------------------------------------------------- MFMA common
// Query operand: lane (g, j) holds heads j and 32+j, channels 64g + 8s .. +7;
// head h's row starts at qp + h * pitch.
template <int PITCH>
__device__ __forceinline__ void load_query_operand(const bf16_t* qp, int lane, bf16x8_t (&qa)[2][8]) {
  const int j = lane & 31, g = lane >> 5;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int s = 0; s < 8; ++s)
      qa[mt][s] = *reinterpret_cast<const bf16x8_t*>(qp + (mt * 32 + j) * PITCH + g * 64 + 8 * s);
}

// Row pitch (bf16) of the query heads staged in LDS by the decode kernel:
// 272 bytes, so the 16-byte reads of consecutive heads (one per lane) spread
// over the banks instead of all landing on one (a 256-byte pitch did: 5.2
// conflict cycles per access measured).
constexpr int kSqPitch = 136;

// Head weights matching the accumulator rows held by this lane.
__device__ __forceinline__ void load_head_weights(const float* wp, int lane, float (&wv)[2][16]) {
  const int g = lane >> 5;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) wv[mt][r] = wp[mt * 32 + 8 * (r >> 2) + 4 * g + (r & 3)];
}

// ReLU as an integer max of the float's bits (negative floats are negative
// integers): one instruction, where fmaxf adds a canonicalisation of the
// MFMA result first.  -0 maps to +0.
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

__device__ __forceinline__ float tile_score(const bf16x8_t (&qa)[2][8], const bf16x8_t (&kb)[8],
                                            const float (&wv)[2][16]) {
  f32x16_t c0 = {}, c1 = {};
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[0][s], kb[s], c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[1][s], kb[s], c1, 0, 0, 0);
  }
  float sc = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) sc += wv[0][r] * relu(c0[r]);
#pragma unroll
  for (int r = 0; r < 16; ++r) sc += wv[1][r] * relu(c1[r]);
  // the other half of the heads sits in lane l ^ 32: v_permlane32_swap (a
  // VALU move, no LDS round trip)
  const uint32_t u = __float_as_uint(sc);
  const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return sc + __uint_as_float(__lane_id() < 32 ? sw[1] : sw[0]);
}

// A lane's share of one key for the decode kernel: channels 64g .. 64g + 63
// of key (l % 32), as eight bf16x8 operands, or as MX FP4 codes (32 bytes)
// with the scale bytes of its two 32-channel blocks, converted when scored.
template <bool FP4>
struct KeyTile;
template <>
struct KeyTile<false> {
  bf16x8_t v[8];
};
template <>
struct KeyTile<true> {
  uint4 c[2];
  uint32_t s;
};

__device__ __forceinline__ void fp4_operand(const KeyTile<true>& kt, bf16x8_t (&kb)[8]) {
  const float s0 = mx_scale_value(kt.s & 255u), s1 = mx_scale_value((kt.s >> 8) & 255u);
  const uint32_t w[8] = {kt.c[0].x, kt.c[0].y, kt.c[0].z, kt.c[0].w,
                         kt.c[1].x, kt.c[1].y, kt.c[1].z, kt.c[1].w};
#pragma unroll
  for (int s = 0; s < 8; ++s) kb[s] = fp4x8_to_bf16(w[s], s < 4 ? s0 : s1);
}

// ------------------------------------------------------------ fresh entries
// The block of m tokens that closes at this decode step, pooled into one
// entry as the compressor does ("DeepSeek-v4 Beyond Basics" section 3.2.2,
// eqs. 9-12; compress.hip): per channel, a softmax over the block's rows of
// z + bias (with overlap, also the previous block's second-stream rows)
// weights the rows of c; then RMSNorm with the gain, and RoPE of the last
// rope_dims channels at the block's position.  One workgroup; thread t holds
// channels 2t and 2t + 1.  The entry goes to row n_entries - 1 of the job's
// pool when the step closes a block for the sequence (the rule of job jrow),
// or with `ring` to the window ring's slot.  For the indexer-key job the
// entry is then scored against every query of the sequence that sees it,
// from the bf16 value as stored.
// 8 rows: a CSA block with its overlap (2m, m = 4) or a window row; larger
// blocks run the compressor as a launch of its own.  The bound sizes the
// row registers, and with it the fused kernel's occupancy (85 VGPRs at 8
// rows, 123 at 16).
constexpr int kFreshMaxRows = 8;

__device__ __forceinline__ void fresh_entry(const IndexArgs& a, const CompressArgs& j,
                                            const CompressArgs& jrow, bool ring, int b,
                                            bool score, float* skey, float* red) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int D = j.D, m = j.m;
  const int c0 = 2 * tid;
  const bool act = c0 < D;
  const int cc = act ? c0 : 0;
  // The row addresses come from the arguments alone, so every load is issued
  // before the first scalar load (the block's start, the entry count) has
  // returned: the previous block's stream is read whenever it is given and
  // pooled only when there is a block before this one (nr rows); rows past
  // the block re-read row 0 and are dropped.
  const bool has_prev = j.overlap && j.prev_c_b;
  const int nr_max = m + (has_prev ? m : 0);
  const bf16_t* ca = (const bf16_t*)j.c_a + (int64_t)b * j.T * D;
  const bool hza = j.z_a != nullptr;
  const bf16_t* za = hza ? (const bf16_t*)j.z_a + (int64_t)b * j.T * D : ca;
  const bf16_t* cb = has_prev ? (const bf16_t*)j.prev_c_b + (int64_t)b * m * D : ca;
  const bf16_t* zb = has_prev ? (const bf16_t*)j.prev_z_b + (int64_t)b * m * D : za;
  uint32_t cw[kFreshMaxRows], zw[kFreshMaxRows];
  float2 bw[kFreshMaxRows];
#pragma unroll
  for (int r = 0; r < kFreshMaxRows; ++r) {
    const int rr = r < nr_max ? r : 0;
    const bool in_a = rr < m;
    const int64_t ro = (int64_t)(in_a ? rr : rr - m) * D + cc;
    cw[r] = *reinterpret_cast<const uint32_t*>((in_a ? ca : cb) + ro);
    zw[r] = *reinterpret_cast<const uint32_t*>((in_a ? za : zb) + ro);
    const float* bp = in_a ? j.bias_a : j.bias_b;
    bw[r] = bp ? *reinterpret_cast<const float2*>(bp + ro) : make_float2(0.f, 0.f);
  }
  const float2 gn = j.gain ? *reinterpret_cast<const float2*>(j.gain + cc) : make_float2(1.f, 1.f);
  const int64_t pos = j.pos0 ? j.pos0[b] : 0;
  const bool prev = has_prev && !(j.pos0 && pos < m);
  const int nr = m + (prev ? m : 0);
  // scoring (indexer-key job): thread (h = tid / 4, quarter qq = tid % 4)
  // takes head h over channels 32 qq .. 32 qq + 31; the first query's slice
  // and weight are requested with the rows
  const int h = tid >> 2, qq = tid & 3;
  auto qslice = [&](int query, uint4 (&qv)[4]) {
    const uint4* qp = reinterpret_cast<const uint4*>((const bf16_t*)a.q +
                                                     ((int64_t)query * 64 + h) * 128 + 32 * qq);
#pragma unroll
    for (int u = 0; u < 4; ++u) qv[u] = qp[u];
  };
  uint4 qv0[4];
  float wh0 = 0.f;
  if (score) {
    qslice(b * a.Tq, qv0);
    wh0 = a.w[(int64_t)b * a.Tq * 64 + h];
  }
  // the sequence's entry count and first query position, requested early too
  const int n_ent = min(a.n_entries[b], a.N_cap);
  const int64_t qpos = a.q_pos0[b];
  // the output row, decided once the loads are in flight: an entry goes to
  // row n_entries - 1 of its pool when the step closes a block (the rule of
  // the key job, jrow), a window row to its ring slot; -1: nothing is stored
  const int row = ring ? (int)compress_out_row(j, b, 0)
                       : (compress_out_row(jrow, b, 0) >= 0 ? n_ent - 1 : -1);
  // the RoPE angle of this thread's channel pair depends on the position
  // alone: computed while the rows are in flight
  const int R = j.rope_dims;
  const bool rot = R > 0 && act && c0 >= D - R;
  float cs = 1.f, sn = 0.f;
  if (rot) rope_cos_sin(pos, (c0 - (D - R)) >> 1, j.rope_theta1, cs, sn);

  auto logit = [&](int r, int e) {  // base-2 logit of row r, channel c0 + e
    const bool in_a = r < m;
    const float z = (in_a ? hza : true) ? bf16_to_f32(e ? zw[r] >> 16 : zw[r] & 0xffffu) : 0.f;
    return (z + (e ? bw[r].y : bw[r].x)) * kLog2e;
  };
  float mx0 = -INFINITY, mx1 = -INFINITY;
#pragma unroll
  for (int r = 0; r < kFreshMaxRows; ++r) {
    if (r < nr) {
      mx0 = fmaxf(mx0, logit(r, 0));
      mx1 = fmaxf(mx1, logit(r, 1));
    }
  }
  float den0 = 0.f, den1 = 0.f, acc0 = 0.f, acc1 = 0.f;
#pragma unroll
  for (int r = 0; r < kFreshMaxRows; ++r) {
    if (r < nr) {
      const float p0 = exp2_weight(logit(r, 0) - mx0);
      const float p1 = exp2_weight(logit(r, 1) - mx1);
      den0 += p0;
      den1 += p1;
      acc0 += p0 * bf16_to_f32(cw[r] & 0xffffu);
      acc1 += p1 * bf16_to_f32(cw[r] >> 16);
    }
  }
  float y0 = acc0 / den0, y1 = acc1 / den1;
  if (j.gain) {
    float ss = act ? y0 * y0 + y1 * y1 : 0.f;
    ss = wave_sum(ss);
    if (lane == 0) red[wave] = ss;
    __syncthreads();
    ss = red[0] + red[1] + red[2] + red[3];
    const float inv = 1.0f / sqrtf(ss / (float)D + j.eps);
    y0 = y0 * inv * gn.x;
    y1 = y1 * inv * gn.y;
  }
  if (rot) {
    const float x0 = y0, x1 = y1;
    y0 = x0 * cs - x1 * sn;
    y1 = x0 * sn + x1 * cs;
  }
  // the stored values, as the scorer sees them
  float v0, v1;
  const int64_t at = (int64_t)b * j.out_bstride + (int64_t)row * D;  // channel offset
  if (j.out_fp8_row > 0) {
    // packed mixed BF16 / FP8 row (the KV job, D = 512; never scored): the
    // 16 threads of a 32-channel block share its scale
    const int Dr = D - j.rope_dims;
    const bool f8 = act && c0 < Dr;
    float am = f8 ? fmaxf(fabsf(y0), fabsf(y1)) : 0.f;
    am = fmaxf(am, __shfl_xor(am, 1));
    am = fmaxf(am, __shfl_xor(am, 2));
    am = fmaxf(am, __shfl_xor(am, 4));
    am = fmaxf(am, __shfl_xor(am, 8));
    const uint32_t sb = mx8_scale_byte(am);
    uint8_t* rp = (uint8_t*)j.out + (int64_t)b * j.out_bstride + (int64_t)row * j.out_fp8_row;
    if (row < 0) return;
    if (f8) {
      *reinterpret_cast<uint16_t*>(rp + c0) = (uint16_t)(e4m3_code(y0, sb) | (e4m3_code(y1, sb) << 8));
      if ((tid & 15) == 0) rp[D + j.rope_dims + (c0 >> 5)] = (uint8_t)sb;
    } else if (act) {
      *reinterpret_cast<uint32_t*>(rp + Dr + 2 * (c0 - Dr)) = pack_bf16x2(y0, y1);
    }
    if (tid == 0) {
      for (int p = D + j.rope_dims + Dr / 32; p < j.out_fp8_row; ++p) rp[p] = 0;
    }
    return;
  }
  if (j.out_scales) {
    // MX FP4: the 16 lanes of a 32-channel block share its scale
    float am = act ? fmaxf(fabsf(y0), fabsf(y1)) : 0.f;
    am = fmaxf(am, __shfl_xor(am, 1));
    am = fmaxf(am, __shfl_xor(am, 2));
    am = fmaxf(am, __shfl_xor(am, 4));
    am = fmaxf(am, __shfl_xor(am, 8));
    const uint32_t sb = mx_scale_byte(am);
    const uint32_t e0 = e2m1_code(y0, sb), e1 = e2m1_code(y1, sb);
    if (act && row >= 0) {
      ((uint8_t*)j.out)[at / 2 + tid] = (uint8_t)(e0 | (e1 << 4));
      if ((tid & 15) == 0) j.out_scales[at / 32 + (tid >> 4)] = (uint8_t)sb;
    }
    v0 = e2m1_value(e0, sb);
    v1 = e2m1_value(e1, sb);
  } else {
    const uint32_t packed = pack_bf16x2(y0, y1);
    if (act && row >= 0) *reinterpret_cast<uint32_t*>((bf16_t*)j.out + at + c0) = packed;
    v0 = bf16_to_f32(packed & 0xffffu);
    v1 = bf16_to_f32(packed >> 16);
  }
  if (!score || row < 0) return;

  // Score the stored entry for every query t of the sequence that sees it:
  // the 4 quarters of a head meet by lane swaps, the 64 heads by a wave sum
  // and the 4 waves through LDS.
  if (act) {
    skey[c0] = v0;
    skey[c0 + 1] = v1;
  }
  __syncthreads();
  for (int t = 0; t < a.Tq; ++t) {
    const int query = b * a.Tq + t;
    if (row >= visible_entries(qpos + t, a.m, n_ent)) continue;
    uint4 qv[4];
    float wh = wh0;
    if (t == 0) {
#pragma unroll
      for (int u = 0; u < 4; ++u) qv[u] = qv0[u];
    } else {
      qslice(query, qv);
      wh = a.w[(int64_t)query * 64 + h];
    }
    float dot = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t wd[4] = {qv[u].x, qv[u].y, qv[u].z, qv[u].w};
      const float* kc = skey + 32 * qq + 8 * u;
      const f32x4_t k0 = *reinterpret_cast<const f32x4_t*>(kc);
      const f32x4_t k1 = *reinterpret_cast<const f32x4_t*>(kc + 4);
      const float kv[8] = {k0[0], k0[1], k0[2], k0[3], k1[0], k1[1], k1[2], k1[3]};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dot += bf16_to_f32(wd[e] & 0xffffu) * kv[2 * e];
        dot += bf16_to_f32(wd[e] >> 16) * kv[2 * e + 1];
      }
    }
    dot += __shfl_xor(dot, 1);
    dot += __shfl_xor(dot, 2);
    const float v = wave_sum(qq == 0 ? wh * fmaxf(dot, 0.f) : 0.f);
    if (lane == 0) red[wave] = v;
    __syncthreads();
    if (tid == 0) a.scores[(int64_t)query * a.N_cap + row] = red[0] + red[1] + red[2] + red[3];
    __syncthreads();
  }
}

// ------------------------------------------------------------------- decode
// 1-D grid: [fresh workgroups,] then chunks x (B*Tq) scoring workgroups, 4
// waves each; chunk = 4 * tiles_per_wave tiles of 32 keys, tiles
// interleaved over the waves so the WG reads one contiguous range.
// FRESH: the first n_jobs * B workgroups (dispatched first) compress the
// closing block of sequence x % B for job x / B (fresh_entry); the scoring
// workgroups score the entries stored before it.
// ONE: one tile per wave (tiles_per_wave == 1): a single key buffer, so the
// kernel fits three waves per SIMD (3 workgroups per CU) and a grid of up
// to 768 workgroups, fresh ones included, runs in one round.
template <bool FRESH, bool ONE, bool FP4>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(ONE ? 3 : 1, 8)))
void index_decode(IndexArgs a, int tiles_per_wave, int chunks, FreshJobs f) {
  __shared__ __attribute__((aligned(16))) bf16_t sq[64 * kSqPitch];
  // head weights: thread i stores a copy of weights 4(i%16) .. +3 in slot i
  // (a store in every thread: a branch around it would drag its load along)
  __shared__ __attribute__((aligned(16))) float sw[256 * 4];
  int id = blockIdx.x;
  if constexpr (FRESH) {
    const int fj = f.n_jobs * a.B;
    if (id < fj) {
      const int fb = id % a.B, jk = id / a.B;
      // entries go to row n_entries - 1 (when the step closes a block); the
      // window row (job 2) to its ring slot
      // (-1: no block closes for the sequence at this step; the entry is
      // still pooled, as its loads do not wait for this, but not stored).
      // One call per job index, so that each reads its job's fields at fixed
      // argument offsets (with a computed index the fields came through a
      // chain of dependent scalar loads ahead of the first row load).
      float* skey = reinterpret_cast<float*>(sq);
      if (jk == 0) fresh_entry(a, f.job[0], f.job[0], false, fb, true, skey, sw);
      else if (jk == 1) fresh_entry(a, f.job[1], f.job[0], false, fb, false, skey, sw);
      else fresh_entry(a, f.job[2], f.job[2], true, fb, false, skey, sw);
      return;
    }
    id -= fj;
  }
  const int query = id / chunks;
  const int cx = id - query * chunks;  // chunk of this scoring workgroup
  const int b = query / a.Tq;
  const int t = query - b * a.Tq;
  const int64_t tpos = a.q_pos0[b] + t;
  const int n_ent = a.n_entries[b];
  const int chunk_tiles = 4 * tiles_per_wave;
  const int tile0 = cx * chunk_tiles;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int j = lane & 31, g = lane >> 5;
  float* out = a.scores + (int64_t)query * a.N_cap;
  // key rows past the visible range are read (every row below N_cap is
  // allocated) but never scored, so no load waits for the visible count
  auto load = [&](int tl, KeyTile<FP4>& dst) {
    const int64_t row = (int64_t)b * a.N_cap + min(tl * 32 + j, a.N_cap - 1);
    if constexpr (FP4) {
      const uint4* cp = reinterpret_cast<const uint4*>((const uint8_t*)a.k + row * 64 + g * 32);
      dst.c[0] = cp[0];
      dst.c[1] = cp[1];
      dst.s = *reinterpret_cast<const uint16_t*>(a.ks + row * 4 + 2 * g);
    } else {
      const bf16_t* kp = (const bf16_t*)a.k + row * 128 + g * 64;
#pragma unroll
      for (int s = 0; s < 8; ++s) dst.v[s] = *reinterpret_cast<const bf16x8_t*>(kp + 8 * s);
    }
  };

  // the query's 64 x 128 head matrix and head weights, fetched once per
  // workgroup (4 + 1 vector loads per thread) and shared by its waves; the
  // first key tile is requested behind them, before the visible count is
  // known, so its latency overlaps theirs.  No branch separates these loads
  // from their use (a workgroup past the visible range runs through with an
  // empty tile loop), so the compiler keeps them at the top.
  uint4 v[4];
  const uint4* qg = reinterpret_cast<const uint4*>((const bf16_t*)a.q + (int64_t)query * 64 * 128);
#pragma unroll
  for (int u = 0; u < 4; ++u) v[u] = qg[threadIdx.x + 256 * u];
  const f32x4_t wq = reinterpret_cast<const f32x4_t*>(a.w + (int64_t)query * 64)[threadIdx.x & 15];
  KeyTile<FP4> k0;
  int tile = tile0 + wave;
  load(tile, k0);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int c = threadIdx.x + 256 * u;  // 16-byte chunk c: head c / 16, channels 8 (c % 16)
    *reinterpret_cast<uint4*>(sq + (c >> 4) * kSqPitch + 8 * (c & 15)) = v[u];
  }
  reinterpret_cast<f32x4_t*>(sw)[threadIdx.x] = wq;
  // with fresh entries the last one is scored by its compressing workgroup
  // (a sequence whose step closes no block, negative block start, has none)
  const bool fresh_b = FRESH && !(f.job[0].pos0 && f.job[0].pos0[b] < 0);
  const int n_vis = fresh_b ? max(min(visible_entries(tpos, a.m, min(n_ent, a.N_cap)),
                                      min(n_ent, a.N_cap) - 1), 0)
                            : visible_entries(tpos, a.m, min(n_ent, a.N_cap));
  __syncthreads();
  bf16x8_t qa[2][8];
  load_query_operand<kSqPitch>(sq, lane, qa);
  float wv[2][16];
  load_head_weights(sw, lane, wv);

  const int tile_end = min(tile0 + chunk_tiles, (n_vis + 31) >> 5);
  auto score = [&](int tl, const KeyTile<FP4>& kt) {
    float sc;
    if constexpr (FP4) {
      bf16x8_t kb[8];
      fp4_operand(kt, kb);
      sc = tile_score(qa, kb, wv);
    } else {
      sc = tile_score(qa, kt.v, wv);
    }
    const int key = tl * 32 + j;
    if (g == 0 && key < n_vis) out[key] = sc;
  };
  if constexpr (ONE) {
    if (tile < tile_end) score(tile, k0);
    return;
  }
  if constexpr (FP4) {
    // An MX FP4 tile is a quarter of a bf16 one, so one tile ahead would keep
    // too few bytes in flight to cover the memory latency: a ring of four
    // tiles keeps three ahead (as many bytes as the bf16 kernel's one).  The
    // refills are unconditional (past the chunk they re-read its last tile,
    // never scored), so the waits before each tile count exactly.
    if (tile >= tile_end) return;
    const int last = tile_end - 1;
    KeyTile<true> r[4];
    r[0] = k0;
#pragma unroll
    for (int i = 1; i < 4; ++i) load(min(tile + 4 * i, last), r[i]);
    for (;;) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tl = tile + 4 * i;
        if (tl >= tile_end) return;
        score(tl, r[i]);
        load(min(tl + 16, last), r[i]);
      }
      tile += 16;
    }
  } else {
    // two key buffers in turn: the next tile's loads are in flight while the
    // current tile is scored, with no register copy between them
    KeyTile<false> k1;
    while (tile < tile_end) {
      const int t1 = tile + 4;
      if (t1 < tile_end) load(t1, k1);
      score(tile, k0);
      if (t1 >= tile_end) break;
      const int t2 = t1 + 4;
      if (t2 < tile_end) load(t2, k0);
      score(t1, k1);
      tile = t2;
    }
  }
}

// ------------------------------------------------------------------ prefill
// grid (ceil(Tq/8), B); 8 waves, wave w scores query 8*blockIdx.x + w
// against 64-key tiles in LDS (row pitch 272 bytes: the 16-byte column
// reads of 16 consecutive rows fall in distinct banks).
constexpr int kPfKeys = 64;
// s_waitcnt immediate for vmcnt(0) with lgkmcnt and expcnt left at their
// maxima (vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int kWaitVmcnt0 = 0x0F70;
constexpr int kPfPitch = 136;  // bf16 elements per LDS row

template <bool FP4>
__global__ __launch_bounds__(512) void index_prefill(IndexArgs a) {
  __shared__ __attribute__((aligned(16))) bf16_t kt[2][kPfKeys * kPfPitch];
  const int b = blockIdx.y;
  const int t0 = blockIdx.x * 8;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int j = lane & 31, g = lane >> 5;
  const int t = t0 + wave;
  const bool live = t < a.Tq;
  const int64_t pos_base = a.q_pos0[b];
  const int n_live = min(a.n_entries[b], a.N_cap);
  const int n_vis = live ? visible_entries(pos_base + t, a.m, n_live) : 0;
  const int t_last = min(t0 + 7, a.Tq - 1);
  const int n_max = visible_entries(pos_base + t_last, a.m, n_live);
  const int64_t query = (int64_t)b * a.Tq + (live ? t : t_last);

  bf16x8_t qa[2][8];
  load_query_operand<128>((const bf16_t*)a.q + query * 64 * 128, lane, qa);
  float wv[2][16];
  load_head_weights(a.w + query * 64, lane, wv);

  const int64_t kbase = (int64_t)b * a.N_cap;  // first key row of the sequence
  float* out = a.scores + query * a.N_cap;

  // cooperative tile load: 64 keys x 128 channels = 1024 pieces of 8
  // channels (16 B of bf16, or a code dword and a scale byte), 2 per thread;
  // FP4 pieces are converted to bf16 on their way into LDS
  struct Piece {
    uint4 v;
    uint32_t s;
  };
  const int p0 = threadIdx.x, p1 = threadIdx.x + 512;
  auto fetch_one = [&](int k0, int p, Piece& d) {
    const int64_t row = kbase + min(k0 + (p >> 4), max(n_max - 1, 0));
    if constexpr (FP4) {
      d.v.x = reinterpret_cast<const uint32_t*>(a.k)[row * 16 + (p & 15)];
      d.s = a.ks[row * 4 + ((p & 15) >> 2)];
    } else {
      d.v = *reinterpret_cast<const uint4*>((const bf16_t*)a.k + row * 128 + (p & 15) * 8);
    }
  };
  auto fetch = [&](int k0, Piece& v0, Piece& v1) {
    fetch_one(k0, p0, v0);
    fetch_one(k0, p1, v1);
  };
  auto put = [&](int buf, int p, const Piece& d) {
    uint4 v = d.v;
    if constexpr (FP4) {
      const bf16x8_t x = fp4x8_to_bf16(d.v.x, mx_scale_value(d.s));
      v = *reinterpret_cast<const uint4*>(&x);
    }
    *reinterpret_cast<uint4*>(&kt[buf][(p >> 4) * kPfPitch + (p & 15) * 8]) = v;
  };
  auto stash = [&](int buf, const Piece& v0, const Piece& v1) {
    put(buf, p0, v0);
    put(buf, p1, v1);
  };

  if (n_max <= 0) return;
  Piece v0, v1;
  fetch(0, v0, v1);
  stash(0, v0, v1);
  // the query operand has landed before the loop: otherwise the compiler's
  // conservative count makes the loop's MFMAs wait on the next tile's fetch
  // (the builtin, not inline asm: the compiler's wait counting sees it)
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  int buf = 0;
  for (int k0 = 0; k0 < n_max; k0 += kPfKeys) {
    const bool more = k0 + kPfKeys < n_max;
    if (more) fetch(k0 + kPfKeys, v0, v1);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      bf16x8_t kb[8];
      const bf16_t* row = &kt[buf][(nt * 32 + j) * kPfPitch + g * 64];
#pragma unroll
      for (int s = 0; s < 8; ++s) kb[s] = *reinterpret_cast<const bf16x8_t*>(row + 8 * s);
      const float sc = tile_score(qa, kb, wv);
      const int key = k0 + nt * 32 + j;
      if (g == 0 && key < n_vis) out[key] = sc;
    }
    if (more) stash(buf ^ 1, v0, v1);
    __syncthreads();
    buf ^= 1;
  }
}

bool index_uses_mfma(const IndexArgs& a) { return a.dt == 1 && a.Hi == 64 && a.Di == 128; }

// Tiles of 32 keys per wave for the decode kernel.  Two workgroups fit a CU,
// so a grid of whole rounds of 512 runs balanced.  bf16 keys: ~1k workgroups
// (two rounds; at 1M, 16 tiles per wave measured 103.5 us against 109.6 for
// 2.9 rounds of 11).  MX FP4 keys are a quarter of the bytes and the kernel
// is bound by its per-tile work, so one round of ~512 spreads the workgroup
// prologue (query to LDS and registers) over the most tiles.
static int decode_tiles_per_wave(const IndexArgs& a) {
  const int64_t keys = (int64_t)a.B * a.Tq * a.N_cap;
  const int64_t per = (a.ks ? 512LL : 1024LL) * 128;
  const int tpw = (int)((keys + per - 1) / per);
  return max(1, min(tpw, 32));
}

hipError_t launch_index_scores(const IndexArgs& a, hipStream_t stream) {
  const int queries = a.B * a.Tq;
  if (queries == 0 || a.N_cap == 0) return hipSuccess;
  const bool fp4 = a.ks != nullptr;
  if (index_uses_mfma(a)) {
    if (a.Tq >= 8) {
      dim3 grid((a.Tq + 7) / 8, a.B);
      if (fp4)
        hipLaunchKernelGGL(index_prefill<true>, grid, dim3(512), 0, stream, a);
      else
        hipLaunchKernelGGL(index_prefill<false>, grid, dim3(512), 0, stream, a);
    } else {
      const int tpw = decode_tiles_per_wave(a);
      const int chunk = 4 * tpw * 32;
      const int chunks = (a.N_cap + chunk - 1) / chunk;
      dim3 grid(chunks * queries);
      const FreshJobs none{};
      if (fp4 && tpw == 1)
        hipLaunchKernelGGL((index_decode<false, true, true>), grid, dim3(256), 0, stream, a, tpw, chunks, none);
      else if (fp4)
        hipLaunchKernelGGL((index_decode<false, false, true>), grid, dim3(256), 0, stream, a, tpw, chunks, none);
      else if (tpw == 1)
        hipLaunchKernelGGL((index_decode<false, true, false>), grid, dim3(256), 0, stream, a, tpw, chunks, none);
      else
        hipLaunchKernelGGL((index_decode<false, false, false>), grid, dim3(256), 0, stream, a, tpw, chunks, none);
    }
    return hipGetLastError();
  }
  const size_t lds = ((size_t)a.Hi * a.Di + a.Hi) * sizeof(float);
  dim3 grid((a.N_cap + 255) / 256, queries);
  if (fp4)
    hipLaunchKernelGGL((index_generic<bf16_t, true>), grid, dim3(256), lds, stream, a);
  else if (a.dt == 1)
    hipLaunchKernelGGL((index_generic<bf16_t, false>), grid, dim3(256), lds, stream, a);
  else
    hipLaunchKernelGGL((index_generic<float, false>), grid, dim3(256), lds, stream, a);
  return hipGetLastError();
}

}  // namespace csa

namespace csa {

bool index_fresh_fused(const IndexArgs& a, const FreshJobs& f) {
  if (!index_uses_mfma(a) || a.Tq >= 8 || f.n_jobs < 1 || f.n_jobs > 3) return false;
  if (f.job[0].D != a.Di) return false;
  // MX FP4 keys: the key job stores FP4 (whole 32-channel blocks), others bf16
  if ((a.ks != nullptr) != (f.job[0].out_scales != nullptr) || (a.ks && a.Di % 32)) return false;
  for (int k = 0; k < f.n_jobs; ++k) {
    const CompressArgs& j = f.job[k];
    if (k > 0 && j.out_scales) return false;
    if (j.out_fp8_row > 0 && (k != 1 || j.D != 512)) return false;
    const int rows = j.m * ((j.overlap && j.prev_c_b) ? 2 : 1);
    if (j.dt != 1 || j.T != j.m || j.D > 512 || (j.D & 1) || rows > kFreshMaxRows) return false;
  }
  return true;
}

hipError_t launch_index_fresh(const IndexArgs& a, const FreshJobs& f, hipStream_t stream) {
  const int queries = a.B * a.Tq;
  if (queries == 0) return hipSuccess;
  const int tpw = decode_tiles_per_wave(a);
  const int chunk = 4 * tpw * 32;
  const int chunks = (a.N_cap + chunk - 1) / chunk;
  dim3 grid(chunks * queries + f.n_jobs * a.B);
  const bool fp4 = a.ks != nullptr;
  if (fp4 && tpw == 1)
    hipLaunchKernelGGL((index_decode<true, true, true>), grid, dim3(256), 0, stream, a, tpw, chunks, f);
  else if (fp4)
    hipLaunchKernelGGL((index_decode<true, false, true>), grid, dim3(256), 0, stream, a, tpw, chunks, f);
  else if (tpw == 1)
    hipLaunchKernelGGL((index_decode<true, true, false>), grid, dim3(256), 0, stream, a, tpw, chunks, f);
  else
    hipLaunchKernelGGL((index_decode<true, false, false>), grid, dim3(256), 0, stream, a, tpw, chunks, f);
  return hipGetLastError();
}

}  // namespace csa
