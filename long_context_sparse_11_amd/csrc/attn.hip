// Shared-K=V multi-query attention with a per-head sink over a list of
// rows: the indexer-selected compressed entries (CSA) or every visible
// compressed entry (HCA), followed by the sliding-window rows.
//
//   "DeepSeek-v4 Beyond Basics" section 3.2.2 (eq. 19) and section 3.3
//   (eq. 26): the compressed entries are key and value of one KV head;
//   the window rows are concatenated with them.
//   "DeepSeek V4 Inside", "What does layer 0 sliding-window attention do to
//   p?" (eq. 27): sink logit in the denominator; scale 1/sqrt(head_dim).
//   transformers "DeepSeek-V4", "Arsitektur": interleaved partial RoPE on
//   the query, rotation by -t of the output's rope slice.
//
// attn_generic  any shape/dtype; one wave per (query, head), VALU.
// attn_hs       bf16, 64 heads x 512 (the Flash shape).  One workgroup of 4
//               waves per (query, key split); wave w owns heads 16w .. 16w+15
//               over all 512 channels.  A tile's 32 rows are copied HBM ->
//               LDS once (each row serves all 64 heads); QK^T and PV run on
//               v_mfma_f32_16x16x32_bf16 with an online softmax per head
//               (running max/sum, seeded empty; the sink enters once at the
//               end).
// combine       merges key-range splits and adds the sink once.
#include "kernels.h"

namespace csa {

// ----------------------------------------------------------- row addressing
struct KeyRange {
  int nsel;    // selected (CSA) or visible (HCA) compressed rows
  int nwin;    // window rows
  int win_r0;  // buffer row of the first window row
};

__device__ __forceinline__ KeyRange key_range(const AttnArgs& a, int b, int qi, int64_t tpos) {
  KeyRange k;
  k.nsel = a.csa ? a.K : visible_entries(tpos, a.m, min(a.n_entries[b], a.N_cap));
  k.nwin = 0;
  k.win_r0 = 0;
  if (a.W > 0 && a.L_win > 0 && !a.win_pos0) {  // ring: token p at row p % L_win
    const int64_t p_lo = max((int64_t)0, tpos - a.W + 1);
    if (tpos >= p_lo) {
      k.nwin = (int)(tpos - p_lo + 1);
      k.win_r0 = (int)(p_lo % a.L_win);
    }
  } else if (a.W > 0 && a.L_win > 0) {
    const int64_t p_lo = max((int64_t)0, tpos - a.W + 1);
    int64_t r_lo = p_lo - a.win_pos0[b];
    int64_t r_hi = tpos - a.win_pos0[b];
    if (r_lo < 0) r_lo = 0;
    if (r_hi > a.L_win - 1) r_hi = a.L_win - 1;
    if (r_hi >= r_lo) {
      k.nwin = (int)(r_hi - r_lo + 1);
      k.win_r0 = (int)r_lo;
    }
  }
  return k;
}

// Row j of the query's key list; `valid` false for an empty (-1) slot, in
// which case a harmless in-bounds row is returned.
template <typename T>
__device__ __forceinline__ const T* key_row(const AttnArgs& a, int b, int qi, const KeyRange& kr,
                                            int j, bool& valid) {
  if (j < kr.nsel) {
    int s = j;
    valid = true;
    if (a.csa) {
      s = a.idx[(int64_t)qi * a.K + j];
      valid = s >= 0 && s < a.N_cap;
      if (!valid) s = 0;
    }
    return (const T*)a.pool + ((int64_t)b * a.N_cap + s) * a.D;
  }
  valid = true;
  int r = kr.win_r0 + (j - kr.nsel);  // wraps only in a ring
  if (r >= a.L_win) r -= a.L_win;
  return (const T*)a.win + ((int64_t)b * a.L_win + r) * a.D;
}

// ------------------------------------------------------------------ generic
// grid (ceil(H/4), B*Tq), 256 threads; lane holds channel pairs
// (2p, 2p+1) for p = lane + 64k, k < NP.
template <typename T, int NP>
__global__ __launch_bounds__(256) void attn_generic(AttnArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h = blockIdx.x * 4 + wave;
  if (h >= a.H) return;
  const int qi = blockIdx.y;
  const int b = qi / a.Tq, t = qi - b * a.Tq;
  const int64_t tpos = a.q_pos0[b] + t;
  const int D = a.D, R = a.R;
  const KeyRange kr = key_range(a, b, qi, tpos);
  const int L = kr.nsel + kr.nwin;

  float q0[NP], q1[NP], o0[NP], o1[NP], cs[NP], sn[NP];
  bool live[NP], rot[NP];
  const T* qp = (const T*)a.q + ((int64_t)qi * a.H + h) * D;
#pragma unroll
  for (int k = 0; k < NP; ++k) {
    const int c = 2 * (lane + 64 * k);
    live[k] = c < D;
    rot[k] = live[k] && c >= D - R;
    q0[k] = live[k] ? Elem<T>::get(qp + c) : 0.f;
    q1[k] = live[k] ? Elem<T>::get(qp + c + 1) : 0.f;
    cs[k] = 1.f;
    sn[k] = 0.f;
    if (rot[k]) {
      rope_cos_sin(tpos, (c - (D - R)) >> 1, a.rope_theta1, cs[k], sn[k]);
      const float x0 = q0[k], x1 = q1[k];
      q0[k] = x0 * cs[k] - x1 * sn[k];
      q1[k] = x0 * sn[k] + x1 * cs[k];
    }
    o0[k] = 0.f;
    o1[k] = 0.f;
  }
  float mrun = -INFINITY, lrun = 0.f;
  for (int jj = 0; jj < L; ++jj) {
    bool valid;
    const T* rp = key_row<T>(a, b, qi, kr, jj, valid);
    if (!valid) continue;  // uniform across the wave
    float r0[NP], r1[NP], dot = 0.f;
#pragma unroll
    for (int k = 0; k < NP; ++k) {
      const int c = 2 * (lane + 64 * k);
      r0[k] = live[k] ? Elem<T>::get(rp + c) : 0.f;
      r1[k] = live[k] ? Elem<T>::get(rp + c + 1) : 0.f;
      dot += q0[k] * r0[k] + q1[k] * r1[k];
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) dot += __shfl_xor(dot, off);
    const float z = dot * a.scale;
    const float mn = fmaxf(mrun, z);
    const float al = expf(mrun - mn);
    const float p = expf(z - mn);
    lrun = lrun * al + p;
    mrun = mn;
#pragma unroll
    for (int k = 0; k < NP; ++k) {
      o0[k] = o0[k] * al + p * r0[k];
      o1[k] = o1[k] * al + p * r1[k];
    }
  }
  const float sk = a.sink[h];
  const float mf = fmaxf(mrun, sk);
  const float lf = lrun * expf(mrun - mf) + expf(sk - mf);
  const float fac = expf(mrun - mf) / lf;
  if (lane == 0 && a.lse) a.lse[(int64_t)qi * a.H + h] = mf + logf(lf);
  T* op = (T*)a.out + ((int64_t)qi * a.H + h) * D;
#pragma unroll
  for (int k = 0; k < NP; ++k) {
    if (!live[k]) continue;
    float x0 = o0[k] * fac, x1 = o1[k] * fac;
    if (rot[k]) {  // rotate by -t: cos unchanged, sin negated
      const float y0 = x0 * cs[k] + x1 * sn[k];
      const float y1 = -x0 * sn[k] + x1 * cs[k];
      x0 = y0;
      x1 = y1;
    }
    const int c = 2 * (lane + 64 * k);
    Elem<T>::put(op + c, x0);
    Elem<T>::put(op + c + 1, x1);
  }
}

// --------------------------------------------------------------------- MFMA
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t* lds_s16x4_ptr;
constexpr int kAtD = 512;
constexpr int kAtH = 64;      // heads per workgroup (NW = 4)
constexpr int kMaxAtH = 128;  // H: a multiple of kAtH up to this (Flash 64, Pro 128)

// Value of lane (l ^ 32): the two halves of the wave swap through
// v_permlane32_swap (a VALU move; no LDS round trip).
__device__ __forceinline__ float half_swap(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(__lane_id() < 32 ? r[1] : r[0]);
}

// ------------------------------------------------------------- head split
// attn_hs: bf16, 64 heads x 512 (the Flash shape).  One workgroup of 4 waves
// per (query, key split); wave w owns heads 16w .. 16w+15 over all 512
// channels, so each head's logits are complete inside one wave: no partial
// logits cross waves and each head's online softmax runs once.
//
// A tile's 32 rows are copied HBM -> LDS once (buffer loads into LDS, 16
// bytes per lane, a whole 1 KiB row per wave instruction) and serve the four waves;
// tiles are double-buffered.  MFMA v_mfma_f32_16x16x32_bf16 throughout
// (lane l feeds A[l % 16][8(l/16) .. +7] and B[8(l/16) .. +7][l % 16];
// accumulator element r is C[4(l/16) + r][l % 16]):
//   S^T[key][head] += R[key][ch] Q^T[ch][head]: A = 16 rows x 32 channels
//     from LDS, B = the lane's query slice held in registers;
//   O^T[ch][head] += R^T[ch][key] P^T[key][head]: B = the lane's own
//     softmax values (the contraction's key slots are permuted so that the
//     accumulator layout of S^T is the operand layout of P^T: slot e < 4 is
//     key 4(l/16) + e, slot e >= 4 is key 16 + 4(l/16) + e - 4), A = rows
//     read transposed from LDS (ds_read_b64_tr_b16, the same key permutation).
// Row r of a tile stores its 16-byte chunk c at position c ^ hs_swz(r), which
// keeps both read patterns free of bank conflicts.
constexpr int kHsRows = 32;
// single-tile grids of at most this many workgroups after halving the heads
// take head groups (one workgroup per compute unit)
constexpr int64_t kHsHeadSplitBelow = 256;
// word 3 of a raw (untyped) buffer descriptor: 32-bit data format
constexpr int kRawBufferWord3 = 0x00020000;
constexpr int kHsMaxSplitRows = 2048;  // rows of a multi-tile CSA split (LDS index stage)

// LDS banks (64 x 4 bytes), as measured with the bank-conflict counter:
// a 16-byte read serves 16 lanes per cycle, those with equal lane bit 5 and
// equal parity of lane bits 2-4; a transposing 8-byte read serves 32
// consecutive lanes per cycle.  With chunk c of row r at c ^ ((r & 7) << 1):
// in a QK read the 8 lanes of a cycle with even G (l / 16) get the even
// slots 2(r & 7) (distinct, as r & 7 is) and those with odd G the odd ones;
// in a transposing read each row's 32 bytes go to the slot pair r & 7,
// distinct over the 8 rows of a 32-lane half.  No read conflicts.
// hs_swz < 16 changes only the low 4 bits of a chunk index, so a read's
// address is written as a per-lane base (from the low bits) plus a constant
// offset (from the high bits) that the compiler folds into the instruction.
__device__ __forceinline__ int hs_swz(int r) { return (r & 7) << 1; }

// Value of lane (l ^ 16): v_permlane16_swap exchanges 16-lane rows 0<->1, 2<->3.
__device__ __forceinline__ float row_swap16(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __uint_as_float(((__lane_id() >> 4) & 1) ? r[0] : r[1]);
}

typedef __attribute__((address_space(3))) void* lds_void_ptr;

// ------------------------------------------- HCA decode step: the new entry
// Row of the pool that a decode step's closing block fills (the entry count
// already includes it), or -1 when no block closes for sequence b.
__device__ __forceinline__ int fresh_entry_row(const AttnArgs& a, int b) {
  return a.fj.pos0[b] >= 0 ? min(a.n_entries[b], a.N_cap) - 1 : -1;
}

// Row of the window buffer that holds the token at tpos (its ring slot, or
// its offset from win_pos0[b]), or -1 when the buffer does not hold it.
__device__ __forceinline__ int window_slot(const AttnArgs& a, int b, int64_t tpos) {
  if (a.L_win <= 0 || tpos < 0) return -1;
  if (!a.win_pos0) return (int)(tpos % a.L_win);
  const int64_t r = tpos - a.win_pos0[b];
  return (r >= 0 && r < a.L_win) ? (int)r : -1;
}

// The new row of a decode step, handled by the last split of its query
// inside the attention launch: hca_decode_attn's closing block, pooled
// beside the other splits' tile loops instead of in launches of its own
// ahead of them, or swa_decode_attn's token row.  "DeepSeek-v4 Beyond
// Basics" section 3.3 (eqs. 20-23): an HCA entry is the softmax-weighted
// pool of the block's m rows per channel, then RMSNorm with its gain and
// RoPE at the block's first position; a window row is the same with m = 1
// (its one row, normalised and rotated at its own position); the same
// section (eq. 26): the row is attended like every other visible one.
//
// Wave w pools rows w, w + NW, ... with an online softmax per channel (lane l
// holds channels 8l .. 8l + 7; eight rows' loads in flight per wave, the
// first batch issued before anything else, since its addresses depend on
// nothing); the waves' partials merge through LDS and wave 0 finishes the
// row: normalises, applies the gain, rotates, and passes the bf16 values a
// reader of the stored row gets back to the other waves through LDS.  The
// split's partial is that one row: the row with its rope slice rotated back
// by -tpos (rounded to bf16) as the unnormalised output, the same for every
// head, and per head a sum of 1 and the logit as the running maximum.  The
// logit q'.row (q' the query rotated at tpos) equals q.(the row rotated back
// by -tpos): a rotation moves to the other operand of a dot product, so it
// is the query's dot with that output chunk; it differs from the tile loop's
// q' rounded to bf16 by rounding alone.  Lane l keeps its 16-byte chunk l of
// everything, so each head's query load and partial store is one contiguous
// 1 KB access per wave, the logits are bf16 pair dots, and the 16 heads'
// logits reduce across the wave in 17 shuffles.  With NW = 2 the query
// slices go straight into LDS at the start (buffer loads into LDS: no
// registers held while the rows arrive).  The row is stored (head group 0
// only; bf16, or a packed mixed BF16 / FP8 row) after the partial.  With
// no new row, or one the query does not see, the partial is empty (maximum
// -inf, sum 0, zero output); the other splits leave the row out when the
// query sees it.
template <int NW, bool FP8>
__device__ __forceinline__ void fresh_split(const AttnArgs& a, int b, int qi, int sp, int S,
                                            bf16_t* s_q, bf16_t* s_buf) {
  // s_buf (32 KB) holds the waves' pooling partials, the row and four rope
  // tables; the barriers below order every LDS hand-over, so NW > 1
  static_assert(NW > 1 && NW * 6144 + 5120 <= kHsRows * kAtD * 2, "fresh split LDS layout");
  const CompressArgs& f = a.fj;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int m = f.m, c0 = 8 * lane;
  const bool hz = f.z_a != nullptr, hb = f.bias_a != nullptr;
  const bf16_t* cbase = (const bf16_t*)f.c_a + (int64_t)b * m * kAtD + c0;
  const bf16_t* zbase = hz ? (const bf16_t*)f.z_a + (int64_t)b * m * kAtD + c0 : cbase;
  // the optional streams' words start at zero once (a skipped load leaves
  // them defined), and every load of a batch goes out before any arithmetic
  u32x4_t cw[8], zw[8], bw[8][2];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    zw[u] = u32x4_t{0u, 0u, 0u, 0u};
    bw[u][0] = bw[u][1] = u32x4_t{0u, 0u, 0u, 0u};
  }
  auto issue = [&](int r0) {  // rows r0, r0 + NW, ... (8 of them; past m, r0 again)
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int r = r0 + u * NW;
      const int64_t ro = (int64_t)(r < m ? r : r0) * kAtD;
      Elem<bf16_t>::template load_raw_stream<8>(cbase + ro, &cw[u]);
      if (hz) Elem<bf16_t>::template load_raw_stream<8>(zbase + ro, &zw[u]);
      if (hb) Elem<float>::template load_raw<8>(f.bias_a + ro + c0, bw[u]);
    }
  };
  if (wave < m) issue(wave);  // [B, m, D] rows: in bounds whether or not a row is new

  // this wave's 16 heads: head 16 (NW z + wave) + k, its query slice at
  // q + (qi H + h) D; with NW = 2, k-th slice into LDS row 16 wave + k
  const int hw = 16 * (NW * (int)blockIdx.z + wave);
  const bf16_t* qbase = (const bf16_t*)a.q + ((int64_t)qi * a.H + hw) * kAtD;
  constexpr bool kQLds = NW == 2;  // 32 heads x 1 KB: the 32 KB s_q holds them
  if constexpr (kQLds) {
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)qbase, (short)0, 16 * kAtD * 2, kRawBufferWord3);
#pragma unroll
    for (int k = 0; k < 16; ++k)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_ptr)(s_q + (16 * wave + k) * kAtD),
                                               16, 16 * lane + 1024 * k, 0, 0, 0);
  }

  const int R = a.R, rope0 = kAtD - R;
  const int64_t tpos = a.q_pos0[b];  // one query per sequence
  const int64_t bp = f.pos0[b];
  // the new row: a pool entry (the closing block's), or the query token's
  // own window row (always the last of its window)
  const bool win_row = a.fresh == 2;
  const int row = win_row ? window_slot(a, b, tpos) : fresh_entry_row(a, b);
  // whether the query sees the row: a window row whenever there is a window
  // (it is the window's last token), a pool entry once the query's position
  // reaches the entry's last token (all row + 1 entries visible)
  const bool vis =
      row >= 0 && (win_row ? a.W > 0 : tpos + 1 >= (int64_t)a.m * (int64_t)(row + 1));
  // rope tables (one pair per thread, the rows' loads in flight): at tpos
  // for the query and the rotation back, at bp for the row (a window row's
  // own position is tpos)
  float* s_f = reinterpret_cast<float*>(s_buf);  // [NW][3][512]: max, sum, weighted sum
  bf16_t* s_row = s_buf + NW * 3 * kAtD * 2;     // the row's bf16 values
  float* s_tc = reinterpret_cast<float*>(s_row + kAtD);
  float* s_ts = s_tc + kAtD / 2;
  float* s_ec = win_row ? s_tc : s_ts + kAtD / 2;
  float* s_es = win_row ? s_ts : s_ec + kAtD / 2;
  for (int p = tid; p < R / 2; p += 64 * NW) {
    rope_cos_sin(tpos, p, a.rope_theta1, s_tc[p], s_ts[p]);
    if (!win_row) rope_cos_sin(bp, p, a.rope_theta1, s_ec[p], s_es[p]);
  }
  float gv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) gv[e] = 1.f;
  if (wave == 0 && f.gain) Elem<float>::template load<8>(f.gain + c0, gv);

  float y[8];
  u32x4_t ent = u32x4_t{0u, 0u, 0u, 0u};
  if (row >= 0) {
    float mx[8], den[8], acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) { mx[e] = -INFINITY; den[e] = 0.f; acc[e] = 0.f; }
    for (int r0 = wave; r0 < m; r0 += 8 * NW) {
      if (r0 != wave) issue(r0);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (r0 + u * NW >= m) break;
        float cv[8], zv[8], bv[8];
        Elem<bf16_t>::template from_raw<8>(&cw[u], cv);
        Elem<bf16_t>::template from_raw<8>(&zw[u], zv);
        Elem<float>::template from_raw<8>(bw[u], bv);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float l = (zv[e] + bv[e]) * kLog2e;  // base 2; absent streams read 0
          const float nm = fmaxf(mx[e], l);
          const float sc = exp2_weight(mx[e] - nm);
          const float p = exp2_weight(l - nm);
          den[e] = den[e] * sc + p;
          acc[e] = acc[e] * sc + p * cv[e];
          mx[e] = nm;
        }
      }
    }
    if constexpr (NW > 1) {
      float* mine = s_f + wave * 3 * kAtD;
#pragma unroll
      for (int e = 0; e < 8; e += 4) {
        *reinterpret_cast<f32x4_t*>(mine + c0 + e) = f32x4_t{mx[e], mx[e + 1], mx[e + 2], mx[e + 3]};
        *reinterpret_cast<f32x4_t*>(mine + kAtD + c0 + e) =
            f32x4_t{den[e], den[e + 1], den[e + 2], den[e + 3]};
        *reinterpret_cast<f32x4_t*>(mine + 2 * kAtD + c0 + e) =
            f32x4_t{acc[e], acc[e + 1], acc[e + 2], acc[e + 3]};
      }
      __syncthreads();
    }
    if (wave == 0) {
      for (int w = 1; w < NW && w < m; ++w) {
        const float* o = s_f + w * 3 * kAtD;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float om = o[c0 + e];
          const float M = fmaxf(mx[e], om);
          const float w0 = mx[e] == -INFINITY ? 0.f : exp2_weight(mx[e] - M);
          const float w1 = om == -INFINITY ? 0.f : exp2_weight(om - M);
          den[e] = den[e] * w0 + o[kAtD + c0 + e] * w1;
          acc[e] = acc[e] * w0 + o[2 * kAtD + c0 + e] * w1;
          mx[e] = M;
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = acc[e] / den[e];
      if (f.gain) {
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += y[e] * y[e];
        ss = wave_sum(ss);
        const float inv = 1.0f / sqrtf(ss / (float)kAtD + f.eps);
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = y[e] * inv * gv[e];
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {  // the row's rotation, at its own position
        const int c = c0 + 2 * k;
        if (c >= rope0) {
          const float cs = s_ec[(c - rope0) >> 1], sn = s_es[(c - rope0) >> 1];
          const float x0 = y[2 * k], x1 = y[2 * k + 1];
          y[2 * k] = x0 * cs - x1 * sn;
          y[2 * k + 1] = x0 * sn + x1 * cs;
        }
      }
      // the bf16 values a reader of the stored row gets back
      if constexpr (FP8) {
        ent = win_row ? u32x4_t{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]),
                                pack_bf16x2(y[4], y[5]), pack_bf16x2(y[6], y[7])}
                      : kv_fp8_row_values(lane, y, R);
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) ent[k] = pack_bf16x2(y[2 * k], y[2 * k + 1]);
      }
      if constexpr (NW > 1) *reinterpret_cast<u32x4_t*>(s_row + c0) = ent;
    }
  }
  if constexpr (kQLds) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the query slices
  if constexpr (NW > 1) __syncthreads();
  if (row >= 0 && wave != 0) ent = *reinterpret_cast<const u32x4_t*>(s_row + c0);

  // the row rotated back by -tpos: this lane's chunk of every head's output
  u32x4_t outw = u32x4_t{0u, 0u, 0u, 0u};
  float s[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) s[k] = 0.f;
  if (vis) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {  // this lane's pairs: rotated back where they are rope pairs
      const int c = c0 + 2 * k, pj = max(0, (c - rope0) >> 1);
      const float cs = s_tc[pj], sn = s_ts[pj];
      const float o0 = __uint_as_float(ent[k] << 16), o1 = __uint_as_float(ent[k] & 0xffff0000u);
      const uint32_t r = pack_bf16x2(o0 * cs + o1 * sn, -o0 * sn + o1 * cs);
      outw[k] = c >= rope0 ? r : ent[k];
    }
    // the query slices (NW = 4: loaded now), one 16-byte chunk per head
    u32x4_t qc[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      if constexpr (kQLds)
        qc[k] = *reinterpret_cast<const u32x4_t*>(s_q + (16 * wave + k) * kAtD + c0);
      else
        qc[k] = *reinterpret_cast<const u32x4_t*>(qbase + k * kAtD + c0);
    }
    // the rotation of the rope pairs moves from the query to the row:
    // q'.row = q.(row rotated back by -tpos), the output chunk itself, so
    // each head's logit is 4 two-product bf16 dots per lane
#pragma unroll
    for (int h = 0; h < 16; ++h) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        // copies first: a bit cast of a vector's element would read element 0
        const uint32_t qj = qc[h][k], oj = outw[k];
        s[h] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qj),
                                               __builtin_bit_cast(bf16x2_t, oj), s[h], false);
      }
    }
  }
  // 16 sums over 64 lanes: each xor step halves the values a lane keeps
  // (bit j of the lane picks the half), then two plain steps; lane l ends
  // with head l & 15's logit
#pragma unroll
  for (int j = 0, n = 16; n > 1; ++j, n >>= 1) {
    const bool hi = (lane >> j) & 1;
#pragma unroll
    for (int i = 0; i < n / 2; ++i) {
      const float keep = hi ? s[2 * i + 1] : s[2 * i], give = hi ? s[2 * i] : s[2 * i + 1];
      s[i] = keep + __shfl_xor(give, 1 << j);
    }
  }
  s[0] += __shfl_xor(s[0], 16);
  s[0] += __shfl_xor(s[0], 32);
  const int64_t slot0 = ((int64_t)qi * S + sp) * a.H + hw;
  if (lane < 16)
    *reinterpret_cast<float2*>(a.part_ml + 2 * (slot0 + lane)) =
        vis ? make_float2(s[0] * a.scale * kLog2e, 1.f) : make_float2(-INFINITY, 0.f);
#pragma unroll
  for (int k = 0; k < 16; ++k)
    *reinterpret_cast<u32x4_t*>(a.part_o + (slot0 + k) * kAtD + c0) = outw;

  // the row itself, last: nothing in this launch reads it back
  if (row >= 0 && wave == 0 && blockIdx.z == 0) {
    if (win_row) {
      *reinterpret_cast<u32x4_t*>((bf16_t*)a.win + ((int64_t)b * a.L_win + row) * kAtD + c0) = ent;
    } else if constexpr (FP8) {
      store_kv_fp8_row((uint8_t*)a.pool + ((int64_t)b * a.N_cap + row) * a.pool_row_bytes, lane,
                       y, R);
    } else {
      *reinterpret_cast<u32x4_t*>((bf16_t*)a.pool + ((int64_t)b * a.N_cap + row) * kAtD + c0) = ent;
    }
  }
}

// NW: waves per workgroup, 16 heads each.  With NW = 4 the workgroup takes
// all 64 heads and four waves share each copied tile; with NW = 2 (single-
// tile splits of few queries, i.e. decode) it takes 32 heads and blockIdx.z
// is the head group: half the query slice and half the partial output per
// workgroup, twice the workgroups.  A workgroup's rows and partials go
// through one compute unit, whose own rate bounds these short workgroups.
//
// FP8: the pool rows are packed mixed BF16 / FP8 rows (pool_row_bytes each:
// the non-RoPE channels as E4M3 codes with one E8M0 scale per 32 channels,
// the RoPE channels in bf16).  A pool row is copied raw into a staging row
// of LDS (the same buffer loads into LDS, 16 bytes per lane), and each wave,
// once its own copies have landed, converts its rows into the bf16 tile with
// v_cvt_scalef32_pk_bf16_fp8 (exact: an E4M3 value times a power of two fits
// bf16); window rows stay bf16 and are copied as before.  Everything after
// the tile copy is unchanged.
//
// Waves per SIMD: the bf16 multi-tile kernel is held to two (256 registers
// each), so that two workgroups share a compute unit and hide each other's
// copy, softmax and barrier waits; to fit, its operand reads run 4 ahead of
// the MFMAs (not 8 and 16) and its LDS addresses are recomputed per tile.
// Prefill attention: 579 -> 469 us.  The others keep one wave per SIMD: a
// single-tile split is one short workgroup per compute unit, and the FP8
// kernel's staging area leaves LDS for one workgroup.
template <bool CSA, bool MULTI, int NW, bool FP8, int RC = 0>
__global__ __launch_bounds__(64 * NW)
__attribute__((amdgpu_waves_per_eu(MULTI && !FP8 ? 2 : 1, MULTI && !FP8 ? 2 : 1)))
void attn_hs(AttnArgs a) {
  constexpr int RPW = kHsRows / NW;  // tile rows each wave copies
  // two row buffers as distinct objects: with every access naming a fixed
  // one, the compiler can tell that a copy into one does not touch the other
  // (it would otherwise wait for the copy before reading)
  __shared__ __attribute__((aligned(16))) bf16_t s_rows0[kHsRows * kAtD];
  __shared__ __attribute__((aligned(16))) bf16_t s_rows1[kHsRows * kAtD];
  __shared__ float s_cos[kAtD / 2], s_sin[kAtD / 2];
  __shared__ __attribute__((aligned(16))) int32_t s_idx[MULTI && CSA ? kHsMaxSplitRows : 4];
  // FP8: raw pool rows, one 1 KiB slot per tile row (a row's copy fills its
  // first pool_row_bytes; the lanes past it read nothing)
  __shared__ __attribute__((aligned(16))) uint8_t s_stage[FP8 ? kHsRows * 1024 : 16];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int c16 = lane & 15, G = lane >> 4;
  const int h = 16 * (NW * (int)blockIdx.z + wave) + c16;  // this lane's head
  const int qi = blockIdx.y, sp = blockIdx.x, S = gridDim.x;
  const int b = qi / a.Tq, t = qi - b * a.Tq;
  const int R = RC > 0 ? RC : a.R;  // RC: rope width fixed at compile time
  const int rope0 = kAtD - R;
  // HCA decode step: the last split pools the closing block's entry; the
  // others divide the key list among themselves
  if constexpr (!CSA) {
    if (a.fresh && sp == S - 1) {
      fresh_split<NW, FP8>(a, b, qi, sp, S, s_rows0, s_rows1);
      return;
    }
  }
  const int Sa = S - ((!CSA && a.fresh) ? 1 : 0);  // splits over the key list

  // ---- split bounds (CSA: a fixed range of [K selected, up to
  // min(W, L_win) window rows], known before the position)
  int start = 0, end = 0;
  if (CSA) {
    const int wc = (a.W > 0 && a.L_win > 0) ? min(a.W, a.L_win) : 0;
    const int Lmax = a.K + wc;
    const int per = (((Lmax + Sa - 1) / Sa) + kHsRows - 1) / kHsRows * kHsRows;
    start = min(Lmax, sp * per);
    end = min(Lmax, start + per);
  }
  // tile 0's selected indices: lane l (< 32) holds row start + l's (a
  // harmless word when there is none; every load here is unconditional so
  // the compiler counts outstanding loads exactly)
  const bool has_idx = CSA && a.K > 0;
  const int32_t* idx_q = has_idx ? a.idx + (int64_t)qi * a.K : (const int32_t*)a.q_pos0;
  const int32_t idx0 = idx_q[has_idx ? min(max(start + (lane & 31), 0), a.K - 1) : 0];

  // the lane's query slice: head h, channels 32 ks + 8G .. +7
  const bf16_t* qrow = (const bf16_t*)a.q + ((int64_t)qi * a.H + h) * kAtD;
  bf16x8_t qb[16];
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) qb[ks] = *reinterpret_cast<const bf16x8_t*>(qrow + 32 * ks + 8 * G);

  const int64_t tpos = a.q_pos0[b] + t;
  KeyRange kr = key_range(a, b, qi, tpos);
  if constexpr (!CSA) {
    // the closing block's entry, when the query sees it, is the last split's
    if (a.fresh == 1) {
      const int row = fresh_entry_row(a, b);
      if (row >= 0 && row == kr.nsel - 1) kr.nsel -= 1;
    } else if (a.fresh == 2) {  // the token's own window row: the last one
      if (window_slot(a, b, tpos) >= 0 && kr.nwin > 0) kr.nwin -= 1;
    }
  }
  if (!CSA) {
    const int L = kr.nsel + kr.nwin;
    const int per = (((L + Sa - 1) / Sa) + kHsRows - 1) / kHsRows * kHsRows;
    start = min(L, sp * per);
    end = min(L, start + per);
  }
  const bf16_t* win_b = (const bf16_t*)a.win + (int64_t)b * a.L_win * kAtD;
  const bf16_t* dummy = (const bf16_t*)a.q + (int64_t)qi * a.H * kAtD;  // 1 KiB always readable

  // A tile's 32 rows reach LDS in two steps.  resolve_tile: lane l (< 32)
  // turns row j0 + l (sidx_l: its selected index) into a source address with
  // selects, not branches (an invalid row reads a harmless 1 KiB), and the
  // tile's validity mask comes back.  issue_row(u): wave w copies row
  // RPW w + u with one buffer load into LDS (1 KiB); the row's address is read from
  // its lane into scalar registers and lane i fetches the 16-byte chunk that
  // belongs at position i (i ^ hs_swz(row)).
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const uint64_t pool_a = (uint64_t)((const uint8_t*)a.pool +
                                     (int64_t)b * a.N_cap * (FP8 ? a.pool_row_bytes : kAtD * 2));
  const uint64_t win_a = (uint64_t)win_b, dummy_a = (uint64_t)dummy;
  const int64_t pool_rb = FP8 ? a.pool_row_bytes : kAtD * 2;
  struct TileSrc {
    int lo, hi;  // this lane's row address
    uint32_t mask;
    uint32_t fp8;  // FP8: rows read from the pool (converted after the copy)
  };
  auto resolve_tile = [&](int j0, int sidx_l) -> TileSrc {
    const int jj = j0 + (lane & 31);
    const bool in_sel = jj < kr.nsel;
    const int srow = CSA ? sidx_l : jj;
    int wrow = jj - kr.nsel + kr.win_r0;  // buffer row; wraps only in a ring
    if (wrow >= a.L_win) wrow -= a.L_win;
    const bool valid =
        lane < 32 && jj < end && (in_sel ? (srow >= 0 && srow < a.N_cap) : jj - kr.nsel < kr.nwin);
    const uint64_t sa = in_sel ? pool_a + (uint64_t)((int64_t)srow * pool_rb)
                               : win_a + (uint64_t)((int64_t)wrow * (kAtD * 2));
    const uint64_t src = valid ? sa : dummy_a;
    return TileSrc{(int)(uint32_t)src, (int)(uint32_t)(src >> 32), (uint32_t)__ballot(valid),
                   FP8 ? (uint32_t)__ballot(valid && in_sel) : 0u};
  };
  // cache policy of the row copies: HCA reads each row once per call, so its
  // copies stream past the caches (nt: HCA 1M 50.5 -> 48.0 us); CSA's
  // selected rows can repeat across queries and stay cached (with nt the
  // prefill chunk's attention took 550 us against 472)
  constexpr int kRowPolicy = CSA ? 0 : 2;
  auto issue_row = [&](const TileSrc& ts, int u, bf16_t* dst) {
    const int r = RPW * wv + u;
    const uint64_t rs = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(ts.hi, r) << 32) |
                        (uint32_t)__builtin_amdgcn_readlane(ts.lo, r);
    if (FP8 && ((ts.fp8 >> r) & 1u)) {
      // a packed pool row, raw into its staging slot: lane i copies bytes
      // 16 i .. 16 i + 15; lanes past the row's end fall outside the
      // descriptor's range and read nothing
      const __amdgpu_buffer_rsrc_t rsrc =
          __builtin_amdgcn_make_buffer_rsrc((void*)rs, (short)0, a.pool_row_bytes, kRawBufferWord3);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_ptr)(s_stage + r * 1024), 16,
                                               16 * lane, 0, 0, kRowPolicy);
      return;
    }
    // a buffer load (not a global one): it counts on vmcnt only, so the
    // LDS reads issued around it keep exact lgkmcnt waits
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)rs, (short)0, kAtD * 2, kRawBufferWord3);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_ptr)(dst + r * kAtD), 16,
                                             16 * (lane ^ hs_swz(r)), 0, 0, kRowPolicy);
  };
  // FP8: this wave's staged pool rows into the bf16 tile (after its copies
  // have landed: the caller waits on vmcnt).  Lane l < nc holds channels
  // 8l .. 8l+7 (8 code bytes, the scale of their 32-channel block); the
  // other lanes one 16-byte chunk of the bf16 RoPE channels.  Each lane
  // writes its 16-byte chunk l of the row at the tile's swizzled position.
  const int nc = (kAtD - R) >> 3;
  auto convert_rows = [&](uint32_t fp8_rows, bf16_t* dst) {
#pragma unroll
    for (int u = 0; u < RPW; ++u) {
      const int r = RPW * wv + u;
      if (!((fp8_rows >> r) & 1u)) continue;
      const uint8_t* st = s_stage + r * 1024;
      u32x4_t w;
      if (lane < nc) {
        const uint2 c8 = *reinterpret_cast<const uint2*>(st + 8 * lane);
        const float sc = mx_scale_value(st[kAtD + R + (lane >> 2)]);
        w[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c8.x, sc, false));
        w[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c8.x, sc, true));
        w[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c8.y, sc, false));
        w[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c8.y, sc, true));
      } else {
        w = *reinterpret_cast<const u32x4_t*>(st + (kAtD - R) + 16 * (lane - nc));
      }
      *reinterpret_cast<u32x4_t*>(dst + r * kAtD + 8 * (lane ^ hs_swz(r))) = w;
    }
  };

  // ---- prologue: tile 0's rows, the rope table, the split's later indices
  uint32_t vmask, fp8_0 = 0;
  {
    const TileSrc t0 = resolve_tile(start, idx0);
#pragma unroll
    for (int u = 0; u < RPW; ++u) issue_row(t0, u, s_rows0);
    vmask = t0.mask;
    fp8_0 = t0.fp8;
  }
  for (int p = tid; p < R / 2; p += 64 * NW) rope_cos_sin(tpos, p, a.rope_theta1, s_cos[p], s_sin[p]);
  if constexpr (MULTI && CSA) {
    const int sel_end = min(end, a.K);
    for (int jj = start + kHsRows + tid; jj < sel_end; jj += 64 * NW)
      s_idx[jj - start] = a.idx[(int64_t)qi * a.K + jj];
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if constexpr (FP8) convert_rows(fp8_0, s_rows0);
  __syncthreads();

  // rotate the query slice's rope channels at +tpos (each lane its own
  // pairs).  Which 32-channel slices hold rope channels is the same for every
  // lane, so the skip is a uniform branch; inside a slice each pair is
  // rotated or passed through by a select (no per-lane branches)
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) {
    if (32 * ks + 32 <= rope0) continue;
    const int c0 = 32 * ks + 8 * G;
    const u32x4_t w = __builtin_bit_cast(u32x4_t, qb[ks]);
    u32x4_t pk;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c = c0 + 2 * k;
      const int pj = max(c - rope0, 0) >> 1;
      const float cs = s_cos[pj], sn = s_sin[pj];
      const float x0 = __uint_as_float(w[k] << 16), x1 = __uint_as_float(w[k] & 0xffff0000u);
      pk[k] = c >= rope0 ? pack_bf16x2(x0 * cs - x1 * sn, x0 * sn + x1 * cs) : w[k];
    }
    qb[ks] = __builtin_bit_cast(bf16x8_t, pk);
  }

  float mrun = -INFINITY, lrun = 0.f;  // this lane's head (shared by its 4 row groups)
  f32x4_t oacc[32];
#pragma unroll
  for (int cb = 0; cb < 32; ++cb) oacc[cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const float sl2 = a.scale * kLog2e;

  // Logits S^T[key][head] of one tile over all 512 channels for two 16-key
  // blocks (two independent accumulator chains, interleaved).  The order is
  // pinned: with one wave per SIMD nothing else hides the LDS latency, so the
  // 32 operand reads run 8 ahead of their MFMAs (4 at two waves per SIMD).
  // hook(f) runs after MFMA step f: in multi-tile splits it issues the next
  // tile's copies, spread between the reads instead of stalling issue up
  // front.  At two waves per SIMD the lane index is made opaque per tile, so
  // the read addresses are recomputed (a few VALU ops) rather than held in
  // registers across the tile loop.
  constexpr bool kTwoWaves = MULTI && !FP8;
  constexpr int kQkAhead = kTwoWaves ? 4 : 8;
  auto qk = [&](const bf16_t* rows, f32x4_t (&acc)[2], auto&& hook) {
    acc[0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    acc[1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    int ln = lane;
    if constexpr (kTwoWaves) asm volatile("" : "+v"(ln));
    const int lc16 = ln & 15, lG = ln >> 4;
    const bf16_t* rpk[2] = {rows + lc16 * kAtD, rows + (16 + lc16) * kAtD};
    const int swk[2] = {hs_swz(lc16), hs_swz(16 + lc16)};
    // step f reads block f % 2, channel slice f / 2
    auto qk_read = [&](int f) {
      const int kb = f & 1, ks = f >> 1;
      return *reinterpret_cast<const bf16x8_t*>(rpk[kb] + 128 * (ks >> 2) +
                                                8 * ((4 * (ks & 3) + lG) ^ swk[kb]));
    };
    bf16x8_t av[kQkAhead];
#pragma unroll
    for (int f = 0; f < kQkAhead; ++f) av[f] = qk_read(f);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int f = 0; f < 32; ++f) {
      acc[f & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[f % kQkAhead], qb[f >> 1], acc[f & 1], 0, 0, 0);
      if (f + kQkAhead < 32) av[f % kQkAhead] = qk_read(f + kQkAhead);
      hook(f);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Online softmax of head h over a tile's 32 keys (lane (G, c16) holds keys
  // 16kb + 4G + r; the other three row groups hold the rest), branch-free
  // but for the rare rescale.  The reference maximum moves lazily: only when
  // the tile maximum exceeds it by more than 2^8 (log2 units); the first tile
  // with a valid key moves it.  The weights come from v_exp_f32 alone
  // (exp2_weight; arguments at most 8): a masked key (-inf) or a head with
  // no valid key yet (reference -inf) gives 0.  Returns the bf16 PV operand.
  auto softmax = [&](const f32x4_t (&sc)[2], uint32_t vm) -> bf16x8_t {
    const uint32_t vg = vm >> (4 * G);  // bit 16 kb + r: key 16 kb + 4G + r
    float p[2][4];
    float tmx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[kb][r] = ((vg >> (16 * kb + r)) & 1) ? sc[kb][r] * sl2 : -INFINITY;
        tmx = fmaxf(tmx, p[kb][r]);
      }
    tmx = fmaxf(tmx, row_swap16(tmx));
    tmx = fmaxf(tmx, half_swap(tmx));
    const bool move = __ballot(tmx > mrun + 8.f) != 0;
    const float mnew = move ? fmaxf(mrun, tmx) : mrun;
    const bool none = mnew == -INFINITY;
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[kb][r] = exp2_weight(none ? -INFINITY : p[kb][r] - mnew);
        rs += p[kb][r];
      }
    rs += row_swap16(rs);
    rs += half_swap(rs);
    if (__ballot(mnew > mrun)) {
      const float alpha = mnew > mrun ? exp2_weight(mrun - mnew) : 1.f;
      lrun *= alpha;
#pragma unroll
      for (int cb = 0; cb < 32; ++cb) oacc[cb] *= alpha;
      mrun = mnew;
    }
    lrun += rs;
    u32x4_t pk;
    pk.x = pack_bf16x2(p[0][0], p[0][1]);
    pk.y = pack_bf16x2(p[0][2], p[0][3]);
    pk.z = pack_bf16x2(p[1][0], p[1][1]);
    pk.w = pack_bf16x2(p[1][2], p[1][3]);
    return __builtin_bit_cast(bf16x8_t, pk);
  };

  // O^T[ch][head] += R^T[ch][key] P^T[key][head]: in each 16-lane group,
  // lane i points at key row 4G + i/4 (and 16 + 4G + i/4), channels
  // 16cb + 4(i % 4) .. +3, and receives channel 16cb + i of the 4 rows.
  auto pv = [&](const bf16_t* rows, bf16x8_t pb) {
    int ln = lane;
    if constexpr (kTwoWaves) asm volatile("" : "+v"(ln));
    const int lc16 = ln & 15, lG = ln >> 4;
    const int kr0 = 4 * lG + (lc16 >> 2);
    const int kr1 = kr0 + 16;
    const bf16_t* rp0 = rows + kr0 * kAtD;
    const bf16_t* rp1 = rows + kr1 * kAtD;
    const int sw0 = hs_swz(kr0), sw1 = hs_swz(kr1);
    const int q4 = lc16 & 3;
#pragma unroll
    for (int c8 = 0; c8 < 4; ++c8) {
      bf16x8_t av[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int cb = 8 * c8 + k;
        const int ch = 2 * cb + (q4 >> 1);          // 16-byte chunk of the channels
        const int sub = 4 * (q4 & 1);               // bf16 offset inside it
        const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4_ptr)(rp0 + 128 * (ch >> 4) + 8 * ((ch & 15) ^ sw0) + sub));
        const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4_ptr)(rp1 + 128 * (ch >> 4) + 8 * ((ch & 15) ^ sw1) + sub));
        const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
        av[k] = __builtin_bit_cast(bf16x8_t, u32x4_t{l2.x, l2.y, h2.x, h2.y});
      }
#pragma unroll
      for (int k = 0; k < 8; ++k)
        oacc[8 * c8 + k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[k], pb, oacc[8 * c8 + k], 0, 0, 0);
    }
    // kPvAhead transposing reads (two per channel block) ahead, then one
    // MFMA per two
    constexpr int kPvAhead = kTwoWaves ? 4 : 16;
    __builtin_amdgcn_sched_group_barrier(0x100, kPvAhead, 1);
#pragma unroll
    for (int i = 0; i < 32 - kPvAhead / 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kPvAhead / 2, 1);
  };

  // the copies of the tile at row j0 into `dst`, one row per (32 / RPW) QK
  // steps; past the split's end every row is invalid and the copy reads the
  // harmless row into the idle buffer, so the request is unconditional
  auto next_tile = [&](int j0) -> TileSrc {
    int sidx_l = 0;
    // row j0 + l's selected index; entries past the selected part (or the
    // split) are never used, the clamp only keeps the read inside s_idx
    if constexpr (MULTI && CSA) sidx_l = s_idx[min(j0 - start + (lane & 31), kHsMaxSplitRows - 1)];
    return resolve_tile(j0, sidx_l);
  };

  if constexpr (!MULTI) {
    // a single tile: logits, softmax, PV
    if (start < end) {
      f32x4_t sc[2];
      qk(s_rows0, sc, [](int) {});
      pv(s_rows0, softmax(sc, vmask));
    }
  } else {
    // multi-tile splits: the next tile's rows are copied into the other
    // buffer while this one is used; one barrier per tile
    auto tile = [&](int j0, const bf16_t* rows, bf16_t* next) {
      const TileSrc nt = next_tile(j0 + kHsRows);
      f32x4_t sc[2];
      qk(rows, sc, [&](int f) {
        if (f % (32 / RPW) == 32 / RPW - 1) issue_row(nt, f / (32 / RPW), next);
      });
      pv(rows, softmax(sc, vmask));
      // the next tile's rows have landed and every wave is done with this one
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      if constexpr (FP8) convert_rows(nt.fp8, next);
      __syncthreads();
      vmask = nt.mask;
    };
    for (int j0 = start; j0 < end; j0 += 2 * kHsRows) {
      tile(j0, s_rows0, s_rows1);
      if (j0 + kHsRows >= end) break;
      tile(j0 + kHsRows, s_rows1, s_rows0);
    }
  }

  // ---- epilogue: lane (G, c16) holds channels 16cb + 4G + r of head h
  // rotate_back: channels c .. c + 3 (block cb) rotated by -tpos where they
  // are rope channels.  In the straight-line single-tile kernels the block
  // test is uniform and each pair is rotated or passed through by a select
  // (per-lane branches there cost hundreds of exec-mask moves: the 64K decode
  // kernel shrank from 6,110 to 5,194 instructions).  The multi-tile kernels
  // keep per-lane branches: with the selects their tile loop no longer fit
  // its registers.
  auto rotate_back = [&](float (&o)[4], int c, int cb) {
    if constexpr (MULTI) {
      if (c + 4 > rope0) {
#pragma unroll
        for (int e = 0; e < 4; e += 2) {
          if (c + e >= rope0) {
            const int pj = (c + e - rope0) >> 1;
            const float cs = s_cos[pj], sn = s_sin[pj];
            const float x0 = o[e], x1 = o[e + 1];
            o[e] = x0 * cs + x1 * sn;
            o[e + 1] = -x0 * sn + x1 * cs;
          }
        }
      }
    } else {
      if (16 * cb + 16 > rope0) {
#pragma unroll
        for (int e = 0; e < 4; e += 2) {
          const bool rot = c + e >= rope0;
          const int pj = max(c + e - rope0, 0) >> 1;
          const float cs = s_cos[pj], sn = s_sin[pj];
          const float x0 = o[e], x1 = o[e + 1];
          o[e] = rot ? x0 * cs + x1 * sn : x0;
          o[e + 1] = rot ? -x0 * sn + x1 * cs : x1;
        }
      }
    }
  };
  if (S == 1) {
    const float skl2 = a.sink[h] * kLog2e;
    const float mf = fmaxf(mrun, skl2);
    const float lf = lrun * exp2f(mrun - mf) + exp2f(skl2 - mf);
    const float fac = exp2f(mrun - mf) / lf;
    if (G == 0 && a.lse) a.lse[(int64_t)qi * a.H + h] = (mf + log2f(lf)) * kLn2;
    bf16_t* op = (bf16_t*)a.out + ((int64_t)qi * a.H + h) * kAtD;
#pragma unroll
    for (int cb = 0; cb < 32; ++cb) {
      float o[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) o[r] = oacc[cb][r] * fac;
      const int c = 16 * cb + 4 * G;
      rotate_back(o, c, cb);
      uint2 pk;
      pk.x = pack_bf16x2(o[0], o[1]);
      pk.y = pack_bf16x2(o[2], o[3]);
      *reinterpret_cast<uint2*>(op + c) = pk;
    }
  } else {
    const int64_t slot = ((int64_t)qi * S + sp) * a.H + h;
    if (G == 0) {
      a.part_ml[2 * slot] = mrun;
      a.part_ml[2 * slot + 1] = lrun;
    }
    // the output's rope slice is rotated back by -tpos here (the rotation is
    // linear, so the merge of the splits commutes with it); the split
    // outputs are stored in bf16, halving the bytes this epilogue writes and
    // the merge reads (each is unnormalised against its own maximum, so the
    // rounding is relative to the values themselves)
    bf16_t* po = a.part_o + slot * kAtD;
#pragma unroll
    for (int cb = 0; cb < 32; ++cb) {
      float o[4] = {oacc[cb][0], oacc[cb][1], oacc[cb][2], oacc[cb][3]};
      const int c = 16 * cb + 4 * G;
      rotate_back(o, c, cb);
      uint2 pk;
      pk.x = pack_bf16x2(o[0], o[1]);
      pk.y = pack_bf16x2(o[2], o[3]);
      *reinterpret_cast<uint2*>(po + c) = pk;
    }
  }
}

// Merge of the key-range splits: partial maxima are in log2 units of the
// scaled logits, partial sums and outputs unnormalised (outputs in bf16,
// already rotated back by -tpos on their rope slice).  grid (B*Tq, H),
// 128 threads of 4 channels each (the 512-wide Flash rows).  The partial
// outputs of the first kCbPre splits are requested before the per-split
// weights are known, so the two dependent reads overlap; the weights go
// through LDS.  32 covers the decode grids (20 splits at 64K: 12.6 ->
// 12.4 us per call against 16, whose last 4 splits waited for the weights).
constexpr int kMaxSplits = 256;
constexpr int kCbPre = 32;

template <typename T>
__global__ __launch_bounds__(128) void attn_combine(AttnArgs a) {
  __shared__ float s_w[kMaxSplits];
  __shared__ float s_lse;
  const int qi = blockIdx.x, h = blockIdx.y;
  const int S = a.splits;
  const int64_t slot0 = (int64_t)qi * S * a.H + h;
  const int c = threadIdx.x * 4;
  const bf16_t* po = a.part_o + slot0 * kAtD + c;
  const int64_t sstride = (int64_t)a.H * kAtD;
  // four bf16 split-output channels to f32
  auto widen = [](uint2 w) {
    return f32x4_t{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                   __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u)};
  };
  uint2 v[kCbPre];
#pragma unroll
  for (int u = 0; u < kCbPre; ++u)
    v[u] = u < S ? *reinterpret_cast<const uint2*>(po + u * sstride) : uint2{0u, 0u};
  if (threadIdx.x < 64) {  // one wave merges the (max, sum) pairs
    // lane l holds the pairs of splits l, l + 64, ... in registers: one
    // round of loads (a second pass over them in memory was a second,
    // dependent round trip)
    const int lane = threadIdx.x;
    const float skl2 = a.sink[h] * kLog2e;
    constexpr int kPer = kMaxSplits / 64;
    float2 ml[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int s = lane + 64 * k;
      ml[k] = s < S ? *reinterpret_cast<const float2*>(a.part_ml + 2 * (slot0 + (int64_t)s * a.H))
                    : make_float2(-INFINITY, 0.f);
    }
    float M = skl2;
#pragma unroll
    for (int k = 0; k < kPer; ++k) M = fmaxf(M, ml[k].x);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    float Ls = 0.f, w[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      w[k] = exp2f(ml[k].x - M);  // 0 for an absent split (max -inf)
      Ls += ml[k].y * w[k];
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) Ls += __shfl_xor(Ls, off);
    Ls += exp2f(skl2 - M);
    const float inv = 1.f / Ls;
#pragma unroll
    for (int k = 0; k < kPer; ++k)
      if (lane + 64 * k < S) s_w[lane + 64 * k] = w[k] * inv;
    if (lane == 0) s_lse = (M + log2f(Ls)) * kLn2;
  }
  __syncthreads();
  if (threadIdx.x == 0 && a.lse) a.lse[(int64_t)qi * a.H + h] = s_lse;
  f32x4_t o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < kCbPre; ++u)
    if (u < S) o += s_w[u] * widen(v[u]);
  for (int s = kCbPre; s < S; s += 8) {
    uint2 w8[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      w8[u] = s + u < S ? *reinterpret_cast<const uint2*>(po + (s + u) * sstride) : uint2{0u, 0u};
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (s + u < S) o += s_w[s + u] * widen(w8[u]);
  }
  float r[4] = {o[0], o[1], o[2], o[3]};
  T* op = (T*)a.out + ((int64_t)qi * a.H + h) * kAtD + c;
#pragma unroll
  for (int e = 0; e < 4; ++e) Elem<T>::put(op + e, r[e]);
}

// ------------------------------------------------------------------- launch
bool attn_uses_mfma(int dt, int H, int D, int R) {
  return dt == 1 && H % kAtH == 0 && H <= kMaxAtH && D == kAtD && R % 2 == 0 && R <= D;
}

int attn_splits(int dt, int B, int Tq, int H, int D, int keys_per_query) {
  if (!(dt == 1 && H % kAtH == 0 && H <= kMaxAtH && D == kAtD)) return 1;
  // a query of H heads is H / 64 workgroups per split
  const int64_t q = (int64_t)B * Tq * (H / kAtH);
  const int tiles = (keys_per_query + kHsRows - 1) / kHsRows;
  // few queries: spread each one's tiles over splits until there are about
  // as many workgroups as compute units (one tile per split at most)
  int s = 1;
  if (q < 256 && tiles >= 2) s = min((int)((256 + q - 1) / q), tiles);
  // a multi-tile split holds at most kHsMaxSplitRows rows (its CSA index
  // stage lives in LDS)
  s = max(s, (keys_per_query + kHsMaxSplitRows - 1) / kHsMaxSplitRows);
  return min(s, kMaxSplits);
}

// every multi-tile CSA split stages its indices in LDS: at most kMaxSplits
// splits of kHsMaxSplitRows rows each
int64_t attn_max_csa_keys() { return (int64_t)kMaxSplits * kHsMaxSplitRows; }

size_t attn_ws_bytes(int dt, int B, int Tq, int H, int D, int keys_per_query) {
  const int s = attn_splits(dt, B, Tq, H, D, keys_per_query);
  if (s <= 1) return 0;
  // (max, sum) pairs in f32, then the split outputs in bf16
  return (size_t)B * Tq * s * H * (2 * sizeof(float) + (size_t)D * sizeof(bf16_t));
}

// Decode steps with a new row (bf16, the Flash shape, one query per
// sequence): the key list's splits plus one for the new row while the grid
// still fits the compute units once (the window-only decode: 4 + 1 splits
// of 16 queries); past that, as many splits as without it, the last one
// given to the new row, so the grid keeps its one workgroup per compute
// unit (one split more per query, 272 workgroups for the 1M-token HCA step
// at batch 16, put two on some compute units: 59 us against 48).
int attn_fresh_splits(int B, int H, int D, int keys_per_query) {
  const int s = attn_splits(1, B, 1, H, D, keys_per_query);
  if ((int64_t)B * (H / kAtH) * (s + 1) <= 256) return min(s + 1, kMaxSplits);
  return max(2, s);
}

size_t attn_fresh_ws_bytes(int B, int H, int D, int keys_per_query) {
  const int s = attn_fresh_splits(B, H, D, keys_per_query);
  return (size_t)B * s * H * (2 * sizeof(float) + (size_t)D * sizeof(bf16_t));
}

template <typename T>
static hipError_t launch_generic(const AttnArgs& a, hipStream_t stream) {
  dim3 grid((a.H + 3) / 4, a.B * a.Tq), block(256);
  const int np = (a.D + 127) / 128;
  if (np <= 1) hipLaunchKernelGGL((attn_generic<T, 1>), grid, block, 0, stream, a);
  else if (np <= 2) hipLaunchKernelGGL((attn_generic<T, 2>), grid, block, 0, stream, a);
  else if (np <= 4) hipLaunchKernelGGL((attn_generic<T, 4>), grid, block, 0, stream, a);
  else hipLaunchKernelGGL((attn_generic<T, 8>), grid, block, 0, stream, a);
  return hipGetLastError();
}

// The single-tile kernels run their code once, straight through, so their
// size is part of their time: for the Flash and Pro rope width (64 channels)
// an instance with it fixed at compile time drops every rope test on the
// other 448 channels (the query rotation, the epilogue).
constexpr int kRopeFixed = 64;

template <bool FP8, int RC>
static void launch_hs_single(const AttnArgs& a, bool halves, dim3 grid, dim3 grid2,
                             hipStream_t stream) {
  const dim3 block4(256), block2(128);
  if (a.csa && !a.fresh) {
    if (halves) hipLaunchKernelGGL((attn_hs<true, false, 2, FP8, RC>), grid2, block2, 0, stream, a);
    else hipLaunchKernelGGL((attn_hs<true, false, 4, FP8, RC>), grid, block4, 0, stream, a);
  } else {
    if (halves) hipLaunchKernelGGL((attn_hs<false, false, 2, FP8, RC>), grid2, block2, 0, stream, a);
    else hipLaunchKernelGGL((attn_hs<false, false, 4, FP8, RC>), grid, block4, 0, stream, a);
  }
}

template <bool FP8>
static void launch_hs(const AttnArgs& a, bool multi, bool halves, dim3 grid, dim3 grid2,
                      hipStream_t stream) {
  if (multi) {
    const dim3 block4(256);
    if (a.csa && !a.fresh) hipLaunchKernelGGL((attn_hs<true, true, 4, FP8>), grid, block4, 0, stream, a);
    else hipLaunchKernelGGL((attn_hs<false, true, 4, FP8>), grid, block4, 0, stream, a);
  } else if (a.R == kRopeFixed) {
    launch_hs_single<FP8, kRopeFixed>(a, halves, grid, grid2, stream);
  } else {
    launch_hs_single<FP8, 0>(a, halves, grid, grid2, stream);
  }
}

// A step with a new row runs the kernels without selected indices (the ones
// with the new-row split); the window-only step sets csa with K = 0, so that
// their key list is the window alone.
hipError_t launch_attn(const AttnArgs& a, hipStream_t stream) {
  if (a.B * a.Tq == 0) return hipSuccess;
  if (attn_uses_mfma(a.dt, a.H, a.D, a.R)) {
    const int hg = a.H / kAtH;  // 64-head groups (grid z)
    dim3 grid(a.splits, a.B * a.Tq, hg);
    // most rows a split can hold: the list length bound over the split count
    const int wc = (a.W > 0 && a.L_win > 0) ? min(a.W, a.L_win) : 0;
    const int64_t lmax = (a.csa ? (int64_t)a.K : (int64_t)a.N_cap) + wc;
    const int sa = a.splits - (a.fresh ? 1 : 0);  // splits over the key list
    const bool multi = (lmax + sa - 1) / sa > kHsRows;
    // single-tile splits in head groups of 32 (two waves, grid z) while the
    // doubled grid still fits the compute units once
    const bool halves = !multi && 2LL * hg * a.splits * a.B * a.Tq <= kHsHeadSplitBelow;
    dim3 grid2(a.splits, a.B * a.Tq, 2 * hg);
    if (a.pool_row_bytes > 0)
      launch_hs<true>(a, multi, halves, grid, grid2, stream);
    else
      launch_hs<false>(a, multi, halves, grid, grid2, stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.splits == 1) return e;
    hipLaunchKernelGGL(attn_combine<bf16_t>, dim3(a.B * a.Tq, a.H), dim3(128), 0, stream, a);
    return hipGetLastError();
  }
  if (a.dt == 1) return launch_generic<bf16_t>(a, stream);
  return launch_generic<float>(a, stream);
}

}  // namespace csa
