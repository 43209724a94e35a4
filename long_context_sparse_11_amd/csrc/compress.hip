// Token-level compressor: softmax-weighted pooling of m-token blocks (two
// overlapped streams for CSA, one stream for HCA), then optional RMSNorm and
// partial RoPE.  "DeepSeek-v4 Beyond Basics" section 3.2.2 (eqs. 9-12) and
// section 3.3 (eqs. 20-23); RMSNorm/RoPE placement from the same page's
// section 3.3 (its quote of the paper's section 2.3.3).
//
// One workgroup per (sequence, entry, channel slice).  A slice of Ds
// channels is covered by L = Ds / VEC lanes holding VEC contiguous channels
// each (16-byte loads, so a row slice is one coalesced read).  The block's
// rows are spread over G lane groups; each group keeps a per-channel online
// softmax (max, denominator, weighted sum) in registers, the groups are
// merged through LDS, and group 0 finishes the entry (normalise, gain,
// rotate, store).  A call with few entries splits each entry's channels over
// several workgroups, so that more compute units stream its rows (one
// workgroup alone pulls its rows at a small fraction of the chip's rate);
// the pooling is per channel, and only the RMSNorm needs the whole row: with
// a gain, the slices leave their pooled values in a workspace and
// compress_finish normalises, rotates and stores.
#include "kernels.h"

namespace csa {

// At most 512 threads: a thread keeps 4 rows' loads in flight, which needs
// more registers than a 1024-thread bound leaves.
template <typename T, int VEC>
__global__ __launch_bounds__(512) void compress_kernel(CompressArgs a0, CompressArgs a1) {
  extern __shared__ float smem[];  // [3][G/2][Ds] merge staging
  // a launch carries one or two jobs (compressors over the same token
  // block, say the KV entry and the indexer key): z = job * slices + slice
  const int job = (int)blockIdx.z / a0.slices;
  const int slice = (int)blockIdx.z - job * a0.slices;
  const CompressArgs a = job ? a1 : a0;
  const int i = blockIdx.x;  // entry within the call
  const int b = blockIdx.y;
  const int D = a.D;
  const int Ds = D / a.slices;  // channels of this workgroup
  const int L = Ds / VEC;
  const int G = blockDim.x / L;
  const int tid = threadIdx.x;
  const int g = tid / L;
  const int lane = tid - g * L;
  const int cl = lane * VEC;                // channel within the slice
  const int c0 = slice * Ds + cl;           // channel within the row
  const int m = a.m;

  const int64_t pos = a.pos0 ? a.pos0[b] + (int64_t)m * i : 0;  // requested early (rope)
  const int64_t a_row0 = (int64_t)m * i;
  const int na = (int)min((int64_t)m, (int64_t)a.T - a_row0);
  const T* cb_base = nullptr;
  const T* zb_base = nullptr;
  int nb = 0;
  if (a.overlap) {
    if (i >= 1) {
      nb = m;
      const int64_t off = ((int64_t)b * a.T + (int64_t)m * (i - 1)) * D;
      cb_base = (const T*)a.c_b + off;
      zb_base = (const T*)a.z_b + off;
    } else if (a.prev_c_b && !(a.pos0 && pos < m)) {  // block 0 has no block before it
      nb = m;
      const int64_t off = (int64_t)b * m * D;
      cb_base = (const T*)a.prev_c_b + off;
      zb_base = (const T*)a.prev_z_b + off;
    }
  }
  const int nr = na + nb;

  float mx[VEC], den[VEC], acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) { mx[e] = -INFINITY; den[e] = 0.f; acc[e] = 0.f; }

  const int64_t a_off = ((int64_t)b * a.T + a_row0) * D;
  // rows g, g+G, ... in batches of 4.  Every load of a batch is issued before
  // any arithmetic: a row past the block reads a valid row (its own group's
  // first) and is skipped afterwards, and the optional z / bias loads go
  // into zero-initialised registers, so no load is waited on before the
  // batch's last one is in flight.
  constexpr int NW = VEC * (int)sizeof(T) / 16;  // 16-byte words per lane per row
  // the optional streams' words are initialised once (a skipped load then
  // leaves a defined value that a select discards), never inside the loop,
  // where a fresh write could be made to wait for an older load
  u32x4_t cw[4][NW], zw[4][NW], bw[4][VEC / 4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
#pragma unroll
    for (int k = 0; k < NW; ++k) zw[u][k] = u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < VEC / 4; ++k) bw[u][k] = u32x4_t{0u, 0u, 0u, 0u};
  }
  for (int r0 = g; r0 < nr; r0 += 4 * G) {
    bool hz[4], hb[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = r0 + u * G;
      const int rr = r < nr ? r : r0;
      const bool in_a = rr < na;
      const int64_t rb = rr - na;
      const T* cp = in_a ? (const T*)a.c_a + a_off + (int64_t)rr * D + c0 : cb_base + rb * D + c0;
      const T* zb = in_a ? (const T*)a.z_a : zb_base;
      const T* zp = in_a ? (const T*)a.z_a + a_off + (int64_t)rr * D + c0 : zb_base + rb * D + c0;
      const float* bb = in_a ? a.bias_a : a.bias_b;
      const float* bp = bb + (int64_t)(in_a ? rr : (int)rb) * D + c0;
      hz[u] = zb != nullptr;
      hb[u] = bb != nullptr;
      Elem<T>::template load_raw<VEC>(cp, cw[u]);
      if (hz[u]) Elem<T>::template load_raw<VEC>(zp, zw[u]);
      if (hb[u]) Elem<float>::template load_raw<VEC>(bp, bw[u]);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (r0 + u * G >= nr) continue;
      float cv[VEC], zv[VEC], bv[VEC];
      Elem<T>::template from_raw<VEC>(cw[u], cv);
      Elem<T>::template from_raw<VEC>(zw[u], zv);
      Elem<float>::template from_raw<VEC>(bw[u], bv);
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float l = ((hz[u] ? zv[e] : 0.f) + (hb[u] ? bv[e] : 0.f)) * kLog2e;  // base 2
        const float nm = fmaxf(mx[e], l);
        const float sc = exp2_weight(mx[e] - nm);
        const float p = exp2_weight(l - nm);
        den[e] = den[e] * sc + p;
        acc[e] = acc[e] * sc + p * cv[e];
        mx[e] = nm;
      }
    }
  }

  // merge the G groups pairwise through LDS (log2 G steps, all groups busy):
  // the upper half of the live groups posts its partials, the lower half
  // folds them in.  LDS layout [3][G/2][D].
  float gv[VEC];
  if (g == 0 && a.gain) Elem<float>::template load<VEC>(a.gain + c0, gv);  // in flight meanwhile
  float* s_mx = smem;
  float* s_den = smem + (G / 2) * Ds;
  float* s_acc = smem + 2 * (G / 2) * Ds;
  for (int half = G >> 1; half >= 1; half >>= 1) {
    if (g >= half && g < 2 * half) {
      const int o = (g - half) * Ds + cl;
#pragma unroll
      for (int e = 0; e < VEC; ++e) { s_mx[o + e] = mx[e]; s_den[o + e] = den[e]; s_acc[o + e] = acc[e]; }
    }
    __syncthreads();
    if (g < half) {
      const int o = g * Ds + cl;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float om = s_mx[o + e];
        const float M = fmaxf(mx[e], om);
        const float w0 = mx[e] == -INFINITY ? 0.f : exp2_weight(mx[e] - M);
        const float w1 = om == -INFINITY ? 0.f : exp2_weight(om - M);
        den[e] = den[e] * w0 + s_den[o + e] * w1;
        acc[e] = acc[e] * w0 + s_acc[o + e] * w1;
        mx[e] = M;
      }
    }
    __syncthreads();
  }
  if (g != 0) return;
  float y[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) y[e] = acc[e] / den[e];

  if (a.slices > 1 && a.gain) {  // the norm needs the whole row: compress_finish
    Elem<float>::template store<VEC>(a.ws_y + ((int64_t)b * a.n_out + i) * D + c0, y);
    return;
  }
  if (a.gain) {
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) ss += y[e] * y[e];
    if (L == 64) {
      ss = wave_sum(ss);
    } else {
      for (int off = L >> 1; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
    }
    const float inv = 1.0f / sqrtf(ss / (float)D + a.eps);
#pragma unroll
    for (int e = 0; e < VEC; ++e) y[e] = y[e] * inv * gv[e];
  }

  const int R = a.rope_dims;
  if (R > 0 && c0 + VEC > D - R) {
#pragma unroll
    for (int e = 0; e < VEC; e += 2) {
      const int c = c0 + e;
      if (c >= D - R) {
        float cs, sn;
        rope_cos_sin(pos, (c - (D - R)) >> 1, a.rope_theta1, cs, sn);
        const float x0 = y[e], x1 = y[e + 1];
        y[e] = x0 * cs - x1 * sn;
        y[e + 1] = x0 * sn + x1 * cs;
      }
    }
  }

  const int64_t ent = compress_out_row(a, b, i);
  if (ent < 0) return;
  if constexpr (VEC == 8) {
    if (a.out_fp8_row > 0) {  // packed mixed BF16 / FP8 row (D = 512: one wave)
      const int64_t bs = a.out_bstride ? a.out_bstride : (int64_t)a.n_out * a.out_fp8_row;
      store_kv_fp8_row((uint8_t*)a.out + (int64_t)b * bs + ent * a.out_fp8_row, lane, y, R);
      return;
    }
  }
  const int64_t bstride = a.out_bstride ? a.out_bstride : (int64_t)a.n_out * D;
  T* op = (T*)a.out + (int64_t)b * bstride + ent * D + c0;
  Elem<T>::template store<VEC>(op, y);
}

// RMSNorm, gain and RoPE of entries whose channel slices were pooled by
// separate workgroups.  grid (n_out, B), one wave; lane l holds channels
// VEC l .. VEC l + VEC - 1 (D = 64 VEC).
template <typename T, int VEC>
__global__ __launch_bounds__(64) void compress_finish(CompressArgs a) {
  const int i = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  const int D = a.D, c0 = lane * VEC;
  const int64_t pos = a.pos0 ? a.pos0[b] + (int64_t)a.m * i : 0;
  float y[VEC], gv[VEC];
  Elem<float>::template load<VEC>(a.ws_y + ((int64_t)b * a.n_out + i) * D + c0, y);
  Elem<float>::template load<VEC>(a.gain + c0, gv);
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < VEC; ++e) ss += y[e] * y[e];
  ss = wave_sum(ss);
  const float inv = 1.0f / sqrtf(ss / (float)D + a.eps);
#pragma unroll
  for (int e = 0; e < VEC; ++e) y[e] = y[e] * inv * gv[e];
  const int R = a.rope_dims;
  if (R > 0 && c0 + VEC > D - R) {
#pragma unroll
    for (int e = 0; e < VEC; e += 2) {
      const int c = c0 + e;
      if (c >= D - R) {
        float cs, sn;
        rope_cos_sin(pos, (c - (D - R)) >> 1, a.rope_theta1, cs, sn);
        const float x0 = y[e], x1 = y[e + 1];
        y[e] = x0 * cs - x1 * sn;
        y[e + 1] = x0 * sn + x1 * cs;
      }
    }
  }
  const int64_t ent = compress_out_row(a, b, i);
  if (ent < 0) return;
  if constexpr (VEC == 8) {
    if (a.out_fp8_row > 0) {  // packed mixed BF16 / FP8 row (D = 512)
      const int64_t bs = a.out_bstride ? a.out_bstride : (int64_t)a.n_out * a.out_fp8_row;
      store_kv_fp8_row((uint8_t*)a.out + (int64_t)b * bs + ent * a.out_fp8_row, lane, y, R);
      return;
    }
  }
  const int64_t bstride = a.out_bstride ? a.out_bstride : (int64_t)a.n_out * D;
  Elem<T>::template store<VEC>((T*)a.out + (int64_t)b * bstride + ent * D + c0, y);
}

// ------------------------------------------------------ short-block streaming
// Many entries of short blocks (CSA m = 4 with its overlap, window rows
// m = 1): a sub-group of L = D / VEC lanes owns one entry, lane l of it
// channels VEC l .. VEC l + VEC - 1, and holds all of the entry's rows for
// them, so the per-channel softmax, the weighted sum, the RMSNorm (a
// sub-group sum), the gain and RoPE need no LDS merge and no barrier.  A
// wave takes 64 / L entries at once and strides over the call's entries.
// The block shape (M rows per stream, the overlap) is a template argument,
// so every row address is a branch-free select and all 2M (or M) row loads
// of an entry are issued back to back before any arithmetic (16 KiB in
// flight per wave for a 512-channel CSA entry).  Each row is read once, so
// the loads stream past the caches (non-temporal: the 1M-token pass 1141 ->
// 1117 us).  The biases sit in LDS in base-2 logit units; the lane's gain
// and RoPE frequencies are loaded once.
constexpr int kRowsMaxD = 512;   // widest row the kernel's bias table holds

template <typename T, int VEC, int M, bool OVERLAP>
__global__ __launch_bounds__(256) void compress_rows_kernel(CompressArgs a0, CompressArgs a1) {
  constexpr int ROWS = M * (OVERLAP ? 2 : 1);
  __shared__ __attribute__((aligned(16))) float s_bias[ROWS * kRowsMaxD];
  const CompressArgs a = blockIdx.y ? a1 : a0;
  const int D = a.D;
  const int L = D / VEC;                // lanes per entry (a power of two <= 64)
  const int lane = threadIdx.x & 63;
  const int sub = lane / L, l = lane - sub * L;
  const int per_wave = 64 / L;
  const int c0 = l * VEC;
  constexpr int NW = VEC * (int)sizeof(T) / 16;  // 16-byte words per lane per row
  for (int x = threadIdx.x; x < ROWS * D; x += blockDim.x) {
    const int r = x / D, c = x - r * D;
    const bool in_a = r < M;
    const float* bp = in_a ? a.bias_a : a.bias_b;
    s_bias[x] = bp ? bp[(int64_t)(in_a ? r : r - M) * D + c] * kLog2e : 0.f;
  }
  __syncthreads();
  float gv[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) gv[e] = a.gain ? a.gain[c0 + e] : 1.f;
  const int R = a.rope_dims;
  const bool rot = R > 0 && c0 + VEC > D - R;
  double theta[VEC / 2];
#pragma unroll
  for (int k = 0; k < VEC / 2; ++k) {
    const int c = c0 + 2 * k;
    theta[k] = (rot && c >= D - R) ? rope_theta(a.rope_theta1, (c - (D - R)) >> 1) : 0.0;
  }
  const bool has_z = a.z_a != nullptr;
  const T* za_base = has_z ? (const T*)a.z_a : (const T*)a.c_a;  // read and ignored without z

  const int64_t entries = (int64_t)a.B * a.n_out;
  const int64_t wave0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / 64;
  const int64_t nwaves = (int64_t)gridDim.x * blockDim.x / 64;
  for (int64_t e0 = wave0 * per_wave; e0 < entries; e0 += nwaves * per_wave) {
    const int64_t ent = e0 + sub;
    const bool live = ent < entries;
    const int64_t ec = live ? ent : entries - 1;     // a dead lane reads a live entry's rows
    const int b = (int)(ec / a.n_out);
    const int i = (int)(ec - (int64_t)b * a.n_out);
    const int64_t a_row0 = (int64_t)M * i;
    const int na = (int)min((int64_t)M, (int64_t)a.T - a_row0);
    // the sequence's first position, requested before the rows: waiting for
    // it (the b-stream choice of entry 0) then leaves the rows in flight
    const int64_t p0 = a.pos0 ? a.pos0[b] : 0;
    // stream a: rows a_row0 + r, clamped into the block (a partial last block
    // re-reads its last row; masked below)
    const int64_t a_off = ((int64_t)b * a.T + a_row0) * D + c0;
    u32x4_t cw[ROWS][NW], zw[ROWS][NW];
#pragma unroll
    for (int r = 0; r < M; ++r) {
      const int64_t ro = a_off + (int64_t)min(r, na - 1) * D;
      Elem<T>::template load_raw_stream<VEC>((const T*)a.c_a + ro, cw[r]);
      Elem<T>::template load_raw_stream<VEC>(za_base + ro, zw[r]);
    }
    int nb = 0;
    if constexpr (OVERLAP) {
      // stream b: block i - 1, or for entry 0 the block before the call
      // (given, and not at the sequence start); otherwise no b rows
      const bool use_prev = i == 0 && a.prev_c_b && (!a.pos0 || p0 >= M);
      nb = (i >= 1 || use_prev) ? M : 0;
      const T* cb = i >= 1 ? (const T*)a.c_b + ((int64_t)b * a.T + a_row0 - M) * D
                           : (use_prev ? (const T*)a.prev_c_b + (int64_t)b * M * D
                                       : (const T*)a.c_a + ((int64_t)b * a.T + a_row0) * D);
      const T* zb = i >= 1 ? (const T*)a.z_b + ((int64_t)b * a.T + a_row0 - M) * D
                           : (use_prev ? (const T*)a.prev_z_b + (int64_t)b * M * D
                                       : za_base + ((int64_t)b * a.T + a_row0) * D);
#pragma unroll
      for (int r = 0; r < M; ++r) {
        Elem<T>::template load_raw_stream<VEC>(cb + (int64_t)r * D + c0, cw[M + r]);
        Elem<T>::template load_raw_stream<VEC>(zb + (int64_t)r * D + c0, zw[M + r]);
      }
    }
    const int64_t pos = p0 + a_row0;
    // base-2 logit of row slot r, channel e; -inf for a row the block lacks
    auto logit = [&](int r, int e, const float* zv) {
      const bool ok = r < M ? r < na : r - M < nb;
      return ok ? (has_z ? zv[e] * kLog2e : 0.f) + s_bias[r * D + c0 + e] : -INFINITY;
    };
    // online softmax over the row slots in order (slot 0, the block's first
    // row, always exists, so the running maximum starts finite); each row's
    // raw words are converted only when its turn comes
    float mx[VEC], den[VEC], acc[VEC];
    {
      float zv[VEC], cv[VEC];
      Elem<T>::template from_raw<VEC>(zw[0], zv);
      Elem<T>::template from_raw<VEC>(cw[0], cv);
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        mx[e] = logit(0, e, zv);
        den[e] = 1.f;
        acc[e] = cv[e];
      }
    }
#pragma unroll
    for (int r = 1; r < ROWS; ++r) {
      float zv[VEC], cv[VEC];
      Elem<T>::template from_raw<VEC>(zw[r], zv);
      Elem<T>::template from_raw<VEC>(cw[r], cv);
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float lg = logit(r, e, zv);          // -inf for a missing row
        const float mn = fmaxf(mx[e], lg);
        const float sc = exp2_weight(mx[e] - mn);
        const float p = exp2_weight(lg - mn);
        den[e] = den[e] * sc + p;
        acc[e] = acc[e] * sc + p * cv[e];
        mx[e] = mn;
      }
    }
    float y[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) y[e] = acc[e] / den[e];
    if (a.gain) {
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < VEC; ++e) ss += y[e] * y[e];
      for (int off = L >> 1; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
      const float inv = 1.0f / sqrtf(ss / (float)D + a.eps);
#pragma unroll
      for (int e = 0; e < VEC; ++e) y[e] = y[e] * inv * gv[e];
    }
    if (rot) {
#pragma unroll
      for (int k = 0; k < VEC / 2; ++k) {
        if (c0 + 2 * k < D - R) continue;
        float cs, sn;
        rope_cos_sin_theta(pos, theta[k], cs, sn);
        const float x0 = y[2 * k], x1 = y[2 * k + 1];
        y[2 * k] = x0 * cs - x1 * sn;
        y[2 * k + 1] = x0 * sn + x1 * cs;
      }
    }
    const int64_t row = live ? compress_out_row(a, b, i) : -1;
    if constexpr (VEC == 8) {
      if (a.out_fp8_row > 0) {  // packed mixed BF16 / FP8 row (D = 512: the whole wave)
        if (row >= 0) {
          const int64_t bs = a.out_bstride ? a.out_bstride : (int64_t)a.n_out * a.out_fp8_row;
          store_kv_fp8_row((uint8_t*)a.out + (int64_t)b * bs + row * a.out_fp8_row, lane, y, R);
        }
        continue;
      }
    }
    if (row >= 0) {
      const int64_t bstride = a.out_bstride ? a.out_bstride : (int64_t)a.n_out * D;
      Elem<T>::template store<VEC>((T*)a.out + (int64_t)b * bstride + row * D + c0, y);
    }
  }
}

// ------------------------------------------------------------ decode state
__global__ __launch_bounds__(256) void decode_advance(int B, int m, int N_cap, int64_t* q_pos,
                                                      int32_t* n_entries, int64_t* block_pos0) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b >= B) return;
  const int64_t t = q_pos[b] + 1;
  q_pos[b] = t;
  const int64_t n = (t + 1) / m;
  n_entries[b] = (int32_t)min(n, (int64_t)N_cap);
  block_pos0[b] = ((t + 1) % m == 0) ? t + 1 - m : -1;
}

hipError_t launch_decode_advance(int B, int m, int N_cap, int64_t* q_pos, int32_t* n_entries,
                                 int64_t* block_pos0, hipStream_t stream) {
  hipLaunchKernelGGL(decode_advance, dim3((B + 255) / 256), dim3(256), 0, stream, B, m, N_cap,
                     q_pos, n_entries, block_pos0);
  return hipGetLastError();
}

// Calls with fewer entries than this split each entry's channels, when an
// entry pools at least kCompressSplitRows rows (shorter blocks are a latency
// matter that a second kernel would only lengthen).
constexpr int64_t kCompressSplitBelow = 128;
constexpr int kCompressSplitRows = 32;

static int compress_vec(int dt, int D) {
  if (dt == 1) return D <= 512 ? 8 : 16;
  return D <= 256 ? 4 : (D == 512 ? 8 : 16);
}

// Channel slices per entry: enough workgroups for about 256 in all, slices
// of at least 8 lanes; with a gain only where the finisher applies (D a
// multiple of 512, so that one wave holds the row in whole 16-byte bf16
// words) and a workspace is given.
static int compress_slices(const CompressArgs& a) {
  const int64_t entries = (int64_t)a.B * a.n_out;
  if (entries >= kCompressSplitBelow || a.m * (a.overlap ? 2 : 1) < kCompressSplitRows) return 1;
  // packed FP8 rows are stored by one wave holding the whole row: the
  // slices' finisher (which needs the gain) or the single workgroup
  if (a.out_fp8_row > 0 && !a.gain) return 1;
  if (a.gain && (a.D % 512 != 0 || !a.ws_y ||
                 a.ws_bytes < (size_t)entries * a.D * sizeof(float)))
    return 1;
  const int vec = compress_vec(a.dt, a.D);
  int s = 1;
  while (2 * s * entries <= 256 && a.D / (2 * s) >= 8 * vec) s *= 2;
  return s;
}

size_t compress_ws_bytes(int dt, int B, int n_out, int D, int rows) {
  (void)dt;
  const int64_t entries = (int64_t)B * n_out;
  if (entries <= 0 || entries >= kCompressSplitBelow || rows < kCompressSplitRows ||
      D % 512 != 0)
    return 0;
  return (size_t)entries * D * sizeof(float);
}

// Row groups: about 4 rows per group (one batch of loads each; a merge step
// costs more than streaming 4 more rows), at most 512 threads, at least one
// full wave.  Threads of a job whose channel slices take L lanes.
static int compress_threads(const CompressArgs& a, int L) {
  const int rows = a.m * (a.overlap ? 2 : 1);
  const size_t ds_bytes = (size_t)(a.D / a.slices) * sizeof(float);
  int G = 1;  // doubling G grows the merge staging to 3 G Ds floats
  while (4 * G < rows && 2 * G * L <= 512 && 3 * G * ds_bytes <= 65536) G <<= 1;
  while (G * L < 64 && 2 * G * L <= 512 && 3 * G * ds_bytes <= 65536) G <<= 1;
  return G * L;
}

// One launch for n (1 or 2) jobs of one VEC; the block is the largest any
// job asks for, and each job spreads its rows over blockDim / L groups.
// The short-block streaming kernel covers a call whose jobs pool at most
// kRowsMax rows per entry, keep whole entries (no channel slices) and have
// many entries: a short block's cost is its bytes, not the merge.
constexpr int64_t kRowsKernelMinEntries = 256;

// Block shapes the kernel is instantiated for: CSA (m = 4, overlap) and
// window rows (m = 1).
static bool rows_kernel_covers(const CompressArgs& a, int vec) {
  const int L = a.D / vec;
  const bool shape = (a.m == 4 && a.overlap) || (a.m == 1 && !a.overlap);
  return shape && a.slices == 1 && L >= 1 && L <= 64 && vec <= 8 && a.D <= kRowsMaxD &&
         (int64_t)a.B * a.n_out >= kRowsKernelMinEntries &&
         (a.out_fp8_row == 0 || L == 64);
}

template <typename T, int VEC>
static hipError_t launch_compress_t(const CompressArgs* jobs, int n, hipStream_t stream) {
  bool rows_ok = true;
  int64_t most = 0;
  for (int k = 0; k < n; ++k) {
    rows_ok = rows_ok && rows_kernel_covers(jobs[k], VEC);
    const int64_t waves = ((int64_t)jobs[k].B * jobs[k].n_out + (64 / (jobs[k].D / VEC)) - 1) /
                          (64 / (jobs[k].D / VEC));
    most = max(most, waves);
  }
  if (rows_ok && (n == 1 || (jobs[1].m == jobs[0].m && jobs[1].overlap == jobs[0].overlap))) {
    // about 12 waves per compute unit, each striding over its entries
    const int64_t wgs = min((most + 3) / 4, (int64_t)256 * 3);
    const dim3 grid((unsigned)wgs, n);
    if constexpr (VEC <= 8) {
      if (jobs[0].m == 4)
        hipLaunchKernelGGL((compress_rows_kernel<T, VEC, 4, true>), grid, dim3(256), 0, stream,
                           jobs[0], n > 1 ? jobs[1] : jobs[0]);
      else
        hipLaunchKernelGGL((compress_rows_kernel<T, VEC, 1, false>), grid, dim3(256), 0, stream,
                           jobs[0], n > 1 ? jobs[1] : jobs[0]);
      return hipGetLastError();
    }
  }
  int threads = 0;
  for (int k = 0; k < n; ++k)
    threads = max(threads, compress_threads(jobs[k], jobs[k].D / jobs[k].slices / VEC));
  size_t smem = 0;
  for (int k = 0; k < n; ++k) {
    const int Ds = jobs[k].D / jobs[k].slices;
    smem = max(smem, 3 * (size_t)(threads / (Ds / VEC) / 2) * Ds * sizeof(float));
  }
  if (n > 1 && smem > 65536) {  // too different to share a block shape: one launch each
    for (int k = 0; k < n; ++k) {
      const hipError_t e = launch_compress_t<T, VEC>(jobs + k, 1, stream);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  const CompressArgs& a = jobs[0];
  dim3 grid(a.n_out, a.B, a.slices * n), block(threads);
  hipLaunchKernelGGL((compress_kernel<T, VEC>), grid, block, smem, stream, a, n > 1 ? jobs[1] : a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || n > 1 || a.slices == 1 || !a.gain) return e;
  const int vf = a.D / 64;
  dim3 fgrid(a.n_out, a.B);
  if (vf == 8) hipLaunchKernelGGL((compress_finish<T, 8>), fgrid, dim3(64), 0, stream, a);
  else hipLaunchKernelGGL((compress_finish<T, 16>), fgrid, dim3(64), 0, stream, a);
  return hipGetLastError();
}

static hipError_t launch_jobs(const CompressArgs* jobs, int n, hipStream_t stream) {
  const CompressArgs& a = jobs[0];
  const int vec = compress_vec(a.dt, a.D);
  if (a.dt == 1) {
    if (vec == 8) return launch_compress_t<bf16_t, 8>(jobs, n, stream);
    return launch_compress_t<bf16_t, 16>(jobs, n, stream);
  }
  if (vec == 4) return launch_compress_t<float, 4>(jobs, n, stream);
  if (vec == 8) return launch_compress_t<float, 8>(jobs, n, stream);
  return launch_compress_t<float, 16>(jobs, n, stream);
}

hipError_t launch_compress(CompressArgs a, hipStream_t stream) {
  a.slices = compress_slices(a);
  return launch_jobs(&a, 1, stream);
}

hipError_t launch_compress_batch(const CompressArgs* jobs_in, int n, hipStream_t stream) {
  CompressArgs jobs[2] = {jobs_in[0], n > 1 ? jobs_in[1] : jobs_in[0]};
  for (int k = 0; k < 2; ++k) jobs[k].slices = 1;  // one workgroup per entry and job
  // jobs of different element widths per lane run one launch each
  if (n > 1 && compress_vec(jobs[0].dt, jobs[0].D) != compress_vec(jobs[1].dt, jobs[1].D)) {
    const hipError_t e = launch_jobs(jobs, 1, stream);
    return e != hipSuccess ? e : launch_jobs(jobs + 1, 1, stream);
  }
  return launch_jobs(jobs, n, stream);
}

}  // namespace csa
