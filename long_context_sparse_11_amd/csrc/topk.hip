// Top-K selector over the causally visible entries ("DeepSeek-v4 Beyond
// Basics" section 3.2.2, eq. 17; mask before ranking per "DeepSeek V4
// Inside", "How does CSA compress 8 tokens into 4 KV entries?"; all rows
// kept when at most K are visible per "07 The Model", "The indexer: a
// learned retrieval mechanism"; -1 for empty slots per the transformers
// "DeepSeek-V4" page, "Tata letak attention mask").
//
// One 512-thread workgroup selects from one segment of at most kTopkCap
// scores, each thread holding 32 consecutive ones as order-preserving uint32
// keys in registers (element e lives in thread e / 32, slot e % 32).  The select is
// an exact most-significant-digit radix select with adaptive 12-bit digits:
// every pass takes the 12 bits just below the common prefix of the keys
// still in play (block min/max), histograms them in LDS (4096 bins, fine
// enough that lanes seldom collide on a bin), and a block-wide suffix scan
// finds the bin holding the K-th largest.  It stops when that bin is taken
// whole or all 32 bits are fixed (three passes at most for distinct keys).
// Keys above the bin are all kept; keys inside it are kept in index order
// until K are chosen, so ties go to the lower index.  Output positions come
// from one block-wide prefix count over the threads' (above, inside) tallies:
// the chosen indices come out ascending and the result is deterministic.
//
// Rows longer than kTopkCap go through two launches: mode 1 selects K per
// chunk, mode 2 selects K from the concatenated chunk winners (still in
// ascending index order, so ties resolve identically).
#include "kernels.h"

namespace csa {

constexpr int kTkThreads = 512;
constexpr int kTkWaves = kTkThreads / 64;
constexpr int kTkRounds = kTopkCap / kTkThreads;  // keys per thread
constexpr int kDigitBits = 12;
constexpr int kBins = 1 << kDigitBits;
constexpr int kBinsPerThread = kBins / kTkThreads;

struct TkShared {
  uint32_t hist[kBins];
  uint32_t red[2][kTkWaves];
  uint32_t sel_digit, sel_above;
};

__device__ __forceinline__ void block_minmax(uint32_t& mn, uint32_t& mx, TkShared& S, int wave,
                                             int lane) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    mn = min(mn, (uint32_t)__shfl_xor((int)mn, off));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, off));
  }
  if (lane == 0) {
    S.red[0][wave] = mn;
    S.red[1][wave] = mx;
  }
  __syncthreads();
  mn = S.red[0][0];
  mx = S.red[1][0];
#pragma unroll
  for (int w = 1; w < kTkWaves; ++w) {
    mn = min(mn, S.red[0][w]);
    mx = max(mx, S.red[1][w]);
  }
  __syncthreads();
}

__global__ __launch_bounds__(kTkThreads) void topk_kernel(TopkArgs a) {
  __shared__ TkShared S;
  const int seg = blockIdx.x;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int K = a.K;

  // ---- segment geometry
  int query, n, base_index = 0;
  const float* src;
  const int32_t* src_idx = nullptr;
  if (a.mode == 2) {
    query = seg;
    n = a.nchunks * K;
    src = a.scores + (int64_t)query * n;
    src_idx = a.in_idx + (int64_t)query * n;
  } else {
    const int c = (a.mode == 1) ? seg % a.nchunks : 0;
    query = (a.mode == 1) ? seg / a.nchunks : seg;
    const int b = query / a.Tq;
    const int t = query - b * a.Tq;
    const int n_vis = visible_entries(a.q_pos0[b] + t, a.m, min(a.n_entries[b], a.N_cap));
    base_index = (a.mode == 1) ? c * a.chunk : 0;
    n = min(max(n_vis - base_index, 0), a.mode == 1 ? a.chunk : n_vis);
    src = a.scores + (int64_t)query * a.N_cap + base_index;
  }
  int32_t* oidx = a.out_idx + (int64_t)seg * K;
  float* osc = a.out_scores ? a.out_scores + (int64_t)seg * K : nullptr;

  // ---- at most K candidates: keep them all (mode 2 always has more than K)
  if (n <= K) {
    for (int e = tid; e < K; e += kTkThreads) {
      const bool v = e < n;
      oidx[e] = v ? base_index + e : -1;
      if (osc) osc[e] = v ? src[e] : -INFINITY;
    }
    return;
  }

  // ---- keys in registers; every load issued before any is consumed.  A
  // slot beyond n, or an empty candidate slot (index -1), takes no part.
  uint32_t key[kTkRounds];
  int32_t vi[kTkRounds];  // candidate indices (mode 2)
  uint32_t live = 0;      // bit i: slot i holds a key
  const int e0 = tid * kTkRounds;
  {
    float v[kTkRounds];
    const bool vec = ((((uintptr_t)src) | ((uintptr_t)src_idx)) & 15) == 0 && e0 + kTkRounds <= n;
    if (vec) {
#pragma unroll
      for (int u = 0; u < kTkRounds / 4; ++u) {
        const f32x4_t x = reinterpret_cast<const f32x4_t*>(src + e0)[u];
        v[4 * u] = x[0]; v[4 * u + 1] = x[1]; v[4 * u + 2] = x[2]; v[4 * u + 3] = x[3];
      }
      if (src_idx) {
#pragma unroll
        for (int u = 0; u < kTkRounds / 4; ++u) {
          const int4 x = reinterpret_cast<const int4*>(src_idx + e0)[u];
          vi[4 * u] = x.x; vi[4 * u + 1] = x.y; vi[4 * u + 2] = x.z; vi[4 * u + 3] = x.w;
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < kTkRounds; ++i) {
        const int e = e0 + i;
        v[i] = e < n ? src[e] : 0.f;
        vi[i] = (src_idx && e < n) ? src_idx[e] : 0;
      }
    }
    if (!src_idx) {
#pragma unroll
      for (int i = 0; i < kTkRounds; ++i) vi[i] = 0;
    }
#pragma unroll
    for (int i = 0; i < kTkRounds; ++i) {
      key[i] = score_key(v[i]);
      if (e0 + i < n && vi[i] >= 0) live |= 1u << i;
    }
  }
#pragma unroll
  for (int k = 0; k < kBinsPerThread; ++k) S.hist[tid * kBinsPerThread + k] = 0;

  // ---- radix select with adaptive 12-bit digits (the histogram is zero on
  // entry to every pass; the barriers of the min/max reduction order the
  // zeroing before the counting)
  uint32_t prefix = 0, mask = 0;
  int remaining = K;
  for (;;) {
    uint32_t mn = 0xffffffffu, mx = 0u;
#pragma unroll
    for (int i = 0; i < kTkRounds; ++i) {
      if (((live >> i) & 1) && (key[i] & mask) == prefix) {
        mn = min(mn, key[i]);
        mx = max(mx, key[i]);
      }
    }
    block_minmax(mn, mx, S, wave, lane);
    const uint32_t diff = mn ^ mx;
    if (diff == 0) {  // every key in play is equal: take them in index order
      prefix = mn;
      mask = 0xffffffffu;
      break;
    }
    const int hb = 31 - __clz(diff);
    const uint32_t common = hb == 31 ? 0u : ~((2u << hb) - 1u);
    mask |= common;
    prefix = mn & mask;
    const int shift = max(hb + 1 - kDigitBits, 0);
    const uint32_t dmask = (1u << (hb + 1 - shift)) - 1u;
#pragma unroll
    for (int i = 0; i < kTkRounds; ++i) {
      if (((live >> i) & 1) && (key[i] & mask) == prefix)
        atomicAdd(&S.hist[(key[i] >> shift) & dmask], 1u);
    }
    __syncthreads();
    // bins 8t .. 8t+7 belong to thread t; suffix sums run from the top bin down
    uint32_t h[kBinsPerThread], local = 0;
#pragma unroll
    for (int k = 0; k < kBinsPerThread; ++k) {
      h[k] = S.hist[tid * kBinsPerThread + k];
      local += h[k];
    }
    uint32_t suffix = local;  // inclusive, over lanes >= lane of this wave
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t o = __shfl_down(suffix, off);
      if (lane + off < 64) suffix += o;
    }
    if (lane == 0) S.red[0][wave] = suffix;  // wave total
    __syncthreads();
    uint32_t above = suffix - local;
    for (int w = wave + 1; w < kTkWaves; ++w) above += S.red[0][w];
#pragma unroll
    for (int k = kBinsPerThread - 1; k >= 0; --k) {
      if (above < (uint32_t)remaining && (uint32_t)remaining <= above + h[k]) {
        S.sel_digit = tid * kBinsPerThread + k;
        S.sel_above = above;
      }
      above += h[k];
    }
    __syncthreads();
    const uint32_t d = S.sel_digit;
    remaining -= (int)S.sel_above;
    mask |= dmask << shift;
    prefix |= d << shift;
    const bool whole = S.hist[d] == (uint32_t)remaining;
    __syncthreads();  // every thread has read hist[d]
#pragma unroll
    for (int k = 0; k < kBinsPerThread; ++k) S.hist[tid * kBinsPerThread + k] = 0;
    if (whole || shift == 0) break;
  }

  // ---- emit in index order: above the threshold bin -> kept; inside it ->
  // kept if among the first `remaining` of the bin.  One block-wide
  // exclusive prefix of the per-thread tallies gives every thread its start.
  uint32_t ngt = 0, neq = 0;
#pragma unroll
  for (int i = 0; i < kTkRounds; ++i) {
    const bool v = (live >> i) & 1;
    const uint32_t k = key[i] & mask;
    ngt += (v && k > prefix) ? 1u : 0u;
    neq += (v && k == prefix) ? 1u : 0u;
  }
  uint32_t igt = ngt, ieq = neq;  // inclusive prefix within the wave
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t og = __shfl_up(igt, off);
    const uint32_t oe = __shfl_up(ieq, off);
    if (lane >= off) { igt += og; ieq += oe; }
  }
  if (lane == 63) { S.red[0][wave] = igt; S.red[1][wave] = ieq; }
  __syncthreads();
  uint32_t before_gt = igt - ngt, before_eq = ieq - neq;
  for (int w = 0; w < wave; ++w) { before_gt += S.red[0][w]; before_eq += S.red[1][w]; }
#pragma unroll
  for (int i = 0; i < kTkRounds; ++i) {
    const bool v = (live >> i) & 1;
    const uint32_t k = key[i] & mask;
    if (v && k > prefix) {
      const uint32_t p = before_gt + min(before_eq, (uint32_t)remaining);
      oidx[p] = src_idx ? vi[i] : base_index + e0 + i;
      if (osc) osc[p] = key_score(key[i]);
      ++before_gt;
    } else if (v && k == prefix) {
      if (before_eq < (uint32_t)remaining) {
        const uint32_t p = before_gt + before_eq;
        oidx[p] = src_idx ? vi[i] : base_index + e0 + i;
        if (osc) osc[p] = key_score(key[i]);
      }
      ++before_eq;
    }
  }
}

hipError_t launch_topk(const TopkArgs& a, int segments, hipStream_t stream) {
  if (segments == 0) return hipSuccess;
  hipLaunchKernelGGL(topk_kernel, dim3(segments), dim3(kTkThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace csa
