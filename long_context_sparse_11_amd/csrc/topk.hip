// Top-K selector over the causally visible entries ("DeepSeek-v4 Beyond
// Basics" section 3.2.2, eq. 17; mask before ranking per "DeepSeek V4
// Inside", "How does CSA compress 8 tokens into 4 KV entries?"; all rows
// kept when at most K are visible per "07 The Model", "The indexer: a
// learned retrieval mechanism"; -1 for empty slots per the transformers
// "DeepSeek-V4" page, "Tata letak attention mask").
//
// One 512-thread workgroup selects from one segment held in LDS (at most
// kTopkCap scores) by an exact most-significant-digit radix select on
// order-preserving uint32 keys: four 8-bit digits, an LDS histogram per
// digit, the digit holding the K-th largest found by a suffix scan, early
// exit as soon as the threshold bin is taken whole.  Elements above the
// threshold are all kept; among those equal to it the lowest indices are
// kept.  The output is compacted in index order with wave ballots, so the
// chosen indices come out ascending and the result is deterministic.
//
// Rows longer than kTopkCap are handled in two launches: mode 1 selects K
// from every kTopkCap-long chunk, mode 2 selects K from the concatenated
// chunk winners (still in ascending index order, so ties resolve the same).
#include "kernels.h"

namespace csa {

constexpr int kTkThreads = 512;
constexpr int kTkWaves = kTkThreads / 64;
constexpr int kTkRounds = kTopkCap / kTkThreads;

__global__ __launch_bounds__(kTkThreads) void topk_kernel(TopkArgs a) {
  __shared__ uint32_t keys[kTopkCap];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t cnt_gt[kTkRounds * kTkWaves];
  __shared__ uint32_t cnt_eq[kTkRounds * kTkWaves];
  __shared__ uint32_t sel_digit, sel_above;

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

  // ---- load keys, first-digit histogram
  for (int e = tid; e < 256; e += kTkThreads) hist[e] = 0;
  __syncthreads();
  for (int e = tid; e < n; e += kTkThreads) {
    uint32_t key = score_key(src[e]);
    if (src_idx && src_idx[e] < 0) key = 0;  // empty candidate slot ranks last
    keys[e] = key;
    atomicAdd(&hist[key >> 24], 1u);
  }
  __syncthreads();

  uint32_t prefix = 0, mask = 0;
  int remaining = K;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    if (pass > 0) {
      for (int e = tid; e < 256; e += kTkThreads) hist[e] = 0;
      __syncthreads();
      for (int e = tid; e < n; e += kTkThreads) {
        const uint32_t key = keys[e];
        if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
    }
    // wave 0: find the digit d with above(d) < remaining <= above(d) + hist[d]
    if (wave == 0) {
      uint32_t h[4], local = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) { h[k] = hist[4 * lane + k]; local += h[k]; }
      uint32_t suffix = local;  // inclusive suffix sum over lanes >= lane
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t o = __shfl_down(suffix, off);
        if (lane + off < 64) suffix += o;
      }
      uint32_t above = suffix - local;  // bins of higher lanes
#pragma unroll
      for (int k = 3; k >= 0; --k) {
        if (above < (uint32_t)remaining && (uint32_t)remaining <= above + h[k]) {
          sel_digit = 4 * lane + k;
          sel_above = above;
        }
        above += h[k];
      }
    }
    __syncthreads();
    const uint32_t d = sel_digit;
    remaining -= (int)sel_above;
    prefix |= d << shift;
    mask |= 255u << shift;
    const bool whole = hist[d] == (uint32_t)remaining;
    __syncthreads();  // hist is rewritten by the next pass
    if (whole) break;
  }

  // ---- compaction in index order: key above the threshold bin -> kept;
  // in the bin -> kept if among the first `remaining` of the bin.
  const int rounds = (n + kTkThreads - 1) / kTkThreads;
  for (int r = 0; r < rounds; ++r) {
    const int e = r * kTkThreads + tid;
    const uint32_t key = e < n ? (keys[e] & mask) : 0u;
    const bool valid = e < n;
    const uint64_t bgt = __ballot(valid && key > prefix);
    const uint64_t beq = __ballot(valid && key == prefix);
    if (lane == 0) {
      cnt_gt[r * kTkWaves + wave] = __popcll(bgt);
      cnt_eq[r * kTkWaves + wave] = __popcll(beq);
    }
  }
  __syncthreads();
  // exclusive scan of the (round, wave) counts; wave 0 does both arrays
  if (wave == 0) {
    const int total = rounds * kTkWaves;
    uint32_t run_gt = 0, run_eq = 0;
    for (int base = 0; base < total; base += 64) {
      const int e = base + lane;
      const uint32_t vg = e < total ? cnt_gt[e] : 0u;
      const uint32_t ve = e < total ? cnt_eq[e] : 0u;
      uint32_t ig = vg, ie = ve;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t og = __shfl_up(ig, off);
        const uint32_t oe = __shfl_up(ie, off);
        if (lane >= off) { ig += og; ie += oe; }
      }
      if (e < total) { cnt_gt[e] = run_gt + ig - vg; cnt_eq[e] = run_eq + ie - ve; }
      run_gt += __shfl(ig, 63);
      run_eq += __shfl(ie, 63);
    }
  }
  __syncthreads();
  for (int r = 0; r < rounds; ++r) {
    const int e = r * kTkThreads + tid;
    const uint32_t key = e < n ? (keys[e] & mask) : 0u;
    const bool valid = e < n;
    const bool gt = valid && key > prefix;
    const bool eq = valid && key == prefix;
    const uint64_t bgt = __ballot(gt);
    const uint64_t beq = __ballot(eq);
    const uint32_t before_gt = cnt_gt[r * kTkWaves + wave] + lanes_below(bgt);
    const uint32_t before_eq = cnt_eq[r * kTkWaves + wave] + lanes_below(beq);
    if (gt || (eq && before_eq < (uint32_t)remaining)) {
      const uint32_t pos = before_gt + min(before_eq, (uint32_t)remaining);
      oidx[pos] = src_idx ? src_idx[e] : base_index + e;
      if (osc) osc[pos] = src[e];
    }
  }
}

hipError_t launch_topk(const TopkArgs& a, int segments, hipStream_t stream) {
  if (segments == 0) return hipSuccess;
  hipLaunchKernelGGL(topk_kernel, dim3(segments), dim3(kTkThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace csa
