// Top-K selector over the causally visible entries ("DeepSeek-v4 Beyond
// Basics" section 3.2.2, eq. 17; mask before ranking per "DeepSeek V4
// Inside", "How does CSA compress 8 tokens into 4 KV entries?"; all rows
// kept when at most K are visible per "07 The Model", "The indexer: a
// learned retrieval mechanism"; -1 for empty slots per the transformers
// "DeepSeek-V4" page, "Tata letak attention mask").
//
// One 1024-thread workgroup selects from one segment of at most kTopkCap
// scores, each thread holding 16 consecutive ones as order-preserving uint32
// keys in registers (element e lives in thread e / 16, slot e % 16).  The
// select is exact and deterministic:
//  1. the first digit of a key is a monotone linear map of its score over
//     the segment's [min, max] onto 4096 bins (a larger score never gets a
//     smaller digit, so every key in a higher bin beats every key in a lower
//     one); one LDS histogram and a block suffix scan find the bin holding
//     the K-th largest.  Spreading the range linearly keeps both same-bin
//     atomic collisions and the threshold bin's population small, unlike
//     digits taken from the float bits, which pile a smooth distribution
//     into a few dozen bins;
//  2. the keys of that bin are compacted into LDS and one wave finds the
//     exact threshold key among them: by direct ranking when there are at
//     most 64, else by a barrier-free radix select on 8-bit digits;
//  3. keys in higher bins and keys above the threshold are all kept, keys
//     equal to it are kept in index order until K are chosen (ties go to the
//     lower index); output positions come from one block-wide prefix count,
//     so the chosen indices come out ascending.
// A degenerate or non-finite score range, or a threshold bin too full for
// one wave (heavy ties), falls back to an adaptive block-level radix select
// on the keys themselves (same answer, slower).
//
// Rows longer than kTopkCap go through two launches: mode 1 selects K per
// chunk, mode 2 selects K from the concatenated chunk winners (still in
// ascending index order, so ties resolve identically).
#include "kernels.h"

namespace csa {

constexpr int kTkThreads = 1024;
constexpr int kTkWaves = kTkThreads / 64;
constexpr int kTkRounds = kTopkCap / kTkThreads;  // keys per thread
constexpr int kDigitBits = 12;
constexpr int kBins = 1 << kDigitBits;
constexpr int kBinsPerThread = kBins / kTkThreads;
constexpr int kBinCap = 2048;  // most keys of the threshold bin one wave resolves
static_assert(kTkRounds <= 32, "slot masks are 32 bits");

constexpr int kMaxTopK = 4096;  // largest K a segment selects
struct TkShared {
  union {
    struct {
      uint32_t hist[kBins];
      uint32_t bin[kBinCap];
    };
    // the chosen (index, score) pairs at their output positions, written
    // once the selection no longer reads hist or bin
    int2 out[kMaxTopK];
  };
  uint32_t red[3][kTkWaves];
  uint32_t sel_digit, sel_above, sel_count, fill;
};

__device__ __forceinline__ void block_minmax(uint32_t& mn, uint32_t& mx, TkShared& S, int wave,
                                             int lane) {
  mn = wave_min(mn);
  mx = wave_max(mx);
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

// Exclusive block prefix of x (all threads take part); also returns the
// block total.  Uses S.red[0] and two barriers; TRAIL false drops the second
// (which keeps S.red[0] from being rewritten while others still read it) where
// a barrier comes before the next write of S.red anyway.
template <bool TRAIL = true>
__device__ __forceinline__ uint32_t block_excl_sum(uint32_t x, uint32_t& total, TkShared& S,
                                                   int wave, int lane) {
  const uint32_t incl = wave_incl_sum(x);
  if (lane == 63) S.red[0][wave] = incl;
  __syncthreads();
  uint32_t before = incl - x, tot = 0;
#pragma unroll
  for (int w = 0; w < kTkWaves; ++w) {
    const uint32_t t = S.red[0][w];
    before += w < wave ? t : 0u;
    tot += t;
  }
  total = tot;
  if (TRAIL) __syncthreads();
  return before;
}

// CAND: the segment is a merge of chunk winners (mode 2), whose candidate
// indices come with the scores; otherwise indices are positions.  WIDE: held
// to 64 VGPRs so that two workgroups share a compute unit, for launches of
// many segments (a prefill chunk's queries: 4,096 selects took 132 us at one
// workgroup per compute unit, 101 us at two); what that spills costs a
// latency-bound decode select ~0.4 us, so few segments keep the unconstrained
// instance.
// RND: keys per thread (the segment's capacity is kTkThreads * RND); the
// merge of at most 8,192 chunk winners takes 8, so every wave holds keys.
template <bool CAND, bool WIDE, int RND = kTkRounds>
__global__ __launch_bounds__(kTkThreads)
__attribute__((amdgpu_waves_per_eu(WIDE ? 8 : 1, WIDE ? 8 : 4)))
void topk_kernel(TopkArgs a) {
  static_assert(RND % 4 == 0 && RND <= kTkRounds, "keys per thread");
  __shared__ TkShared S;
  const int seg = blockIdx.x;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int K = a.K;
  // the scores stay in registers for the first digit where registers allow
  constexpr bool KEEP_V = !WIDE;

  // ---- segment geometry from the arguments alone: the scores are requested
  // before the visible count (two dependent scalar loads) is known.  `cap`
  // is what the segment's row holds; slots past the visible count are read
  // (clamped into the row) and take no part.
  int query, base_index = 0, cap;
  const float* src;
  const int32_t* src_idx = nullptr;
  if (CAND) {
    query = seg;
    cap = a.nchunks * K;
    src = a.scores + (int64_t)query * cap;
    src_idx = a.in_idx + (int64_t)query * cap;
  } else {
    const int c = (a.mode == 1) ? seg % a.nchunks : 0;
    query = (a.mode == 1) ? seg / a.nchunks : seg;
    base_index = (a.mode == 1) ? c * a.chunk : 0;
    cap = (a.mode == 1) ? min(a.chunk, a.N_cap - base_index) : a.N_cap;
    src = a.scores + (int64_t)query * a.N_cap + base_index;
  }
  int32_t* oidx = a.out_idx + (int64_t)seg * K;
  float* osc = a.out_scores ? a.out_scores + (int64_t)seg * K : nullptr;
  // an empty pool (no entry yet, N_cap = 0): nothing to read, every slot
  // is empty; decided from the arguments before any load
  if (cap <= 0) {
    for (int e = tid; e < K; e += kTkThreads) {
      oidx[e] = -1;
      if (osc) osc[e] = -INFINITY;
    }
    return;
  }

  // ---- keys in registers; every load issued before any is consumed
  uint32_t key[RND];
  int32_t vi[CAND ? RND : 1];  // candidate indices (mode 2)
  const int e0 = tid * RND;
  float v[RND];
  {
    const bool vec = ((((uintptr_t)src) | ((uintptr_t)src_idx)) & 15) == 0 && e0 + RND <= cap;
    if (vec) {
#pragma unroll
      for (int u = 0; u < RND / 4; ++u) {
        const f32x4_t x = reinterpret_cast<const f32x4_t*>(src + e0)[u];
        v[4 * u] = x[0]; v[4 * u + 1] = x[1]; v[4 * u + 2] = x[2]; v[4 * u + 3] = x[3];
      }
      if constexpr (CAND) {
#pragma unroll
        for (int u = 0; u < RND / 4; ++u) {
          const int4 x = reinterpret_cast<const int4*>(src_idx + e0)[u];
          vi[4 * u] = x.x; vi[4 * u + 1] = x.y; vi[4 * u + 2] = x.z; vi[4 * u + 3] = x.w;
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < RND; ++i) {
        const int e = min(e0 + i, cap - 1);
        v[i] = src[e];
        if constexpr (CAND) vi[i] = src_idx[e];
      }
    }

  }
  int n = cap;
  if (!CAND) {
    const int b = query / a.Tq;
    const int t = query - b * a.Tq;
    const int n_vis = visible_entries(a.q_pos0[b] + t, a.m, min(a.n_entries[b], a.N_cap));
    n = min(max(n_vis - base_index, 0), a.mode == 1 ? a.chunk : n_vis);
  }

  // ---- at most K candidates: keep them all (mode 2 always has more than K)
  if (n <= K) {
    for (int e = tid; e < K; e += kTkThreads) {
      const bool ok = e < n;
      oidx[e] = ok ? base_index + e : -1;
      if (osc) osc[e] = ok ? src[e] : -INFINITY;
    }
    return;
  }
  // a slot beyond n, or an empty candidate slot (index -1), takes no part
  uint32_t live = 0;  // bit i: slot i holds a key
#pragma unroll
  for (int i = 0; i < RND; ++i) {
    key[i] = score_key(v[i]);
    if (e0 + i < n && (!CAND || vi[CAND ? i : 0] >= 0)) live |= 1u << i;
  }
#pragma unroll
  for (int k = 0; k < kBinsPerThread; ++k) S.hist[tid * kBinsPerThread + k] = 0;
  if (tid == 0) S.fill = 0;

  // ---- radix select with adaptive 12-bit digits over the register slots in
  // `act`: returns (prefix, mask, remaining) such that the chosen keys are
  // those with (key & mask) > prefix plus the first `remaining` (in index
  // order) with (key & mask) == prefix.  The histogram is zero on entry to
  // every pass; the barriers of the min/max reduction order the zeroing
  // before the counting.
  auto select = [&](uint32_t act, int want, uint32_t& prefix, uint32_t& mask, int& remaining) {
    prefix = 0;
    mask = 0;
    remaining = want;
    for (;;) {
      uint32_t mn = 0xffffffffu, mx = 0u;
#pragma unroll
      for (int i = 0; i < RND; ++i) {
        if (((act >> i) & 1) && (key[i] & mask) == prefix) {
          mn = min(mn, key[i]);
          mx = max(mx, key[i]);
        }
      }
      block_minmax(mn, mx, S, wave, lane);
      const uint32_t diff = mn ^ mx;
      if (diff == 0) {  // every key in play is equal: take them in index order
        prefix = mn;
        mask = 0xffffffffu;
        return;
      }
      const int hb = 31 - __clz(diff);
      const uint32_t common = hb == 31 ? 0u : ~((2u << hb) - 1u);
      mask |= common;
      prefix = mn & mask;
      const int shift = max(hb + 1 - kDigitBits, 0);
      const uint32_t dmask = (1u << (hb + 1 - shift)) - 1u;
#pragma unroll
      for (int i = 0; i < RND; ++i) {
        if (((act >> i) & 1) && (key[i] & mask) == prefix)
          atomicAdd(&S.hist[(key[i] >> shift) & dmask], 1u);
      }
      __syncthreads();
      // bins kBinsPerThread*t .. +kBinsPerThread-1 belong to thread t; the
      // suffix sums run from the top bin down
      uint32_t h[kBinsPerThread], local = 0;
#pragma unroll
      for (int k = 0; k < kBinsPerThread; ++k) {
        h[k] = S.hist[tid * kBinsPerThread + k];
        local += h[k];
      }
      uint32_t total;
      const uint32_t below = block_excl_sum(local, total, S, wave, lane);
      uint32_t above = total - below - local;
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
      if (whole || shift == 0) return;
    }
  };

  // ---- 1. key range and live count, then the histogram of the linear
  // first digit
  uint32_t kmn = 0xffffffffu, kmx = 0u;
#pragma unroll
  for (int i = 0; i < RND; ++i) {
    if ((live >> i) & 1) {
      kmn = min(kmn, key[i]);
      kmx = max(kmx, key[i]);
    }
  }
  uint32_t n_live;
  {
    kmn = wave_min(kmn);
    kmx = wave_max(kmx);
    const uint32_t cnt = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_sum(__popc(live)), 63);
    if (lane == 0) {
      S.red[0][wave] = kmn;
      S.red[1][wave] = kmx;
      S.red[2][wave] = cnt;
    }
    __syncthreads();  // also orders the zeroing above before the counting
    n_live = 0;
#pragma unroll
    for (int w = 0; w < kTkWaves; ++w) {
      kmn = min(kmn, S.red[0][w]);
      kmx = max(kmx, S.red[1][w]);
      n_live += S.red[2][w];
    }
  }
  const float fmn = key_score(kmn), fmx = key_score(kmx);
  const float range = fmx - fmn;
  const float scale = (float)kBins / range;
  const bool linear = kmn < kmx && isfinite(fmn) && isfinite(fmx) && isfinite(range) &&
                      isfinite(scale) && scale > 0.f;
  // S.red is read above and rewritten next: by the linear path only after
  // the histogram's barrier, by the other two paths at once (the values
  // every thread read are equal, so the branch is uniform)
  if (!linear || n_live <= (uint32_t)K) __syncthreads();

  uint32_t prefix = 0, mask = 0;   // threshold among the keys of in_bin
  int remaining = K;
  uint32_t above_m = 0;            // slots in a bin above the threshold bin: always kept
  uint32_t in_bin = live;          // slots competing at the threshold
  if (n_live <= (uint32_t)K) {
    // at most K candidates (mode 2 with few visible entries): keep them all
    above_m = live;
    in_bin = 0;
    remaining = 0;
    for (int e = (int)n_live + tid; e < K; e += kTkThreads) {
      oidx[e] = -1;
      if (osc) osc[e] = -INFINITY;
    }
  } else if (linear) {
    // the linear first digit, recomputed where it is used again (held in
    // registers it would cost 16 per thread): one FMA on the score, which
    // the unconstrained instance keeps in registers (the other converts the
    // key back).  Monotone in the score: the FMA rounds its exact value
    // once, and the conversion truncates (a value just below 0 gives 0).
    const float off = -fmn * scale;
    auto digit = [&](int i) {
      const float x = KEEP_V ? v[i] : key_score(key[i]);
      return min((uint32_t)fmaf(x, scale, off), (uint32_t)(kBins - 1));
    };
    if (!CAND && !WIDE) {
      // a decode select: every slot adds its live bit (0 for a dead slot,
      // whose digit is any bin), in straight-line code (19.2 -> 18.8 us per
      // 64K decode call).  The merge of chunk winners and the two-per-CU
      // instance keep the branch per slot: without it they measured slower
      // (the 1M merge by ~5 us, a prefill chunk's selects by ~45 us).
#pragma unroll
      for (int i = 0; i < RND; ++i) atomicAdd(&S.hist[digit(i)], (live >> i) & 1u);
    } else {
#pragma unroll
      for (int i = 0; i < RND; ++i) {
        if ((live >> i) & 1) atomicAdd(&S.hist[digit(i)], 1u);
      }
    }
    __syncthreads();
    uint32_t h[kBinsPerThread], local = 0;
#pragma unroll
    for (int k = 0; k < kBinsPerThread; ++k) {
      h[k] = S.hist[tid * kBinsPerThread + k];
      local += h[k];
    }
    uint32_t total;
    // S.red is next written after the selection's barrier below
    const uint32_t below = block_excl_sum<false>(local, total, S, wave, lane);
    uint32_t above = total - below - local;
#pragma unroll
    for (int k = kBinsPerThread - 1; k >= 0; --k) {
      if (above < (uint32_t)K && (uint32_t)K <= above + h[k]) {
        S.sel_digit = tid * kBinsPerThread + k;
        S.sel_above = above;
        S.sel_count = h[k];
      }
      above += h[k];
    }
    __syncthreads();
    const uint32_t d1 = S.sel_digit;
    const uint32_t c1 = S.sel_count;
    remaining = K - (int)S.sel_above;
    in_bin = 0;
#pragma unroll
    for (int i = 0; i < RND; ++i) {
      const bool v = (live >> i) & 1;
      const uint32_t d = digit(i);
      above_m |= (v && d > d1) ? (1u << i) : 0u;
      in_bin |= (v && d == d1) ? (1u << i) : 0u;
    }
    // sel_* are rewritten below only after a barrier (the compaction's, or
    // those of the block-level select), which every thread reaches after
    // its reads above

    if (c1 == (uint32_t)remaining) {
      // the whole bin is taken: every key of in_bin is "equal" and all fit
    } else if (c1 <= (uint32_t)kBinCap) {
      // ---- 2. compact the bin's keys (any order), one wave finishes
      const uint32_t mine = __popc(in_bin);
      const uint32_t incl = wave_incl_sum(mine);
      uint32_t base = 0;
      if (lane == 63) base = atomicAdd(&S.fill, incl);
      uint32_t pos = (uint32_t)__builtin_amdgcn_readlane((int)base, 63) + incl - mine;
#pragma unroll
      for (int i = 0; i < RND; ++i) {
        if ((in_bin >> i) & 1) S.bin[pos++] = key[i];
      }
      __syncthreads();
      if (wave == 0) {
        uint32_t pre, msk;
        int rem = remaining;
        if (c1 <= 64) {
          // rank the (at most 64) keys against each other
          const bool valid = (uint32_t)lane < c1;
          const uint32_t k = valid ? S.bin[lane] : 0u;
          uint32_t gt = 0, ge = 0;
          for (uint32_t j = 0; j < c1; ++j) {
            const uint32_t kj = (uint32_t)__builtin_amdgcn_readlane((int)k, (int)j);
            gt += kj > k ? 1u : 0u;
            ge += kj >= k ? 1u : 0u;
          }
          const bool hit = valid && gt < (uint32_t)rem && (uint32_t)rem <= ge;
          const uint64_t hm = __ballot(hit);
          const int src_lane = __ffsll((long long)hm) - 1;
          pre = (uint32_t)__builtin_amdgcn_readlane((int)k, src_lane);
          rem -= (int)(uint32_t)__builtin_amdgcn_readlane((int)gt, src_lane);
          msk = 0xffffffffu;
        } else {
          // barrier-free radix select on 8-bit digits below the bin's common
          // prefix; LDS operations of one wave complete in order
          uint32_t bmn = 0xffffffffu, bmx = 0u;
          for (uint32_t e = lane; e < c1; e += 64) {
            const uint32_t k = S.bin[e];
            bmn = min(bmn, k);
            bmx = max(bmx, k);
          }
          bmn = wave_min(bmn);
          bmx = wave_max(bmx);
          const uint32_t diff = bmn ^ bmx;
          if (diff == 0) {
            pre = bmn;
            msk = 0xffffffffu;
          } else {
            const int hb = 31 - __clz(diff);
            msk = hb == 31 ? 0u : ~((2u << hb) - 1u);
            pre = bmn & msk;
            uint32_t* wh = S.hist;  // 256 bins, 4 per lane
            for (int top = hb; top >= 0; top -= 8) {
              const int shift = max(top - 7, 0);
              const uint32_t dm = (1u << (top + 1 - shift)) - 1u;
#pragma unroll
              for (int k = 0; k < 4; ++k) wh[4 * lane + k] = 0;
              __builtin_amdgcn_wave_barrier();
              for (uint32_t e = lane; e < c1; e += 64) {
                const uint32_t k = S.bin[e];
                if ((k & msk) == pre) atomicAdd(&wh[(k >> shift) & dm], 1u);
              }
              __builtin_amdgcn_wave_barrier();
              uint32_t hh[4], loc = 0;
#pragma unroll
              for (int k = 0; k < 4; ++k) { hh[k] = wh[4 * lane + k]; loc += hh[k]; }
              const uint32_t inc = wave_incl_sum(loc);
              const uint32_t tot = (uint32_t)__builtin_amdgcn_readlane((int)inc, 63);
              uint32_t abv = tot - inc;  // bins of higher lanes
              uint32_t dsel = 0, asel = 0, csel = 0;
              bool hit = false;
#pragma unroll
              for (int k = 3; k >= 0; --k) {
                if (!hit && abv < (uint32_t)rem && (uint32_t)rem <= abv + hh[k]) {
                  hit = true; dsel = 4 * lane + k; asel = abv; csel = hh[k];
                }
                abv += hh[k];
              }
              const uint64_t hm = __ballot(hit);
              const int src_lane = __ffsll((long long)hm) - 1;
              dsel = (uint32_t)__builtin_amdgcn_readlane((int)dsel, src_lane);
              asel = (uint32_t)__builtin_amdgcn_readlane((int)asel, src_lane);
              csel = (uint32_t)__builtin_amdgcn_readlane((int)csel, src_lane);
              __builtin_amdgcn_wave_barrier();
              rem -= (int)asel;
              pre |= dsel << shift;
              msk |= dm << shift;
              if (csel == (uint32_t)rem) break;  // the whole digit bin is taken
            }
          }
        }
        if (lane == 0) {
          S.sel_digit = pre;
          S.sel_above = msk;
          S.sel_count = (uint32_t)rem;
        }
      }
      __syncthreads();
      prefix = S.sel_digit;
      mask = S.sel_above;
      remaining = (int)S.sel_count;
    } else {
      // ---- heavy ties: adaptive block-level radix inside the bin
#pragma unroll
      for (int k = 0; k < kBinsPerThread; ++k) S.hist[tid * kBinsPerThread + k] = 0;
      select(in_bin, remaining, prefix, mask, remaining);
    }
  } else {
    select(live, K, prefix, mask, remaining);
  }

  // ---- 3. emit in index order: chosen are the keys of higher bins, the
  // bin's keys above the threshold and, in index order, the first
  // `remaining` equal to it.  A thread's chosen keys fill one contiguous run
  // of the output, starting after everything chosen by lower threads.
  uint32_t gt_m = above_m, eq_m = 0;
#pragma unroll
  for (int i = 0; i < RND; ++i) {
    const bool v = (in_bin >> i) & 1;
    const uint32_t k = key[i] & mask;
    gt_m |= (v && k > prefix) ? (1u << i) : 0u;
    eq_m |= (v && k == prefix) ? (1u << i) : 0u;
  }
  const uint32_t ngt = __popc(gt_m), neq = __popc(eq_m);
  uint32_t total;  // counts packed as gt | eq << 16 (each at most kTopkCap)
  const uint32_t before = block_excl_sum<false>(ngt | (neq << 16), total, S, wave, lane);
  const uint32_t before_gt = before & 0xffffu, before_eq = before >> 16;
  // the first `take` of this thread's equal keys are chosen; the clamp comes
  // before the subtraction so that no intermediate can wrap
  const uint32_t eq_before = min(before_eq, (uint32_t)remaining);
  const uint32_t take = min(neq, (uint32_t)remaining - eq_before);
  uint32_t p = before_gt + eq_before;
  uint32_t seen_eq = 0;
  // the unconstrained instance gathers the chosen pairs in LDS at their
  // output positions (hist and bin are no longer read: every thread passed
  // the prefix count's barrier after its last read), then stores them
  // coalesced; the two-per-CU instance stores each pair where it is chosen
  // (the staging's registers cost it spills)
#pragma unroll
  for (int i = 0; i < RND; ++i) {
    const bool g = (gt_m >> i) & 1, e = (eq_m >> i) & 1;
    const bool c = g || (e && seen_eq < take);
    seen_eq += e ? 1u : 0u;
    if (c) {
      const int32_t ix = CAND ? vi[CAND ? i : 0] : base_index + e0 + i;
      const float sc = key_score(key[i]);
      if (WIDE) {
        oidx[p] = ix;
        if (osc) osc[p] = sc;
      } else {
        S.out[p] = make_int2(ix, (int)__float_as_uint(sc));
      }
      ++p;
    }
  }
  if (WIDE) return;
  const int chosen = (int)((total & 0xffffu) + min(total >> 16, (uint32_t)remaining));
  __syncthreads();
  for (int e = tid; e < chosen; e += kTkThreads) {
    const int2 o = S.out[e];
    oidx[e] = o.x;
    if (osc) osc[e] = __uint_as_float((uint32_t)o.y);
  }
}

// launches of at least this many segments take the two-per-CU instance
constexpr int kTkWideSegments = 1024;

hipError_t launch_topk(const TopkArgs& a, int segments, hipStream_t stream) {
  if (segments == 0) return hipSuccess;
  if (a.mode == 2 && (int64_t)a.nchunks * a.K <= kTkThreads * (kTkRounds / 2))
    hipLaunchKernelGGL((topk_kernel<true, false, kTkRounds / 2>), dim3(segments), dim3(kTkThreads), 0,
                       stream, a);
  else if (a.mode == 2)
    hipLaunchKernelGGL((topk_kernel<true, false>), dim3(segments), dim3(kTkThreads), 0, stream, a);
  else if (segments >= kTkWideSegments)
    hipLaunchKernelGGL((topk_kernel<false, true>), dim3(segments), dim3(kTkThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((topk_kernel<false, false>), dim3(segments), dim3(kTkThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace csa
