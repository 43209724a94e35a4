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
// attn_mfma     bf16, 64 heads x 512 (the Flash shape).  One workgroup of 4
//               waves per (query, key split).  Wave w owns 128 channels of
//               every row (16 of each 64-channel stretch): it gathers its
//               share of 32 rows per tile straight from HBM into MFMA
//               operands (each row is read once and serves all 64 heads),
//               computes
//               the partial logits S^T[row][head] over its channels,
//               the four partials are summed through LDS, every wave runs
//               the same online softmax (running max/sum per head, seeded
//               empty; the sink enters once at the end), and the wave
//               accumulates O^T[channel][head] for its own channels.
//               v_mfma_f32_32x32x16_bf16 throughout; the PV step reads its
//               row operand transposed from a wave-private LDS copy of the
//               tile, and its P operand is the lane's own softmax output.
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
  if (a.W > 0 && a.L_win > 0) {
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
  return (const T*)a.win + ((int64_t)b * a.L_win + kr.win_r0 + (j - kr.nsel)) * a.D;
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
constexpr int kAtRows = 32;       // rows per tile
constexpr int kRtPitch = 128;     // bf16 per LDS row of a wave's row copy (256 B, swizzled)

// The wave's copy of a tile row (its 256-byte slice, sixteen 16-byte chunks)
// stores chunk c at position c ^ rt_swz(row): the 16-byte stash writes of 16
// consecutive rows and the 8-byte transposing reads of 4 consecutive rows
// then fall on distinct LDS banks.
__device__ __forceinline__ int rt_swz(int row) { return (4 * row + (row >> 2)) & 15; }

constexpr int kAtMaxSplitRows = 4096;  // rows of a multi-tile CSA split (LDS index stage)
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t* lds_s16x4_ptr;
constexpr int kAtD = 512;
constexpr int kAtH = 64;

// Value of lane (l ^ 32): the two halves of the wave swap through
// v_permlane32_swap (a VALU move; no LDS round trip).
__device__ __forceinline__ float half_swap(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(__lane_id() < 32 ? r[1] : r[0]);
}

// CSA: rows come from the selected index list (else every visible entry).
// MULTI: a split may hold more than one 32-row tile (else exactly one, and
// the kernel is straight-line code with no prefetch).
template <bool CSA, bool MULTI>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_mfma(AttnArgs a) {
  __shared__ float s_cos[kAtD / 2], s_sin[kAtD / 2];
  __shared__ __attribute__((aligned(16))) f32x4_t sx[2][4][2][4][64];  // [buf][wave][ht][rq][lane]
  __shared__ __attribute__((aligned(16))) bf16_t rt[4][kAtRows * kRtPitch];
  __shared__ int32_t s_idx[MULTI && CSA ? kAtMaxSplitRows : 1];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int j = lane & 31, g = lane >> 5;
  const int qi = blockIdx.y, sp = blockIdx.x, S = gridDim.x;
  const int b = qi / a.Tq, t = qi - b * a.Tq;
  const int R = a.R;
  const int rope0 = kAtD - R;
  // Channel ownership: lane (g, j) of wave w holds, in its slot s (0..7),
  // 8 consecutive channels of row / head j (+32); the wave's local channel
  // 64g + 8s + e (its LDS row copy, its PV rows) is global channel
  // 8 * blk(s, g) + e.  Multi-tile splits stream rows, and there each lane
  // reads one contiguous 128-byte stretch (blocks 16w + 8g + s).  A
  // single-tile split is latency-bound instead, and there the blocks are
  // 8s + 2w + g: the eight lane groups each own one block of every
  // 64-channel stretch, so the rope channels at the end of the row are
  // spread over all of them rather than piled on one half-wave, whose
  // rotation would otherwise hold up the whole workgroup.
  auto blk = [&](int s, int gg) { return MULTI ? 16 * wave + 8 * gg + s : 8 * s + 2 * wave + gg; };
  auto chan = [&](int s) { return 8 * blk(s, g); };

  // ---- Every global load below is unconditional (clamped or redirected
  // addresses), so the compiler can count outstanding loads exactly and
  // waits only for the one it needs.  Order: the selected indices of tiles
  // 0 and 1 (the row loads wait on them), the query slice, then tile 0's
  // rows.  A CSA split covers a fixed range of the list [K selected rows,
  // then up to min(W, L_win) window rows], so its bounds are known before
  // the query position is.
  int start = 0, end = 0;
  if (CSA) {
    const int wc = (a.W > 0 && a.L_win > 0) ? min(a.W, a.L_win) : 0;
    const int Lmax = a.K + wc;
    const int per = (((Lmax + S - 1) / S) + kAtRows - 1) / kAtRows * kAtRows;
    start = min(Lmax, sp * per);
    end = min(Lmax, start + per);
  }
  // selected index of this lane's row at list position j0 + j (a harmless
  // word when there is none: a position past K, or K == 0)
  const bool has_idx = CSA && a.K > 0;
  const int32_t* idx_q = has_idx ? a.idx + (int64_t)qi * a.K : (const int32_t*)a.q_pos0;
  auto load_idx = [&](int j0) -> int32_t {
    return idx_q[has_idx ? min(max(j0 + j, 0), a.K - 1) : 0];
  };
  const int32_t idx0 = CSA ? load_idx(start) : 0;  // tile 0
  bf16x8_t qb[2][8];
#pragma unroll
  for (int ht = 0; ht < 2; ++ht) {
    const bf16_t* qp = (const bf16_t*)a.q + ((int64_t)qi * kAtH + ht * 32 + j) * kAtD;
#pragma unroll
    for (int s = 0; s < 8; ++s) qb[ht][s] = *reinterpret_cast<const bf16x8_t*>(qp + chan(s));
  }
  const bf16_t* q_slice = (const bf16_t*)a.q + ((int64_t)qi * kAtH + j) * kAtD;
  const int64_t tpos = a.q_pos0[b] + t;
  const KeyRange kr = key_range(a, b, qi, tpos);
  if (!CSA) {
    const int L = kr.nsel + kr.nwin;
    const int per = (((L + S - 1) / S) + kAtRows - 1) / kAtRows * kAtRows;
    start = min(L, sp * per);
    end = min(L, start + per);
  }

  // Row at list position j0 + j into this wave's operand registers (its 128
  // channels of the row).  An absent row (empty index slot, window row
  // beyond the buffer, or past the split) reads the lane's own query slice
  // instead: `valid` masks it out of the softmax, so its (finite) values
  // meet a zero weight in the PV product.
  const bf16_t* pool_b = (const bf16_t*)a.pool + (int64_t)b * a.N_cap * kAtD;
  const bf16_t* win_b = (const bf16_t*)a.win + ((int64_t)b * a.L_win + kr.win_r0) * kAtD;
  auto load_rows = [&](int j0, int sidx, bf16x8_t(&dst)[8], bool& valid) {
    const int jj = j0 + j;
    const bool in_sel = jj < kr.nsel;
    const int srow = CSA ? sidx : jj;
    const int wrow = jj - kr.nsel;
    valid = jj < end && (in_sel ? (srow >= 0 && srow < a.N_cap) : wrow < kr.nwin);
    const bf16_t* pb = pool_b;  // values, so the selects below are of pointers, not of
    const bf16_t* wb = win_b;   // the captured variables (which would put them in scratch)
    const bf16_t* p = (in_sel ? pb : wb) + (int64_t)(in_sel ? srow : wrow) * kAtD;
    p = valid ? p : q_slice;
#pragma unroll
    for (int s = 0; s < 8; ++s) dst[s] = *reinterpret_cast<const bf16x8_t*>(p + chan(s));
  };

  // rope table at +tpos (computed while tile 0's indices are in flight)
  for (int p = tid; p < R / 2; p += 256) rope_cos_sin(tpos, p, a.rope_theta1, s_cos[p], s_sin[p]);

  bf16x8_t ra[8];
  bool va = false;
  load_rows(start, idx0, ra, va);
  if constexpr (MULTI && CSA) {
    // later tiles' indices, staged once for the whole split (after tile 0's
    // rows are requested: waiting on these loads then costs nothing extra)
    const int sel_end = min(end, a.K);
    for (int jj = start + kAtRows + tid; jj < sel_end; jj += 256)
      s_idx[jj - start] = a.idx[(int64_t)qi * a.K + jj];
  }
  __syncthreads();  // rope table, staged indices

  // rotate the query's rope channels at +tpos: only the lane's slots that
  // reach the rope part
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int c0 = chan(s);
    if (c0 + 8 <= rope0) continue;
    float cs[4], sn[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c = c0 + 2 * k;
      const int pj = max(c - rope0, 0) >> 1;
      const bool rot = c >= rope0;
      cs[k] = rot ? s_cos[pj] : 1.f;
      sn[k] = rot ? s_sin[pj] : 0.f;
    }
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
      const u32x4_t w = __builtin_bit_cast(u32x4_t, qb[ht][s]);
      u32x4_t pk;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float x0 = __uint_as_float(w[k] << 16), x1 = __uint_as_float(w[k] & 0xffff0000u);
        pk[k] = pack_bf16x2(x0 * cs[k] - x1 * sn[k], x0 * sn[k] + x1 * cs[k]);
      }
      qb[ht][s] = __builtin_bit_cast(bf16x8_t, pk);
    }
  }

  float mrun[2] = {-INFINITY, -INFINITY}, lrun[2] = {0.f, 0.f};
  f32x16_t oacc[4][2];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) oacc[dt][ht] = f32x16_t{};
  const float sl2 = a.scale * kLog2e;
  bf16_t* myrt = rt[wave];

  int buf = 0;
  for (int j0 = start; j0 < end; j0 += kAtRows) {
    // partial logits over this wave's 128 channels
    f32x16_t s0 = {}, s1 = {};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[s], qb[0][s], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[s], qb[1][s], s1, 0, 0, 0);
    }
    // wave-private copy of the rows for the transposed PV operand
#pragma unroll
    for (int s = 0; s < 8; ++s)
      *reinterpret_cast<bf16x8_t*>(&myrt[j * kRtPitch + 8 * ((8 * g + s) ^ rt_swz(j))]) = ra[s];
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      sx[buf][wave][0][rq][lane] = f32x4_t{s0[4 * rq], s0[4 * rq + 1], s0[4 * rq + 2], s0[4 * rq + 3]};
      sx[buf][wave][1][rq][lane] = f32x4_t{s1[4 * rq], s1[4 * rq + 1], s1[4 * rq + 2], s1[4 * rq + 3]};
    }
    const uint64_t vmask = __ballot(va);
    // the rows now live in LDS: reuse their registers for the next tile's
    // loads, which then overlap this tile's softmax and PV
    if constexpr (MULTI) {
      if (j0 + kAtRows < end) {
        const int jn = j0 + kAtRows + j;
        const int idx_n = (CSA && jn < min(end, a.K)) ? s_idx[jn - start] : 0;
        load_rows(j0 + kAtRows, idx_n, ra, va);
      }
    }
    __syncthreads();

    float p[2][16];
#pragma unroll
    for (int ht = 0; ht < 2; ++ht)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        f32x4_t x = sx[buf][0][ht][rq][lane];
        x += sx[buf][1][ht][rq][lane];
        x += sx[buf][2][ht][rq][lane];
        x += sx[buf][3][ht][rq][lane];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int n = 8 * rq + 4 * g + e;
          p[ht][4 * rq + e] = ((vmask >> n) & 1) ? x[e] * sl2 : -INFINITY;
        }
      }
    buf ^= 1;

    // Online softmax with a lazily moved reference: a head's running max
    // only moves when a tile exceeds it by more than 2^8 (log2 units), so
    // exp2(s - mrun) stays below 256 and the accumulator is rescaled only on
    // those (rare) tiles.  The first tile with a valid row always moves it.
    float tm[2];
    bool move = false;
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
      float x = p[ht][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) x = fmaxf(x, p[ht][r]);
      tm[ht] = fmaxf(x, half_swap(x));
      move |= tm[ht] > mrun[ht] + 8.f;
    }
    if (__ballot(move)) {
#pragma unroll
      for (int ht = 0; ht < 2; ++ht) {
        const float mnew = fmaxf(mrun[ht], tm[ht]);
        if (mnew > mrun[ht]) {
          const float alpha = exp2f(mrun[ht] - mnew);
          lrun[ht] *= alpha;
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) oacc[dt][ht] *= alpha;
          mrun[ht] = mnew;
        }
      }
    }
    bf16x8_t pb[2][2];
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
      const bool none = mrun[ht] == -INFINITY;  // no valid row seen yet
#pragma unroll
      for (int r = 0; r < 16; ++r) p[ht][r] = none ? 0.f : exp2f(p[ht][r] - mrun[ht]);
      float rs = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) rs += p[ht][r];
      rs += half_swap(rs);
      lrun[ht] += rs;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        u32x4_t pk;
        pk.x = pack_bf16x2(p[ht][8 * ks + 0], p[ht][8 * ks + 1]);
        pk.y = pack_bf16x2(p[ht][8 * ks + 2], p[ht][8 * ks + 3]);
        pk.z = pack_bf16x2(p[ht][8 * ks + 4], p[ht][8 * ks + 5]);
        pk.w = pack_bf16x2(p[ht][8 * ks + 6], p[ht][8 * ks + 7]);
        pb[ht][ks] = __builtin_bit_cast(bf16x8_t, pk);
      }
    }

    // O^T[channel][head] += R^T[channel][row] P^T[row][head].  The R^T
    // operand comes from ds_read_b64_tr_b16: in each 16-lane group, lane c
    // points at 4 consecutive channels of row (c / 4) of a 4-row block and
    // lane i receives channel i of all 4 rows, i.e. 4 consecutive K slots of
    // its own M row; two reads (rows +0..3 and +8..11) make one operand.
    const int tr_row = 4 * g + ((lane & 15) >> 2);
    const int tr_q = lane & 3;
    const int tr_h = (lane >> 4) & 1;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const int chunk = dt * 4 + 2 * tr_h + (tr_q >> 1);   // 16-byte chunk of the channel
      const int sub = 4 * (tr_q & 1);                       // bf16 offset inside it
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int r0 = 16 * ks + tr_row, r1 = r0 + 8;
        const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4_ptr)(&myrt[r0 * kRtPitch + 8 * (chunk ^ rt_swz(r0)) + sub]));
        const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4_ptr)(&myrt[r1 * kRtPitch + 8 * (chunk ^ rt_swz(r1)) + sub]));
        const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
        const bf16x8_t av = __builtin_bit_cast(bf16x8_t, u32x4_t{l2.x, l2.y, h2.x, h2.y});
#pragma unroll
        for (int ht = 0; ht < 2; ++ht)
          oacc[dt][ht] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[ht][ks], oacc[dt][ht], 0, 0, 0);
      }
    }
  }

  // ---- epilogue.  Accumulator element (dt, rq, e) of lane (g, j) is the
  // wave's local channel 32dt + 8rq + 4g + e, i.e. global channel
  // out_chan(dt, rq) + e (4 consecutive channels).
  auto out_chan = [&](int dt, int rq) {
    const int sl = 4 * (dt & 1) + rq;  // slot and lane half of the local channel
    return 8 * blk(sl, dt >> 1) + 4 * g;
  };
  if (S == 1) {
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
      const int h = ht * 32 + j;
      const float skl2 = a.sink[h] * kLog2e;
      const float mf = fmaxf(mrun[ht], skl2);
      const float lf = lrun[ht] * exp2f(mrun[ht] - mf) + exp2f(skl2 - mf);
      const float fac = exp2f(mrun[ht] - mf) / lf;
      if (wave == 0 && g == 0 && a.lse) a.lse[(int64_t)qi * kAtH + h] = (mf + log2f(lf)) * kLn2;
      bf16_t* op = (bf16_t*)a.out + ((int64_t)qi * kAtH + h) * kAtD;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          float o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = oacc[dt][ht][4 * rq + e] * fac;
          const int c = out_chan(dt, rq);
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
          uint2 pk;
          pk.x = pack_bf16x2(o[0], o[1]);
          pk.y = pack_bf16x2(o[2], o[3]);
          *reinterpret_cast<uint2*>(op + c) = pk;
        }
      }
    }
  } else {
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
      const int h = ht * 32 + j;
      const int64_t slot = ((int64_t)qi * S + sp) * kAtH + h;
      if (wave == 0 && g == 0) {
        a.part_ml[2 * slot] = mrun[ht];
        a.part_ml[2 * slot + 1] = lrun[ht];
      }
      // the output's rope slice is rotated back by -tpos here (the rotation
      // is linear, so the merge of the splits commutes with it)
      float* po = a.part_o + slot * kAtD;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          float o[4] = {oacc[dt][ht][4 * rq], oacc[dt][ht][4 * rq + 1], oacc[dt][ht][4 * rq + 2],
                        oacc[dt][ht][4 * rq + 3]};
          const int c = out_chan(dt, rq);
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
          *reinterpret_cast<f32x4_t*>(po + c) = f32x4_t{o[0], o[1], o[2], o[3]};
        }
    }
  }
}

// Merge of the key-range splits: partial maxima are in log2 units of the
// scaled logits, partial sums and outputs unnormalised (outputs already
// rotated back by -tpos on their rope slice).  grid (B*Tq, H),
// 128 threads of 4 channels each (the 512-wide Flash rows).  The partial
// outputs of the first kCbPre splits are requested before the per-split
// weights are known, so the two dependent reads overlap; the weights go
// through LDS.
constexpr int kMaxSplits = 256;
constexpr int kCbPre = 16;

template <typename T>
__global__ __launch_bounds__(128) void attn_combine(AttnArgs a) {
  __shared__ float s_w[kMaxSplits];
  __shared__ float s_lse;
  const int qi = blockIdx.x, h = blockIdx.y;
  const int S = a.splits;
  const int64_t slot0 = (int64_t)qi * S * a.H + h;
  const int c = threadIdx.x * 4;
  const float* po = a.part_o + slot0 * kAtD + c;
  const int64_t sstride = (int64_t)a.H * kAtD;
  f32x4_t v[kCbPre];
#pragma unroll
  for (int u = 0; u < kCbPre; ++u)
    v[u] = u < S ? *reinterpret_cast<const f32x4_t*>(po + u * sstride) : f32x4_t{0.f, 0.f, 0.f, 0.f};
  if (threadIdx.x < 64) {  // one wave merges the (max, sum) pairs
    const int lane = threadIdx.x;
    const float skl2 = a.sink[h] * kLog2e;
    float M = skl2;
    for (int s = lane; s < S; s += 64) M = fmaxf(M, a.part_ml[2 * (slot0 + (int64_t)s * a.H)]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    float Ls = 0.f;
    for (int s = lane; s < S; s += 64) {
      const int64_t sl = slot0 + (int64_t)s * a.H;
      Ls += a.part_ml[2 * sl + 1] * exp2f(a.part_ml[2 * sl] - M);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) Ls += __shfl_xor(Ls, off);
    Ls += exp2f(skl2 - M);
    const float inv = 1.f / Ls;
    for (int s = lane; s < S; s += 64)
      s_w[s] = exp2f(a.part_ml[2 * (slot0 + (int64_t)s * a.H)] - M) * inv;
    if (lane == 0) s_lse = (M + log2f(Ls)) * kLn2;
  }
  __syncthreads();
  if (threadIdx.x == 0 && a.lse) a.lse[(int64_t)qi * a.H + h] = s_lse;
  f32x4_t o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < kCbPre; ++u)
    if (u < S) o += s_w[u] * v[u];
  for (int s = kCbPre; s < S; s += 8) {
    f32x4_t w8[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      w8[u] = s + u < S ? *reinterpret_cast<const f32x4_t*>(po + (s + u) * sstride) : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (s + u < S) o += s_w[s + u] * w8[u];
  }
  float r[4] = {o[0], o[1], o[2], o[3]};
  T* op = (T*)a.out + ((int64_t)qi * a.H + h) * kAtD + c;
#pragma unroll
  for (int e = 0; e < 4; ++e) Elem<T>::put(op + e, r[e]);
}

// ------------------------------------------------------------------- launch
bool attn_uses_mfma(int dt, int H, int D, int R) {
  return dt == 1 && H == kAtH && D == kAtD && R % 2 == 0 && R <= D;
}

int attn_splits(int dt, int B, int Tq, int H, int D, int keys_per_query) {
  if (!(dt == 1 && H == kAtH && D == kAtD)) return 1;
  const int64_t q = (int64_t)B * Tq;
  const int tiles = (keys_per_query + kAtRows - 1) / kAtRows;
  // few queries: spread each one's tiles over splits until there are about
  // as many workgroups as compute units (one tile per split at most)
  int s = 1;
  if (q < 256 && tiles >= 2) s = min((int)((256 + q - 1) / q), tiles);
  // a multi-tile split holds at most kAtMaxSplitRows rows (its CSA index
  // stage lives in LDS)
  s = max(s, (keys_per_query + kAtMaxSplitRows - 1) / kAtMaxSplitRows);
  return min(s, kMaxSplits);
}

size_t attn_ws_bytes(int dt, int B, int Tq, int H, int D, int keys_per_query) {
  const int s = attn_splits(dt, B, Tq, H, D, keys_per_query);
  if (s <= 1) return 0;
  return (size_t)B * Tq * s * H * ((size_t)D + 2) * sizeof(float);
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

hipError_t launch_attn(const AttnArgs& a, hipStream_t stream) {
  if (a.B * a.Tq == 0) return hipSuccess;
  if (attn_uses_mfma(a.dt, a.H, a.D, a.R)) {
    dim3 grid(a.splits, a.B * a.Tq);
    // most rows a split can hold: the list length bound over the split count
    const int wc = (a.W > 0 && a.L_win > 0) ? min(a.W, a.L_win) : 0;
    const int64_t lmax = (a.csa ? (int64_t)a.K : (int64_t)a.N_cap) + wc;
    const bool multi = (lmax + a.splits - 1) / a.splits > kAtRows;
    if (a.csa) {
      if (multi) hipLaunchKernelGGL((attn_mfma<true, true>), grid, dim3(256), 0, stream, a);
      else hipLaunchKernelGGL((attn_mfma<true, false>), grid, dim3(256), 0, stream, a);
    } else {
      if (multi) hipLaunchKernelGGL((attn_mfma<false, true>), grid, dim3(256), 0, stream, a);
      else hipLaunchKernelGGL((attn_mfma<false, false>), grid, dim3(256), 0, stream, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.splits == 1) return e;
    hipLaunchKernelGGL(attn_combine<bf16_t>, dim3(a.B * a.Tq, a.H), dim3(128), 0, stream, a);
    return hipGetLastError();
  }
  if (a.dt == 1) return launch_generic<bf16_t>(a, stream);
  return launch_generic<float>(a, stream);
}

}  // namespace csa
