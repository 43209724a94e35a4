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
//               waves per (query, key split).  Wave w owns channels
//               128w .. 128w+127 of every row: it gathers its 256-byte slice
//               of 32 rows per tile straight from HBM into MFMA operands
//               (each row is read once and serves all 64 heads), computes
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

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t* lds_s16x4_ptr;
constexpr int kAtD = 512;
constexpr int kAtH = 64;
constexpr int kAtMaxSplitRows = 4096;  // rows of one key split (LDS index stage)

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_mfma(AttnArgs a) {
  __shared__ float s_cos[kAtD / 2], s_sin[kAtD / 2];
  __shared__ __attribute__((aligned(16))) f32x4_t sx[2][4][2][4][64];  // [buf][wave][ht][rq][lane]
  __shared__ __attribute__((aligned(16))) bf16_t rt[4][kAtRows * kRtPitch];
  __shared__ int32_t s_idx[kAtMaxSplitRows];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int j = lane & 31, g = lane >> 5;
  const int qi = blockIdx.y, sp = blockIdx.x, S = gridDim.x;
  const int b = qi / a.Tq, t = qi - b * a.Tq;
  const int64_t tpos = a.q_pos0[b] + t;
  const int R = a.R;
  const int rope0 = kAtD - R;

  for (int p = tid; p < R / 2; p += 256) rope_cos_sin(tpos, p, a.rope_theta1, s_cos[p], s_sin[p]);

  const KeyRange kr = key_range(a, b, qi, tpos);
  const int L = kr.nsel + kr.nwin;
  const int per = (((L + S - 1) / S) + kAtRows - 1) / kAtRows * kAtRows;
  const int start = min(L, sp * per);
  const int end = min(L, start + per);
  // the split's selected pool indices, staged once (row addresses then need
  // no dependent global load inside the tile loop)
  if (a.csa) {
    const int sel_end = min(end, kr.nsel);
    for (int jj = start + tid; jj < sel_end; jj += 256) s_idx[jj - start] = a.idx[(int64_t)qi * a.K + jj];
  }
  __syncthreads();

  // query operand, rotated at +tpos: lane (g, j) holds head j (+32) at
  // channels fbase + 8s .. +7
  const int fbase = wave * 128 + g * 64;
  bf16x8_t qb[2][8];
#pragma unroll
  for (int ht = 0; ht < 2; ++ht) {
    const bf16_t* qp = (const bf16_t*)a.q + ((int64_t)qi * kAtH + ht * 32 + j) * kAtD + fbase;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      float v[8];
      Elem<bf16_t>::load<8>(qp + 8 * s, v);
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const int c = fbase + 8 * s + e;
        if (c >= rope0) {
          const int pj = (c - rope0) >> 1;
          const float cs = s_cos[pj], sn = s_sin[pj];
          const float x0 = v[e], x1 = v[e + 1];
          v[e] = x0 * cs - x1 * sn;
          v[e + 1] = x0 * sn + x1 * cs;
        }
      }
      u32x4_t pk;
      pk.x = pack_bf16x2(v[0], v[1]);
      pk.y = pack_bf16x2(v[2], v[3]);
      pk.z = pack_bf16x2(v[4], v[5]);
      pk.w = pack_bf16x2(v[6], v[7]);
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

  bf16x8_t ra[8];
  bool va = false;
  auto load_rows = [&](int j0, bf16x8_t(&dst)[8], bool& valid) {
    const int jj = j0 + j;
    const int jr = jj < end ? jj : start;
    const bf16_t* p;
    bool rv = true;
    if (jr < kr.nsel) {
      int srow = jr;
      if (a.csa) {
        srow = s_idx[jr - start];
        rv = srow >= 0 && srow < a.N_cap;
        if (!rv) srow = 0;
      }
      p = (const bf16_t*)a.pool + ((int64_t)b * a.N_cap + srow) * kAtD;
    } else {
      p = (const bf16_t*)a.win + ((int64_t)b * a.L_win + kr.win_r0 + (jr - kr.nsel)) * kAtD;
    }
    valid = rv && jj < end;
    p += fbase;
#pragma unroll
    for (int s = 0; s < 8; ++s) dst[s] = *reinterpret_cast<const bf16x8_t*>(p + 8 * s);
  };

  int buf = 0;
  if (start < end) load_rows(start, ra, va);
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
    if (j0 + kAtRows < end) load_rows(j0 + kAtRows, ra, va);
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
      tm[ht] = fmaxf(x, __shfl_xor(x, 32));
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
      rs += __shfl_xor(rs, 32);
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

  // ---- epilogue
  if (S == 1) {
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
      const int h = ht * 32 + j;
      const float skl2 = a.sink[h] * kLog2e;
      const float mf = fmaxf(mrun[ht], skl2);
      const float lf = lrun[ht] * exp2f(mrun[ht] - mf) + exp2f(skl2 - mf);
      const float fac = exp2f(mrun[ht] - mf) / lf;
      if (wave == 0 && g == 0 && a.lse) a.lse[(int64_t)qi * kAtH + h] = (mf + log2f(lf)) * kLn2;
      bf16_t* op = (bf16_t*)a.out + ((int64_t)qi * kAtH + h) * kAtD + wave * 128;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          float o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = oacc[dt][ht][4 * rq + e] * fac;
          const int c = wave * 128 + dt * 32 + 8 * rq + 4 * g;
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
          *reinterpret_cast<uint2*>(op + dt * 32 + 8 * rq + 4 * g) = pk;
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
      float* po = a.part_o + slot * kAtD + wave * 128;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq)
          *reinterpret_cast<f32x4_t*>(po + dt * 32 + 8 * rq + 4 * g) =
              f32x4_t{oacc[dt][ht][4 * rq], oacc[dt][ht][4 * rq + 1], oacc[dt][ht][4 * rq + 2],
                      oacc[dt][ht][4 * rq + 3]};
    }
  }
}

// Merge of the key-range splits: partial maxima are in log2 units of the
// scaled logits, partial sums and outputs unnormalised.  grid (B*Tq, H),
// 128 threads, 4 channels per thread per step.  The per-split weights are
// computed once into LDS; the split loop is unrolled so the loads of several
// splits are in flight together.
constexpr int kMaxSplits = 256;

template <typename T>
__global__ __launch_bounds__(128) void attn_combine(AttnArgs a) {
  __shared__ float s_w[kMaxSplits];
  __shared__ float s_lse;
  const int qi = blockIdx.x, h = blockIdx.y;
  const int S = a.splits, D = a.D, R = a.R;
  const int b = qi / a.Tq, t = qi - b * a.Tq;
  const int64_t tpos = a.q_pos0[b] + t;
  const int64_t slot0 = (int64_t)qi * S * a.H + h;
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
  for (int c = threadIdx.x * 4; c < D; c += 512) {
    f32x4_t o = {0.f, 0.f, 0.f, 0.f};
    int s = 0;
    for (; s + 8 <= S; s += 8) {
      f32x4_t v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        v[u] = *reinterpret_cast<const f32x4_t*>(a.part_o + (slot0 + (int64_t)(s + u) * a.H) * D + c);
#pragma unroll
      for (int u = 0; u < 8; ++u) o += s_w[s + u] * v[u];
    }
    for (; s < S; ++s)
      o += s_w[s] * *reinterpret_cast<const f32x4_t*>(a.part_o + (slot0 + (int64_t)s * a.H) * D + c);
    float r[4] = {o[0], o[1], o[2], o[3]};
#pragma unroll
    for (int e = 0; e < 4; e += 2) {
      if (c + e >= D - R) {
        float cs, sn;
        rope_cos_sin(tpos, (c + e - (D - R)) >> 1, a.rope_theta1, cs, sn);
        const float x0 = r[e], x1 = r[e + 1];
        r[e] = x0 * cs + x1 * sn;
        r[e + 1] = -x0 * sn + x1 * cs;
      }
    }
    T* op = (T*)a.out + ((int64_t)qi * a.H + h) * D + c;
#pragma unroll
    for (int e = 0; e < 4; ++e) Elem<T>::put(op + e, r[e]);
  }
}

// ------------------------------------------------------------------- launch
bool attn_uses_mfma(int dt, int H, int D, int R) {
  return dt == 1 && H == kAtH && D == kAtD && R % 2 == 0 && R <= D;
}

int attn_splits(int dt, int B, int Tq, int H, int D, int keys_per_query) {
  if (!(dt == 1 && H == kAtH && D == kAtD)) return 1;
  const int64_t q = (int64_t)B * Tq;
  const int tiles = (keys_per_query + kAtRows - 1) / kAtRows;
  int s = 1;
  if (q < 256 && tiles >= 4) s = min((int)((256 + q - 1) / q), tiles / 2);
  // a split holds at most kAtMaxSplitRows rows (its index stage lives in LDS)
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
    hipLaunchKernelGGL(attn_mfma, grid, dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.splits == 1) return e;
    hipLaunchKernelGGL(attn_combine<bf16_t>, dim3(a.B * a.Tq, a.H), dim3(128), 0, stream, a);
    return hipGetLastError();
  }
  if (a.dt == 1) return launch_generic<bf16_t>(a, stream);
  return launch_generic<float>(a, stream);
}

}  // namespace csa
