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
      rope_cos_sin(tpos, (c - (D - R)) >> 1, R, a.rope_base, cs[k], sn[k]);
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
constexpr int kRtPitch = 136;     // bf16 per LDS row of the transposition copy (272 B)
constexpr int kAtD = 512;
constexpr int kAtH = 64;

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_mfma(AttnArgs a) {
  __shared__ float s_cos[kAtD / 2], s_sin[kAtD / 2];
  __shared__ __attribute__((aligned(16))) f32x4_t sx[2][4][2][4][64];  // [buf][wave][ht][rq][lane]
  __shared__ __attribute__((aligned(16))) bf16_t rt[4][kAtRows * kRtPitch];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int j = lane & 31, g = lane >> 5;
  const int qi = blockIdx.y, sp = blockIdx.x, S = gridDim.x;
  const int b = qi / a.Tq, t = qi - b * a.Tq;
  const int64_t tpos = a.q_pos0[b] + t;
  const int R = a.R;
  const int rope0 = kAtD - R;

  for (int p = tid; p < R / 2; p += 256) rope_cos_sin(tpos, p, R, a.rope_base, s_cos[p], s_sin[p]);

  const KeyRange kr = key_range(a, b, qi, tpos);
  const int L = kr.nsel + kr.nwin;
  const int per = (((L + S - 1) / S) + kAtRows - 1) / kAtRows * kAtRows;
  const int start = min(L, sp * per);
  const int end = min(L, start + per);
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

  bf16x8_t ra[8], rn[8];
  bool va = false, vn = false;
  auto load_rows = [&](int j0, bf16x8_t(&dst)[8], bool& valid) {
    const int jj = j0 + j;
    bool rv;
    const bf16_t* p = key_row<bf16_t>(a, b, qi, kr, jj < end ? jj : start, rv);
    valid = rv && jj < end;
    p += fbase;
#pragma unroll
    for (int s = 0; s < 8; ++s) dst[s] = *reinterpret_cast<const bf16x8_t*>(p + 8 * s);
  };

  int buf = 0;
  if (start < end) load_rows(start, ra, va);
  for (int j0 = start; j0 < end; j0 += kAtRows) {
    const bool more = j0 + kAtRows < end;
    if (more) load_rows(j0 + kAtRows, rn, vn);

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
      *reinterpret_cast<bf16x8_t*>(&myrt[j * kRtPitch + g * 64 + 8 * s]) = ra[s];
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      sx[buf][wave][0][rq][lane] = f32x4_t{s0[4 * rq], s0[4 * rq + 1], s0[4 * rq + 2], s0[4 * rq + 3]};
      sx[buf][wave][1][rq][lane] = f32x4_t{s1[4 * rq], s1[4 * rq + 1], s1[4 * rq + 2], s1[4 * rq + 3]};
    }
    const uint64_t vmask = __ballot(va);
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

    bf16x8_t pb[2][2];
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
      float tm = p[ht][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) tm = fmaxf(tm, p[ht][r]);
      tm = fmaxf(tm, __shfl_xor(tm, 32));
      const float mnew = fmaxf(mrun[ht], tm);
      float alpha = 1.f;
      if (mnew == -INFINITY) {
#pragma unroll
        for (int r = 0; r < 16; ++r) p[ht][r] = 0.f;
      } else {
        alpha = exp2f(mrun[ht] - mnew);
#pragma unroll
        for (int r = 0; r < 16; ++r) p[ht][r] = exp2f(p[ht][r] - mnew);
      }
      float rs = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) rs += p[ht][r];
      rs += __shfl_xor(rs, 32);
      lrun[ht] = lrun[ht] * alpha + rs;
      mrun[ht] = mnew;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) oacc[dt][ht] *= alpha;
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

    // O^T[channel][head] += R^T[channel][row] P^T[row][head]
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const int col = dt * 32 + j;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int n0 = 16 * ks + 4 * g;
        uint32_t w4[4];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const uint32_t lo = myrt[(n0 + 2 * e) * kRtPitch + col];
          const uint32_t hi = myrt[(n0 + 2 * e + 1) * kRtPitch + col];
          w4[e] = lo | (hi << 16);
          const uint32_t lo2 = myrt[(n0 + 8 + 2 * e) * kRtPitch + col];
          const uint32_t hi2 = myrt[(n0 + 8 + 2 * e + 1) * kRtPitch + col];
          w4[2 + e] = lo2 | (hi2 << 16);
        }
        const bf16x8_t av = __builtin_bit_cast(bf16x8_t, u32x4_t{w4[0], w4[1], w4[2], w4[3]});
#pragma unroll
        for (int ht = 0; ht < 2; ++ht)
          oacc[dt][ht] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[ht][ks], oacc[dt][ht], 0, 0, 0);
      }
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) ra[s] = rn[s];
    va = vn;
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
// 128 threads, 4 channels per thread per step.
template <typename T>
__global__ __launch_bounds__(128) void attn_combine(AttnArgs a) {
  const int qi = blockIdx.x, h = blockIdx.y;
  const int S = a.splits, D = a.D, R = a.R;
  const int b = qi / a.Tq, t = qi - b * a.Tq;
  const int64_t tpos = a.q_pos0[b] + t;
  const float skl2 = a.sink[h] * kLog2e;
  const int64_t slot0 = (int64_t)qi * S * a.H + h;
  float M = skl2;
  for (int s = 0; s < S; ++s) M = fmaxf(M, a.part_ml[2 * (slot0 + (int64_t)s * a.H)]);
  float Ls = exp2f(skl2 - M);
  for (int s = 0; s < S; ++s) {
    const int64_t sl = slot0 + (int64_t)s * a.H;
    Ls += a.part_ml[2 * sl + 1] * exp2f(a.part_ml[2 * sl] - M);
  }
  if (threadIdx.x == 0 && a.lse) a.lse[(int64_t)qi * a.H + h] = (M + log2f(Ls)) * kLn2;
  const float inv = 1.f / Ls;
  for (int c = threadIdx.x * 4; c < D; c += 512) {
    float o[4] = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < S; ++s) {
      const int64_t sl = slot0 + (int64_t)s * a.H;
      const float w = exp2f(a.part_ml[2 * sl] - M) * inv;
      const f32x4_t v = *reinterpret_cast<const f32x4_t*>(a.part_o + sl * D + c);
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] += w * v[e];
    }
#pragma unroll
    for (int e = 0; e < 4; e += 2) {
      if (c + e >= D - R) {
        float cs, sn;
        rope_cos_sin(tpos, (c + e - (D - R)) >> 1, R, a.rope_base, cs, sn);
        const float x0 = o[e], x1 = o[e + 1];
        o[e] = x0 * cs + x1 * sn;
        o[e + 1] = -x0 * sn + x1 * cs;
      }
    }
    T* op = (T*)a.out + ((int64_t)qi * a.H + h) * D + c;
#pragma unroll
    for (int e = 0; e < 4; ++e) Elem<T>::put(op + e, o[e]);
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
  if (q >= 512 || tiles < 4) return 1;
  int s = (int)((512 + q - 1) / q);
  s = min(s, tiles / 2);
  return max(s, 1);
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
