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

// NW: waves per workgroup, 16 heads each.  With NW = 4 the workgroup takes
// all 64 heads and four waves share each copied tile; with NW = 2 (single-
// tile splits of few queries, i.e. decode) it takes 32 heads and blockIdx.z
// is the head group: half the query slice and half the partial output per
// workgroup, twice the workgroups.  A workgroup's rows and partials go
// through one compute unit, whose own rate bounds these short workgroups.
template <bool CSA, bool MULTI, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_hs(AttnArgs a) {
  constexpr int RPW = kHsRows / NW;  // tile rows each wave copies
  // two row buffers as distinct objects: with every access naming a fixed
  // one, the compiler can tell that a copy into one does not touch the other
  // (it would otherwise wait for the copy before reading)
  __shared__ __attribute__((aligned(16))) bf16_t s_rows0[kHsRows * kAtD];
  __shared__ __attribute__((aligned(16))) bf16_t s_rows1[kHsRows * kAtD];
  __shared__ float s_cos[kAtD / 2], s_sin[kAtD / 2];
  __shared__ __attribute__((aligned(16))) int32_t s_idx[MULTI && CSA ? kHsMaxSplitRows : 4];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int c16 = lane & 15, G = lane >> 4;
  const int h = 16 * (NW * (int)blockIdx.z + wave) + c16;  // this lane's head
  const int qi = blockIdx.y, sp = blockIdx.x, S = gridDim.x;
  const int b = qi / a.Tq, t = qi - b * a.Tq;
  const int R = a.R;
  const int rope0 = kAtD - R;

  // ---- split bounds (CSA: a fixed range of [K selected, up to
  // min(W, L_win) window rows], known before the position)
  int start = 0, end = 0;
  if (CSA) {
    const int wc = (a.W > 0 && a.L_win > 0) ? min(a.W, a.L_win) : 0;
    const int Lmax = a.K + wc;
    const int per = (((Lmax + S - 1) / S) + kHsRows - 1) / kHsRows * kHsRows;
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
  const KeyRange kr = key_range(a, b, qi, tpos);
  if (!CSA) {
    const int L = kr.nsel + kr.nwin;
    const int per = (((L + S - 1) / S) + kHsRows - 1) / kHsRows * kHsRows;
    start = min(L, sp * per);
    end = min(L, start + per);
  }
  const bf16_t* pool_b = (const bf16_t*)a.pool + (int64_t)b * a.N_cap * kAtD;
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
  const uint64_t pool_a = (uint64_t)pool_b, win_a = (uint64_t)win_b, dummy_a = (uint64_t)dummy;
  struct TileSrc {
    int lo, hi;  // this lane's row address
    uint32_t mask;
  };
  auto resolve_tile = [&](int j0, int sidx_l) -> TileSrc {
    const int jj = j0 + (lane & 31);
    const bool in_sel = jj < kr.nsel;
    const int srow = CSA ? sidx_l : jj;
    int wrow = jj - kr.nsel + kr.win_r0;  // buffer row; wraps only in a ring
    if (wrow >= a.L_win) wrow -= a.L_win;
    const bool valid =
        lane < 32 && jj < end && (in_sel ? (srow >= 0 && srow < a.N_cap) : jj - kr.nsel < kr.nwin);
    const uint64_t sa = in_sel ? pool_a + (uint64_t)((int64_t)srow * (kAtD * 2))
                               : win_a + (uint64_t)((int64_t)wrow * (kAtD * 2));
    const uint64_t src = valid ? sa : dummy_a;
    return TileSrc{(int)(uint32_t)src, (int)(uint32_t)(src >> 32), (uint32_t)__ballot(valid)};
  };
  auto issue_row = [&](const TileSrc& ts, int u, bf16_t* dst) {
    const int r = RPW * wv + u;
    const uint64_t rs = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(ts.hi, r) << 32) |
                        (uint32_t)__builtin_amdgcn_readlane(ts.lo, r);
    // a buffer load (not a global one): it counts on vmcnt only, so the
    // LDS reads issued around it keep exact lgkmcnt waits
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)rs, (short)0, kAtD * 2, kRawBufferWord3);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_ptr)(dst + r * kAtD), 16,
                                             16 * (lane ^ hs_swz(r)), 0, 0, 0);
  };

  // ---- prologue: tile 0's rows, the rope table, the split's later indices
  uint32_t vmask;
  {
    const TileSrc t0 = resolve_tile(start, idx0);
#pragma unroll
    for (int u = 0; u < RPW; ++u) issue_row(t0, u, s_rows0);
    vmask = t0.mask;
  }
  for (int p = tid; p < R / 2; p += 64 * NW) rope_cos_sin(tpos, p, a.rope_theta1, s_cos[p], s_sin[p]);
  if constexpr (MULTI && CSA) {
    const int sel_end = min(end, a.K);
    for (int jj = start + kHsRows + tid; jj < sel_end; jj += 64 * NW)
      s_idx[jj - start] = a.idx[(int64_t)qi * a.K + jj];
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // rotate the query slice's rope channels at +tpos (each lane its own pairs)
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) {
    const int c0 = 32 * ks + 8 * G;
    if (c0 + 8 <= rope0) continue;
    const u32x4_t w = __builtin_bit_cast(u32x4_t, qb[ks]);
    u32x4_t pk;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c = c0 + 2 * k;
      const bool rot = c >= rope0;
      const int pj = max(c - rope0, 0) >> 1;
      const float cs = rot ? s_cos[pj] : 1.f, sn = rot ? s_sin[pj] : 0.f;
      const float x0 = __uint_as_float(w[k] << 16), x1 = __uint_as_float(w[k] & 0xffff0000u);
      pk[k] = pack_bf16x2(x0 * cs - x1 * sn, x0 * sn + x1 * cs);
    }
    qb[ks] = __builtin_bit_cast(bf16x8_t, pk);
  }

  float mrun = -INFINITY, lrun = 0.f;  // this lane's head (shared by its 4 row groups)
  f32x4_t oacc[32];
#pragma unroll
  for (int cb = 0; cb < 32; ++cb) oacc[cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const float sl2 = a.scale * kLog2e;

  // One tile: logits, softmax, PV from `rows`; in multi-tile splits the
  // next tile's rows are first requested into `next` (the other buffer).
  auto tile_step = [&](int j0, const bf16_t* rows, bf16_t* next) {
    // multi-tile splits request the next tile while this one is used; past
    // the split's end every row is invalid and the copy reads the harmless
    // row into the idle buffer, so the request is unconditional
    TileSrc nt{0, 0, 0u};
    if constexpr (MULTI) {
      const int jn = j0 + kHsRows;
      int sidx_l = 0;
      // row jn + l's selected index; entries past the selected part (or the
      // split) are never used, the clamp only keeps the read inside s_idx
      if constexpr (CSA) sidx_l = s_idx[min(jn - start + (lane & 31), kHsMaxSplitRows - 1)];
      nt = resolve_tile(jn, sidx_l);
    }

    // logits S^T[key][head] over all 512 channels for two 16-key blocks (two
    // independent accumulator chains, interleaved).  The order is pinned:
    // with one wave per SIMD nothing else hides the LDS latency, so the 32
    // operand reads run 8 ahead of their MFMAs, and the next tile's 8 row
    // copies are spread between them instead of stalling issue up front.
    f32x4_t sacc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
    {
      const bf16_t* rpk[2] = {rows + c16 * kAtD, rows + (16 + c16) * kAtD};
      const int swk[2] = {hs_swz(c16), hs_swz(16 + c16)};
      // step f reads block f % 2, channel slice f / 2
      auto qk_read = [&](int f) {
        const int kb = f & 1, ks = f >> 1;
        return *reinterpret_cast<const bf16x8_t*>(rpk[kb] + 128 * (ks >> 2) +
                                                  8 * ((4 * (ks & 3) + G) ^ swk[kb]));
      };
      bf16x8_t av[8];
#pragma unroll
      for (int f = 0; f < 8; ++f) av[f] = qk_read(f);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int f = 0; f < 32; ++f) {
        sacc[f & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[f & 7], qb[f >> 1], sacc[f & 1], 0, 0, 0);
        if (f + 8 < 32) av[f & 7] = qk_read(f + 8);
        if constexpr (MULTI) {
          if (f % (32 / RPW) == 32 / RPW - 1) issue_row(nt, f / (32 / RPW), next);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // online softmax of head h over this tile's 32 keys: lane (G, c16) holds
    // keys 16kb + 4G + r; the other three row groups hold the rest
    float p[2][4];
    float tmx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = 16 * kb + 4 * G + r;
        p[kb][r] = ((vmask >> key) & 1) ? sacc[kb][r] * sl2 : -INFINITY;
        tmx = fmaxf(tmx, p[kb][r]);
      }
    tmx = fmaxf(tmx, row_swap16(tmx));
    tmx = fmaxf(tmx, half_swap(tmx));
    // lazily moved reference: rescale only when the tile max exceeds it by
    // more than 2^8 (log2 units); the first tile with a valid key moves it
    if (__ballot(tmx > mrun + 8.f)) {
      const float mnew = fmaxf(mrun, tmx);
      if (mnew > mrun) {
        const float alpha = exp2f(mrun - mnew);
        lrun *= alpha;
#pragma unroll
        for (int cb = 0; cb < 32; ++cb) oacc[cb] *= alpha;
        mrun = mnew;
      }
    }
    const bool none = mrun == -INFINITY;
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[kb][r] = none ? 0.f : exp2f(p[kb][r] - mrun);
        rs += p[kb][r];
      }
    rs += row_swap16(rs);
    rs += half_swap(rs);
    lrun += rs;
    u32x4_t pk;
    pk.x = pack_bf16x2(p[0][0], p[0][1]);
    pk.y = pack_bf16x2(p[0][2], p[0][3]);
    pk.z = pack_bf16x2(p[1][0], p[1][1]);
    pk.w = pack_bf16x2(p[1][2], p[1][3]);
    const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pk);

    // O^T[ch][head] += R^T[ch][key] P^T[key][head]: in each 16-lane group,
    // lane i points at key row 4G + i/4 (and 16 + 4G + i/4), channels
    // 16cb + 4(i % 4) .. +3, and receives channel 16cb + i of the 4 rows.
    const int kr0 = 4 * G + (c16 >> 2);
    const int kr1 = kr0 + 16;
    const bf16_t* rp0 = rows + kr0 * kAtD;
    const bf16_t* rp1 = rows + kr1 * kAtD;
    const int sw0 = hs_swz(kr0), sw1 = hs_swz(kr1);
    const int q4 = c16 & 3;
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
    // 16 transposing reads (8 channel blocks) ahead, then one MFMA per two
    __builtin_amdgcn_sched_group_barrier(0x100, 16, 1);
#pragma unroll
    for (int i = 0; i < 24; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 1);

    if constexpr (MULTI) {
      // the next tile's rows have landed and every wave is done with this one
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      vmask = nt.mask;
    }
  };

  for (int j0 = start; j0 < end; j0 += 2 * kHsRows) {
    tile_step(j0, s_rows0, s_rows1);
    if (j0 + kHsRows >= end) break;
    tile_step(j0 + kHsRows, s_rows1, s_rows0);
  }

  // ---- epilogue: lane (G, c16) holds channels 16cb + 4G + r of head h
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
    // linear, so the merge of the splits commutes with it)
    float* po = a.part_o + slot * kAtD;
#pragma unroll
    for (int cb = 0; cb < 32; ++cb) {
      float o[4] = {oacc[cb][0], oacc[cb][1], oacc[cb][2], oacc[cb][3]};
      const int c = 16 * cb + 4 * G;
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
    const int hg = a.H / kAtH;  // 64-head groups (grid z)
    dim3 grid(a.splits, a.B * a.Tq, hg);
    // most rows a split can hold: the list length bound over the split count
    const int wc = (a.W > 0 && a.L_win > 0) ? min(a.W, a.L_win) : 0;
    const int64_t lmax = (a.csa ? (int64_t)a.K : (int64_t)a.N_cap) + wc;
    const bool multi = (lmax + a.splits - 1) / a.splits > kHsRows;
    // single-tile splits in head groups of 32 (two waves, grid z) while the
    // doubled grid still fits the compute units once
    const bool halves = !multi && 2LL * hg * a.splits * a.B * a.Tq <= kHsHeadSplitBelow;
    dim3 grid2(a.splits, a.B * a.Tq, 2 * hg), block4(256), block2(128);
    if (a.csa) {
      if (multi) hipLaunchKernelGGL((attn_hs<true, true, 4>), grid, block4, 0, stream, a);
      else if (halves) hipLaunchKernelGGL((attn_hs<true, false, 2>), grid2, block2, 0, stream, a);
      else hipLaunchKernelGGL((attn_hs<true, false, 4>), grid, block4, 0, stream, a);
    } else {
      if (multi) hipLaunchKernelGGL((attn_hs<false, true, 4>), grid, block4, 0, stream, a);
      else if (halves) hipLaunchKernelGGL((attn_hs<false, false, 2>), grid2, block2, 0, stream, a);
      else hipLaunchKernelGGL((attn_hs<false, false, 4>), grid, block4, 0, stream, a);
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
