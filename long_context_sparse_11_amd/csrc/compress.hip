// Token-level compressor: softmax-weighted pooling of m-token blocks (two
// overlapped streams for CSA, one stream for HCA), then optional RMSNorm and
// partial RoPE.  "DeepSeek-v4 Beyond Basics" section 3.2.2 (eqs. 9-12) and
// section 3.3 (eqs. 20-23); RMSNorm/RoPE placement from the same page's
// section 3.3 (its quote of the paper's section 2.3.3).
//
// One workgroup per (sequence, entry).  A row of D channels is covered by
// L = D / VEC lanes holding VEC contiguous channels each (16-byte loads, so
// a row is one coalesced read).  The block's rows are spread over G lane
// groups; each group keeps a per-channel online softmax (max, denominator,
// weighted sum) in registers, the groups are merged through LDS, and group 0
// finishes the entry (normalise, gain, rotate, store).
#include "kernels.h"

namespace csa {

template <typename T, int VEC, int GMAX>
__global__ __launch_bounds__(GMAX * 64) void compress_kernel(CompressArgs a) {
  __shared__ float smem[3 * (GMAX / 2) * 64 * VEC];
  const int i = blockIdx.x;  // entry within the call
  const int b = blockIdx.y;
  const int D = a.D;
  const int L = D / VEC;
  const int G = blockDim.x / L;
  const int tid = threadIdx.x;
  const int g = tid / L;
  const int lane = tid - g * L;
  const int c0 = lane * VEC;
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
    } else if (a.prev_c_b) {
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
        const float sc = exp2f(mx[e] - nm);
        const float p = exp2f(l - nm);
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
  float* s_den = smem + (GMAX / 2) * 64 * VEC;
  float* s_acc = smem + 2 * (GMAX / 2) * 64 * VEC;
  for (int half = G >> 1; half >= 1; half >>= 1) {
    if (g >= half && g < 2 * half) {
      const int o = (g - half) * D + c0;
#pragma unroll
      for (int e = 0; e < VEC; ++e) { s_mx[o + e] = mx[e]; s_den[o + e] = den[e]; s_acc[o + e] = acc[e]; }
    }
    __syncthreads();
    if (g < half) {
      const int o = g * D + c0;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float om = s_mx[o + e];
        const float M = fmaxf(mx[e], om);
        const float w0 = mx[e] == -INFINITY ? 0.f : exp2f(mx[e] - M);
        const float w1 = om == -INFINITY ? 0.f : exp2f(om - M);
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

  const int64_t bstride = a.out_bstride ? a.out_bstride : (int64_t)a.n_out * D;
  T* op = (T*)a.out + (int64_t)b * bstride + (int64_t)i * D + c0;
  Elem<T>::template store<VEC>(op, y);
}

template <typename T, int VEC, int GMAX>
static hipError_t launch_compress_g(const CompressArgs& a, int G, hipStream_t stream) {
  const int L = a.D / VEC;
  dim3 grid(a.n_out, a.B), block(G * L);
  hipLaunchKernelGGL((compress_kernel<T, VEC, GMAX>), grid, block, 0, stream, a);
  return hipGetLastError();
}

// Row groups: about 4 rows per group (one batch of loads each; a merge step
// costs more than streaming 4 more rows), at most 16 groups / 1024 threads,
// at least one full wave; more than 8 groups take the 16-group variant.
template <typename T, int VEC>
static hipError_t launch_compress_t(const CompressArgs& a, hipStream_t stream) {
  const int L = a.D / VEC;
  const int rows = a.m * (a.overlap ? 2 : 1);
  int G = 1;
  while (4 * G < rows && G * L < 1024 && G < 16) G <<= 1;
  while (G * L < 64 && G < 16) G <<= 1;
  if (G <= 8 || VEC > 8) return launch_compress_g<T, VEC, 8>(a, min(G, 8), stream);
  return launch_compress_g<T, VEC, (VEC > 8 ? 8 : 16)>(a, G, stream);
}

hipError_t launch_compress(const CompressArgs& a, hipStream_t stream) {
  if (a.dt == 1) {
    if (a.D <= 512) return launch_compress_t<bf16_t, 8>(a, stream);
    return launch_compress_t<bf16_t, 16>(a, stream);
  }
  if (a.D <= 256) return launch_compress_t<float, 4>(a, stream);
  if (a.D == 512) return launch_compress_t<float, 8>(a, stream);
  return launch_compress_t<float, 16>(a, stream);
}

}  // namespace csa
