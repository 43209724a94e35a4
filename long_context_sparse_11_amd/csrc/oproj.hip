// Grouped low-rank output projection ("DeepSeek-v4 Beyond Basics" section
// 3.3, after eq. 26; "DeepSeek V4 Inside: One Token Through Every Block",
// "What does layer 0 sliding-window attention do to p?"; Hugging Face
// "DeepSeek-V4", "Arsitektur"): the H head outputs of a token are split into
// G groups of consecutive heads, each group's concatenation is projected to
// r intermediate channels, and the G intermediates, concatenated, are
// projected to the hidden size.
//
// Decode-sized token counts (T <= 16): every weight is read once, so the two
// products stream their weights from HBM.  One kernel serves both:
// y[t, g, n] = sum_k x[t, g, k] w[g, n, k] on v_mfma_f32_16x16x32_bf16 with
// A = 16 weight rows and B = the (up to 16) tokens; the intermediates are
// rounded to bf16 between the two launches.
#include "kernels.h"

namespace csa {

constexpr int kPjRows = 16;   // output rows per workgroup
constexpr int kPjStep = 128;  // contraction per wave step (4 MFMAs of 32)

// grid (N / 16, G); NW waves split K evenly (K % (NW * 128) == 0).  Lane l
// serves weight row (l & 15) and token (l & 15); its quarter q = l >> 4 holds
// the step's channels 32q .. 32q + 31, so a row's 128 channels are one
// 256-byte read by four lanes.  MFMA s takes channels 32q + 8s .. + 7 from
// both operands (the same map on A and B, so the contraction covers each
// channel once).  Lane l's accumulator element i is row 4q + i, token l & 15.
// The NW partial tiles meet in LDS (a fixed order: deterministic).
template <int NW>
__global__ __launch_bounds__(64 * NW) void proj_rows(const bf16_t* x, int64_t x_tstride,
                                                     const bf16_t* w, bf16_t* y,
                                                     int64_t y_tstride, int T, int N, int K) {
  __shared__ float part[NW][256];
  const int g = blockIdx.y, n0 = blockIdx.x * kPjRows;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, q = lane >> 4;
  const int kw = K / NW;
  const int kb = wave * kw + 32 * q;
  const bf16_t* wp = w + ((int64_t)g * N + n0 + r) * K + kb;
  // tokens past T read token T - 1 (always there) and feed zeros
  const bf16_t* xp = x + (int64_t)min(r, T - 1) * x_tstride + (int64_t)g * K + kb;
  const bool tok = r < T;
  const int steps = kw / kPjStep;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  uint4 wa[4], xa[4], wb[4], xb[4];
  auto load = [&](int st, uint4(&wv)[4], uint4(&xv)[4]) {
    const uint4* a = reinterpret_cast<const uint4*>(wp + (int64_t)st * kPjStep);
    const uint4* b = reinterpret_cast<const uint4*>(xp + (int64_t)st * kPjStep);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      wv[s] = a[s];
      xv[s] = b[s];
    }
  };
  auto mma = [&](const uint4(&wv)[4], const uint4(&xv)[4]) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint4 xs = tok ? xv[s] : make_uint4(0u, 0u, 0u, 0u);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, wv[s]),
                                                    __builtin_bit_cast(bf16x8_t, xs), acc, 0, 0,
                                                    0);
    }
  };
  // two steps in turn; the next step's loads are issued before the current
  // step's MFMAs (past the end they re-read the last step, never used)
  load(0, wa, xa);
  for (int st = 0; st < steps; st += 2) {
    load(min(st + 1, steps - 1), wb, xb);
    mma(wa, xa);
    if (st + 1 >= steps) break;
    load(min(st + 2, steps - 1), wa, xa);
    mma(wb, xb);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) part[wave][i * 64 + lane] = acc[i];
  __syncthreads();
  if (threadIdx.x < 256) {
    const int i = threadIdx.x >> 6, l = threadIdx.x & 63;
    float sum = 0.f;
#pragma unroll
    for (int v = 0; v < NW; ++v) sum += part[v][threadIdx.x];
    const int t = l & 15, n = n0 + 4 * (l >> 4) + i;
    if (t < T) y[(int64_t)t * y_tstride + (int64_t)g * N + n] = (bf16_t)f32_to_bf16(sum);
  }
}

bool out_proj_supported(const OprojArgs& a) {
  const int ka = (a.H / a.G) * a.D, kb = a.G * a.r;
  return a.T >= 1 && a.T <= kOprojMaxTokens && a.H % a.G == 0 && ka % (4 * kPjStep) == 0 &&
         kb % (8 * kPjStep) == 0 && a.r % kPjRows == 0 && a.d % kPjRows == 0;
}

hipError_t launch_out_proj(const OprojArgs& a, hipStream_t stream) {
  const int ka = (a.H / a.G) * a.D, kb = a.G * a.r;
  // o [T, H, D] seen as [T, G, ka] (a group's heads are consecutive)
  hipLaunchKernelGGL(proj_rows<4>, dim3(a.r / kPjRows, a.G), dim3(256), 0, stream,
                     (const bf16_t*)a.o, (int64_t)a.H * a.D, (const bf16_t*)a.w_a, (bf16_t*)a.mid,
                     (int64_t)kb, a.T, a.r, ka);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(proj_rows<8>, dim3(a.d / kPjRows, 1), dim3(512), 0, stream,
                     (const bf16_t*)a.mid, (int64_t)kb, (const bf16_t*)a.w_b, (bf16_t*)a.out,
                     (int64_t)a.d, a.T, a.d, kb);
  return hipGetLastError();
}

}  // namespace csa
