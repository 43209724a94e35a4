// Grouped low-rank output projection ("DeepSeek-v4 Beyond Basics" section
// 3.3, after eq. 26; "DeepSeek V4 Inside: One Token Through Every Block",
// "What does layer 0 sliding-window attention do to p?"; Hugging Face
// "DeepSeek-V4", "Arsitektur"): the H head outputs of a token are split into
// G groups of consecutive heads, each group's concatenation is projected to
// r intermediate channels, and the G intermediates, concatenated, are
// projected to the hidden size.
//
// Decode-sized token counts (T <= 16): every weight is read once, so the two
// products stream their weights from HBM (proj_rows); larger token counts
// take a tiled GEMM (proj_gemm).  One kernel serves both:
// y[t, g, n] = sum_k x[t, g, k] w[g, n, k] on v_mfma_f32_16x16x32_bf16 with
// A = 16 weight rows and B = the (up to 16) tokens; the intermediates are
// rounded to bf16 between the two launches.
#include "kernels.h"
#include "oproj.h"

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

// ------------------------------------------------------------ many tokens
// More than 16 tokens (prefill chunks): each weight serves many tokens, so
// the products are ordinary GEMMs, C[t, g, n] = sum_k X[t, g, k] W[g, n, k].
// 1-D grid over the tiles of (group, token tile, weight-row tile), 4 waves
// as 2 x 2 quadrants of (32 MI) tokens x (32 NJ) weight rows;
// v_mfma_f32_32x32x16_bf16 (lane l: A row = token l % 32, B column = weight
// row l % 32, K slots 8 (l / 32) .. + 7; accumulator element e of lane l is
// token 8 (e / 4) + 4 (l / 32) + e % 4, row l % 32).  64-channel steps are
// copied global -> registers -> LDS (double-buffered, one barrier per step);
// the LDS row pitch of 72 bf16 (144 B) puts the 16 rows a 16-byte read
// serves in distinct banks.
//
// Operand reuse.  Per 16 channels a wave reads MI + NJ 16-byte operands from
// LDS for MI x NJ MFMAs.  At MI = NJ = 2 (128 x 128 tiles) that is one read
// per MFMA, more than the LDS delivers to four waves running MFMAs back to
// back; 256 x 256 tiles (MI = NJ = 4, 256 accumulators per lane, 144 KiB of
// LDS, one workgroup per compute unit) halve it.
//
// Tile order.  Workgroup id goes to XCD id % 8, each XCD with its own L2, so
// XCD x takes the contiguous range x * per .. of the logical tiles; within a
// group, logical tiles run over 8 token tiles for each weight-row tile in
// turn, so the workgroups an XCD runs together share their activation and
// weight tiles through its L2 instead of fetching them from HBM each.
constexpr int kGmSwizzle = 8;
constexpr int kGmTile = 128;  // the smallest tile (both sides)
constexpr int kGmK = 64;
constexpr int kGmPitch = 72;

// STAGE only names the launch (0: grouped product, 1: final product), so the
// two show up apart in kernel traces.
template <int STAGE, int MI, int NJ>
__global__ __launch_bounds__(256) void proj_gemm(const bf16_t* x, int64_t x_tstride,
                                                 const bf16_t* w, bf16_t* y, int64_t y_tstride,
                                                 int T, int N, int K, int G) {
  constexpr int TT = 64 * MI, TR = 64 * NJ;  // workgroup tile: tokens x weight rows
  constexpr int CA = TT * 8 / 256, CB = TR * 8 / 256;  // 16-byte chunks per thread and step
  __shared__ __attribute__((aligned(16))) bf16_t sa[2][TT * kGmPitch];  // tokens x k
  __shared__ __attribute__((aligned(16))) bf16_t sb[2][TR * kGmPitch];  // weight rows x k
  const int nt = N / TR, tt = (T + TT - 1) / TT;
  const int total = nt * tt * G, per = (total + 7) / 8;
  const int logical = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
  if (logical >= total) return;  // padding of the last XCD's range (whole workgroup)
  const int g = logical / (nt * tt);
  const int rest = logical - g * nt * tt;
  const int band = rest / (kGmSwizzle * nt);          // 8 token tiles x all row tiles
  const int first_t = band * kGmSwizzle;
  const int rows_t = min(tt - first_t, kGmSwizzle);
  const int in_band = rest - band * kGmSwizzle * nt;
  const int t0 = (first_t + in_band % rows_t) * TT;
  const int n0 = (in_band / rows_t) * TR;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  // copy role: chunk q = tid + 256 i of a tile is row q / 8, channels
  // 8 (q % 8) .. + 7 of the step (one 128-byte row segment per 8 threads).
  // Addresses are a uniform base per chunk plus one 32-bit lane offset per
  // operand (the global loads' scalar-base form: two address registers in
  // all).  Tokens past T re-read token T - 1 and are never stored; the
  // 256 x 256 instance runs only where T divides into its tiles.
  const int ck = (tid & 7) * 8;
  const int rc = tid >> 3;
  const uint32_t la = (uint32_t)(((int64_t)rc * x_tstride + ck) * 2);
  const uint32_t lb = (uint32_t)(((int64_t)rc * K + ck) * 2);
  const char* xbase = reinterpret_cast<const char*>(x + (int64_t)t0 * x_tstride + (int64_t)g * K);
  const char* wbase = reinterpret_cast<const char*>(w + ((int64_t)g * N + n0) * K);
  u32x4_t ra[CA], rb[CB];
  auto fetch = [&](int k0) {
    if constexpr (MI == 2) {
      // the 128-tile instance serves ragged token counts: clamped rows
#pragma unroll
      for (int i = 0; i < CA; ++i)
        ra[i] = *reinterpret_cast<const u32x4_t*>(
            x + (int64_t)min(t0 + rc + 32 * i, T - 1) * x_tstride + (int64_t)g * K + ck + k0);
    } else {
#pragma unroll
      for (int i = 0; i < CA; ++i)
        ra[i] = *reinterpret_cast<const u32x4_t*>(xbase + (int64_t)32 * i * x_tstride * 2 +
                                                  (int64_t)k0 * 2 + la);
    }
#pragma unroll
    for (int i = 0; i < CB; ++i)
      rb[i] = *reinterpret_cast<const u32x4_t*>(wbase + (int64_t)32 * i * K * 2 + (int64_t)k0 * 2 + lb);
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CA; ++i)
      *reinterpret_cast<u32x4_t*>(&sa[buf][((tid >> 3) + 32 * i) * kGmPitch + ck]) = ra[i];
#pragma unroll
    for (int i = 0; i < CB; ++i)
      *reinterpret_cast<u32x4_t*>(&sb[buf][((tid >> 3) + 32 * i) * kGmPitch + ck]) = rb[i];
  };
  f32x16_t c[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) c[i][j] = f32x16_t{};
  const int nk = K / kGmK;
  fetch(0);
  stash(0);
  __syncthreads();
  const int ar = lane & 31, ah = 8 * (lane >> 5);
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    // unconditional: the last step re-reads itself and fills the idle buffer,
    // which nothing reads afterwards
    fetch(min(kt + 1, nk - 1) * kGmK);
#pragma unroll
    for (int ks = 0; ks < kGmK / 16; ++ks) {
      const bf16_t* pa = &sa[buf][(wm * 32 * MI + ar) * kGmPitch + ks * 16 + ah];
      const bf16_t* pb = &sb[buf][(wn * 32 * NJ + ar) * kGmPitch + ks * 16 + ah];
      bf16x8_t av[MI], bv[NJ];
#pragma unroll
      for (int i = 0; i < MI; ++i) av[i] = *reinterpret_cast<const bf16x8_t*>(pa + 32 * i * kGmPitch);
#pragma unroll
      for (int j = 0; j < NJ; ++j) bv[j] = *reinterpret_cast<const bf16x8_t*>(pb + 32 * j * kGmPitch);
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          c[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], c[i][j], 0, 0, 0);
    }
    // the other buffer was last read in the previous step, before its barrier
    stash(buf ^ 1);
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int n = n0 + wn * 32 * NJ + j * 32 + ar;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int t = t0 + wm * 32 * MI + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        // the 256-tile instance runs only where T fills its tiles
        if (MI != 2 || t < T)
          y[(int64_t)t * y_tstride + (int64_t)g * N + n] = (bf16_t)f32_to_bf16(c[i][j][e]);
      }
    }
}

bool out_proj_supported(const OprojArgs& a) {
  const int ka = (a.H / a.G) * a.D, kb = a.G * a.r;
  if (a.T < 1 || a.H % a.G) return false;
  if (a.T <= kOprojMaxTokens)
    return ka % (4 * kPjStep) == 0 && kb % (8 * kPjStep) == 0 && a.r % kPjRows == 0 &&
           a.d % kPjRows == 0;
  return a.T <= (1 << 22) && ka % kGmK == 0 && kb % kGmK == 0 && a.r % kGmTile == 0 &&
         a.d % kGmTile == 0;
}

hipError_t launch_out_proj(const OprojArgs& a, hipStream_t stream) {
  const int ka = (a.H / a.G) * a.D, kb = a.G * a.r;
  if (a.T > kOprojMaxTokens) {
    // grids padded to 8 equal XCD ranges (the kernel maps and drops the rest)
    auto grid = [&](int N, int G, int TT, int TR) {
      const int64_t total = (int64_t)(N / TR) * ((a.T + TT - 1) / TT) * G;
      return dim3((unsigned)(8 * ((total + 7) / 8)));
    };
    // 256 x 256 tiles where the weight rows divide into them, else 128 x 128
    auto run = [&](auto stage, const bf16_t* x, int64_t xs, const bf16_t* w, bf16_t* y,
                   int64_t ys, int N, int K, int G) {
      constexpr int S = decltype(stage)::value;
      if (N % 256 == 0 && a.T % 256 == 0 && (int64_t)31 * xs + K < (1LL << 30) &&
          (int64_t)31 * K + K < (1LL << 30))
        hipLaunchKernelGGL((proj_gemm<S, 4, 4>), grid(N, G, 256, 256), dim3(256), 0, stream, x, xs,
                           w, y, ys, a.T, N, K, G);
      else
        hipLaunchKernelGGL((proj_gemm<S, 2, 2>), grid(N, G, 128, 128), dim3(256), 0, stream, x, xs,
                           w, y, ys, a.T, N, K, G);
      return hipGetLastError();
    };
    hipError_t e = run(std::integral_constant<int, 0>{}, (const bf16_t*)a.o, (int64_t)a.H * a.D,
                       (const bf16_t*)a.w_a, (bf16_t*)a.mid, (int64_t)kb, a.r, ka, a.G);
    if (e != hipSuccess) return e;
    return run(std::integral_constant<int, 1>{}, (const bf16_t*)a.mid, (int64_t)kb,
               (const bf16_t*)a.w_b, (bf16_t*)a.out, (int64_t)a.d, a.d, kb, 1);
  }
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
