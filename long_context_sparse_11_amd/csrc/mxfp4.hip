// MX FP4 storage of indexer keys.  The pages name FP4 for the indexer cache
// ("DeepSeek V4 Inside: One Token Through Every Block", "What does HCA
// change?") without a format; the format here is the OCP Microscaling FP4
// one that gfx950 converts in hardware: E2M1 elements, one E8M0 scale per 32
// channels (element and scale rules in common.h).
#include "kernels.h"

namespace csa {

// One thread per channel pair (one code byte); the 16 lanes of a 32-channel
// block meet by lane swaps for the block maximum.  D / 2 is a multiple of 16,
// so a 16-lane group never straddles two rows and is live or dead as a whole.
template <typename T>
__global__ __launch_bounds__(256) void mxfp4_quantize_kernel(const T* x, int64_t pairs,
                                                             uint8_t* codes, uint8_t* scales) {
  const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool live = p < pairs;
  float x0 = 0.f, x1 = 0.f;
  if (live) {
    x0 = Elem<T>::get(x + 2 * p);
    x1 = Elem<T>::get(x + 2 * p + 1);
  }
  float am = fmaxf(fabsf(x0), fabsf(x1));
  am = fmaxf(am, __shfl_xor(am, 1));
  am = fmaxf(am, __shfl_xor(am, 2));
  am = fmaxf(am, __shfl_xor(am, 4));
  am = fmaxf(am, __shfl_xor(am, 8));
  const uint32_t s = mx_scale_byte(am);
  if (!live) return;
  codes[p] = (uint8_t)(e2m1_code(x0, s) | (e2m1_code(x1, s) << 4));
  if ((p & 15) == 0) scales[p >> 4] = (uint8_t)s;
}

hipError_t launch_mxfp4_quantize(int dt, int64_t rows, int D, const void* x, uint8_t* codes,
                                 uint8_t* scales, hipStream_t stream) {
  const int64_t pairs = rows * (D / 2);
  if (pairs == 0) return hipSuccess;
  const dim3 grid((unsigned)((pairs + 255) / 256));
  if (dt == 1)
    hipLaunchKernelGGL(mxfp4_quantize_kernel<bf16_t>, grid, dim3(256), 0, stream,
                       (const bf16_t*)x, pairs, codes, scales);
  else
    hipLaunchKernelGGL(mxfp4_quantize_kernel<float>, grid, dim3(256), 0, stream, (const float*)x,
                       pairs, codes, scales);
  return hipGetLastError();
}

}  // namespace csa
