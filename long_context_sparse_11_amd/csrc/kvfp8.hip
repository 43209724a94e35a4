// Mixed BF16 / FP8 storage of the KV entries.  The pages name BF16 for the
// RoPE channels and FP8 for the rest ("DeepSeek V4 Inside: One Token Through
// Every Block", "What does HCA change?", quoting the paper's section 2.3.4)
// without a format; the format here is the OCP Microscaling FP8 one (E4M3
// elements, one E8M0 scale per 32 channels) that gfx950 converts in
// hardware.  Element and scale rules in common.h.
#include "kernels.h"

namespace csa {

// One thread per 4 channels; D / 4 threads per row divide the workgroup's
// 256, and the 8 threads of a 32-channel block are 8 consecutive lanes of one
// wave (D and R multiples of 32), so a block's maximum comes from lane swaps.
template <typename T>
__global__ __launch_bounds__(256) void kv_fp8_quantize_kernel(const T* x, int64_t rows, int D,
                                                              int R, int row_bytes, uint8_t* out) {
  const int tpr = D >> 2;
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = g / tpr;
  const int t = (int)(g - row * tpr);
  const bool live = row < rows;
  const int c0 = 4 * t;
  const bool fp8 = c0 < D - R;
  float v[4] = {0.f, 0.f, 0.f, 0.f};
  if (live) {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = Elem<T>::get(x + row * D + c0 + e);
  }
  float am = fp8 ? fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))) : 0.f;
  am = fmaxf(am, __shfl_xor(am, 1));
  am = fmaxf(am, __shfl_xor(am, 2));
  am = fmaxf(am, __shfl_xor(am, 4));
  const uint32_t s = mx8_scale_byte(am);
  if (!live) return;
  uint8_t* o = out + row * row_bytes;
  if (fp8) {
    const uint32_t w = e4m3_code(v[0], s) | (e4m3_code(v[1], s) << 8) |
                       (e4m3_code(v[2], s) << 16) | (e4m3_code(v[3], s) << 24);
    *reinterpret_cast<uint32_t*>(o + c0) = w;
    if ((t & 7) == 0) o[D + R + (c0 >> 5)] = (uint8_t)s;
  } else {
    uint2 pk;
    pk.x = pack_bf16x2(v[0], v[1]);
    pk.y = pack_bf16x2(v[2], v[3]);
    *reinterpret_cast<uint2*>(o + (D - R) + 2 * (c0 - (D - R))) = pk;
  }
  if (t == 0) {  // the scale padding
    for (int p = D + R + (D - R) / 32; p < row_bytes; ++p) o[p] = 0;
  }
}

// Rows back to bfloat16 values (exact: an E4M3 value times a power of two
// has 4 significant bits), with the hardware conversion the attention uses.
// One thread per 4 channels.
__global__ __launch_bounds__(256) void kv_fp8_dequantize_kernel(const uint8_t* in, int64_t rows,
                                                                int D, int R, int row_bytes,
                                                                bf16_t* out) {
  const int tpr = D >> 2;
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = g / tpr;
  const int t = (int)(g - row * tpr);
  if (row >= rows) return;
  const int c0 = 4 * t;
  const uint8_t* ip = in + row * row_bytes;
  uint2 pk;
  if (c0 < D - R) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(ip + c0);
    const float sc = mx_scale_value(ip[D + R + (c0 >> 5)]);
    const bf16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, sc, false);
    const bf16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, sc, true);
    pk.x = __builtin_bit_cast(uint32_t, lo);
    pk.y = __builtin_bit_cast(uint32_t, hi);
  } else {
    pk = *reinterpret_cast<const uint2*>(ip + (D - R) + 2 * (c0 - (D - R)));
  }
  *reinterpret_cast<uint2*>(out + row * D + c0) = pk;
}

int kv_fp8_row_bytes_host(int D, int R) { return (D - R) + 2 * R + 16 * ((((D - R) / 32) + 15) / 16); }

hipError_t launch_kv_fp8_quantize(int dt, int64_t rows, int D, int R, const void* x, void* out,
                                  hipStream_t stream) {
  const int64_t threads = rows * (D / 4);
  if (threads == 0) return hipSuccess;
  const dim3 grid((unsigned)((threads + 255) / 256));
  const int rb = kv_fp8_row_bytes_host(D, R);
  if (dt == 1)
    hipLaunchKernelGGL(kv_fp8_quantize_kernel<bf16_t>, grid, dim3(256), 0, stream,
                       (const bf16_t*)x, rows, D, R, rb, (uint8_t*)out);
  else
    hipLaunchKernelGGL(kv_fp8_quantize_kernel<float>, grid, dim3(256), 0, stream,
                       (const float*)x, rows, D, R, rb, (uint8_t*)out);
  return hipGetLastError();
}

hipError_t launch_kv_fp8_dequantize(int64_t rows, int D, int R, const void* in, void* out,
                                    hipStream_t stream) {
  const int64_t threads = rows * (D / 4);
  if (threads == 0) return hipSuccess;
  const dim3 grid((unsigned)((threads + 255) / 256));
  hipLaunchKernelGGL(kv_fp8_dequantize_kernel, grid, dim3(256), 0, stream, (const uint8_t*)in,
                     rows, D, R, kv_fp8_row_bytes_host(D, R), (bf16_t*)out);
  return hipGetLastError();
}

}  // namespace csa
