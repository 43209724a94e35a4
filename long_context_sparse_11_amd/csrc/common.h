// Shared device helpers for the CSA / HCA kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace csa {

typedef uint16_t bf16_t;

// MFMA operand / accumulator vector types.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// bfloat16 <-> float32
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

// Element access for the two storage types.  VEC elements per call, VEC a
// multiple of (16 bytes / element size) so every access is a 16-byte vector.
template <typename T>
struct Elem;

template <>
struct Elem<float> {
  static constexpr int kPer16 = 4;
  template <int VEC>
  __device__ __forceinline__ static void load(const float* p, float* v) {
#pragma unroll
    for (int c = 0; c < VEC / 4; ++c) {
      float4 x = reinterpret_cast<const float4*>(p)[c];
      v[4 * c + 0] = x.x; v[4 * c + 1] = x.y; v[4 * c + 2] = x.z; v[4 * c + 3] = x.w;
    }
  }
  template <int VEC>
  __device__ __forceinline__ static void store(float* p, const float* v) {
#pragma unroll
    for (int c = 0; c < VEC / 4; ++c)
      reinterpret_cast<float4*>(p)[c] = make_float4(v[4 * c], v[4 * c + 1], v[4 * c + 2], v[4 * c + 3]);
  }
  __device__ __forceinline__ static float get(const float* p) { return *p; }
  __device__ __forceinline__ static void put(float* p, float v) { *p = v; }
};

template <>
struct Elem<bf16_t> {
  static constexpr int kPer16 = 8;
  template <int VEC>
  __device__ __forceinline__ static void load(const bf16_t* p, float* v) {
#pragma unroll
    for (int c = 0; c < VEC / 8; ++c) {
      uint4 x = reinterpret_cast<const uint4*>(p)[c];
      uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[8 * c + 2 * k] = __uint_as_float(w[k] << 16);
        v[8 * c + 2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
      }
    }
  }
  template <int VEC>
  __device__ __forceinline__ static void store(bf16_t* p, const float* v) {
#pragma unroll
    for (int c = 0; c < VEC / 8; ++c) {
      uint4 x;
      x.x = pack_bf16x2(v[8 * c + 0], v[8 * c + 1]);
      x.y = pack_bf16x2(v[8 * c + 2], v[8 * c + 3]);
      x.z = pack_bf16x2(v[8 * c + 4], v[8 * c + 5]);
      x.w = pack_bf16x2(v[8 * c + 6], v[8 * c + 7]);
      reinterpret_cast<uint4*>(p)[c] = x;
    }
  }
  __device__ __forceinline__ static float get(const bf16_t* p) { return bf16_to_f32(*p); }
  __device__ __forceinline__ static void put(bf16_t* p, float v) { *p = (bf16_t)f32_to_bf16(v); }
};

// ---------------------------------------------------------------------------
// RoPE angle of pair j (of R/2) at an absolute position, float64 throughout:
// theta_j = base^(-2j/R), phi = pos * theta_j.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void rope_cos_sin(int64_t pos, int j, int R, double base, float& c,
                                             float& s) {
  const double theta = pow(base, -2.0 * (double)j / (double)R);
  const double phi = (double)pos * theta;
  double sd, cd;
  sincos(phi, &sd, &cd);
  c = (float)cd;
  s = (float)sd;
}

// ---------------------------------------------------------------------------
// Wave (64-lane) helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Order-preserving map of a float32 score to uint32 (larger float, larger
// key); -0 is folded onto +0 first.
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f == 0.0f ? 0.0f : f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Visible compressed entries for a query at absolute position tpos.
__device__ __forceinline__ int visible_entries(int64_t tpos, int m, int n_entries) {
  int64_t v = (tpos + 1) / m;
  if (v > n_entries) v = n_entries;
  if (v < 0) v = 0;
  return (int)v;
}

}  // namespace csa
