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
// 2^x by v_exp_f32 alone (about 1 ulp; results below 2^-126 flush to 0,
// -inf gives 0).  For softmax weights taken against the running maximum,
// where a weight below 2^-126 next to the maximum's weight of 1 cannot
// change a sum; exp2f adds a rescaling around the instruction to keep such
// results, seven instructions in place of one.
__device__ __forceinline__ float exp2_weight(float x) { return __builtin_amdgcn_exp2f(x); }
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// bfloat16 <-> float32
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// float32 -> bfloat16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{lo, hi}), bf16x2_t));
}

__device__ __forceinline__ uint32_t f32_to_bf16(float f) { return pack_bf16x2(f, 0.f) & 0xffffu; }

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
  // raw 16-byte words (VEC / 4 of them) and their conversion, kept apart so
  // a load can be issued long before its value is needed
  template <int VEC>
  __device__ __forceinline__ static void load_raw(const float* p, u32x4_t* w) {
#pragma unroll
    for (int c = 0; c < VEC / 4; ++c) w[c] = reinterpret_cast<const u32x4_t*>(p)[c];
  }
  // the same, for data read once: streamed past the caches (non-temporal)
  template <int VEC>
  __device__ __forceinline__ static void load_raw_stream(const float* p, u32x4_t* w) {
#pragma unroll
    for (int c = 0; c < VEC / 4; ++c)
      w[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p) + c);
  }
  template <int VEC>
  __device__ __forceinline__ static void from_raw(const u32x4_t* w, float* v) {
#pragma unroll
    for (int c = 0; c < VEC / 4; ++c)
#pragma unroll
      for (int k = 0; k < 4; ++k) v[4 * c + k] = __uint_as_float(w[c][k]);
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
  template <int VEC>
  __device__ __forceinline__ static void load_raw(const bf16_t* p, u32x4_t* w) {
#pragma unroll
    for (int c = 0; c < VEC / 8; ++c) w[c] = reinterpret_cast<const u32x4_t*>(p)[c];
  }
  template <int VEC>
  __device__ __forceinline__ static void load_raw_stream(const bf16_t* p, u32x4_t* w) {
#pragma unroll
    for (int c = 0; c < VEC / 8; ++c)
      w[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p) + c);
  }
  template <int VEC>
  __device__ __forceinline__ static void from_raw(const u32x4_t* w, float* v) {
#pragma unroll
    for (int c = 0; c < VEC / 8; ++c)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[8 * c + 2 * k] = __uint_as_float(w[c][k] << 16);
        v[8 * c + 2 * k + 1] = __uint_as_float(w[c][k] & 0xffff0000u);
      }
  }
  __device__ __forceinline__ static float get(const bf16_t* p) { return bf16_to_f32(*p); }
  __device__ __forceinline__ static void put(bf16_t* p, float v) { *p = (bf16_t)f32_to_bf16(v); }
};

// ---------------------------------------------------------------------------
// RoPE angle of pair j (of R/2) at an absolute position.  theta_j =
// base^(-2j/R) = theta1^j with theta1 = base^(-2/R) computed once on the host
// (float64 libm); theta1^j by binary powering in float64 (relative error
// ~j * 1e-16).  phi = pos * theta_j in float64, reduced modulo 2*pi in
// float64 (2*pi split into a double and its remainder, Cody-Waite style,
// exact to far below float precision for |phi| < 2^40); sin/cos of the
// reduced angle in float32.
// ---------------------------------------------------------------------------
__device__ __forceinline__ double rope_theta(double theta1, int j) {
  double th = 1.0, b = theta1;
  for (int e = j; e; e >>= 1) {
    if (e & 1) th *= b;
    b *= b;
  }
  return th;
}

// cos / sin of pos * theta (theta_j from rope_theta), the angle reduced in
// float64 as above.
__device__ __forceinline__ void rope_cos_sin_theta(int64_t pos, double theta, float& c, float& s) {
  constexpr double kTwoPiHi = 6.283185307179586;        // nearest double to 2*pi
  constexpr double kTwoPiLo = 2.4492935982947064e-16;   // 2*pi - kTwoPiHi
  constexpr double kInvTwoPi = 0.15915494309189535;
  const double phi = (double)pos * theta;
  const double k = rint(phi * kInvTwoPi);
  double r = fma(-k, kTwoPiHi, phi);
  r = fma(-k, kTwoPiLo, r);
  sincosf((float)r, &s, &c);
}

__device__ __forceinline__ void rope_cos_sin(int64_t pos, int j, double theta1, float& c, float& s) {
  rope_cos_sin_theta(pos, rope_theta(theta1, j), c, s);
}

// ---------------------------------------------------------------------------
// Wave (64-lane) helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Inclusive scan over the 64 lanes of a wave with DPP moves (no LDS
// traffic): shifts by 1, 2, 4 and 8 inside each 16-lane row, then row
// broadcasts of lane 15 and lane 31 into the rows above.  Lanes without a
// source read the operation's identity.
template <typename F>
__device__ __forceinline__ uint32_t wave_scan_dpp(uint32_t x, uint32_t id, F f) {
  x = f(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x111, 0xf, 0xf, false));
  x = f(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x112, 0xf, 0xf, false));
  x = f(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x114, 0xf, 0xf, false));
  x = f(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x118, 0xf, 0xf, false));
  x = f(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x142, 0xa, 0xf, false));
  x = f(x, (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x143, 0xc, 0xf, false));
  return x;
}
__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t x) {
  return wave_scan_dpp(x, 0u, [](uint32_t a, uint32_t b) { return a + b; });
}
// Whole-wave min / max, uniform result (lane 63 of the inclusive scan).
__device__ __forceinline__ uint32_t wave_min(uint32_t x) {
  x = wave_scan_dpp(x, 0xffffffffu, [](uint32_t a, uint32_t b) { return min(a, b); });
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}
__device__ __forceinline__ uint32_t wave_max(uint32_t x) {
  x = wave_scan_dpp(x, 0u, [](uint32_t a, uint32_t b) { return max(a, b); });
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

// Sum over the 64 lanes of a wave (DPP moves; the result is uniform).
__device__ __forceinline__ float wave_sum(float x) {
  const uint32_t r = wave_scan_dpp(__float_as_uint(x), 0u, [](uint32_t a, uint32_t b) {
    return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
  });
  return __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)r, 63));
}

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

// Inverse of score_key (a -0 score comes back as +0).
__device__ __forceinline__ float key_score(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Visible compressed entries for a query at absolute position tpos.
// min(floor((tpos + 1) / m), n_entries), at least 0.  Past the cap the
// division is skipped, and below it the dividend is under m * n_entries, which
// for any context under 2^32 tokens fits a 32-bit division (a few scalar
// instructions instead of the 64-bit division's long expansion and branch).
__device__ __forceinline__ int visible_entries(int64_t tpos, int m, int n_entries) {
  const int64_t x = tpos + 1;
  if (x <= 0 || n_entries <= 0) return 0;
  const int64_t lim = (int64_t)m * n_entries;
  if (x >= lim) return n_entries;
  if (lim <= 0xffffffffLL) return (int)((uint32_t)x / (uint32_t)m);
  return (int)(x / m);
}

// ------------------------------------------------------------- MX FP4 keys
// Indexer keys in the OCP Microscaling FP4 format: E2M1 elements (sign bit 3,
// magnitude code c in bits 0-2 holding 0, .5, 1, 1.5, 2, 3, 4, 6) and one
// E8M0 scale byte s = 2^(s - 127) per 32 channels, two channels per byte
// (the even channel in the low nibble).  The scale is floor(log2 amax) - 2,
// and each element is rounded to the nearest grid value, ties to the even
// code.

// E8M0 scale byte of a block with largest magnitude amax (finite, >= 0):
// the exponent field minus 2, at least 0 (zero and tiny blocks take 0).
__device__ __forceinline__ uint32_t mx_scale_byte(float amax) {
  const uint32_t ef = __float_as_uint(amax) >> 23;
  return ef > 2u ? ef - 2u : 0u;
}

// 2^(s - 127) as a float (s = 0 is the subnormal 2^-127).
__device__ __forceinline__ float mx_scale_value(uint32_t s) {
  return s ? __uint_as_float(s << 23) : __uint_as_float(0x00400000u);
}

// E2M1 code of x under scale byte s: |x| / 2^(s-127) is below 8 whenever s
// came from the block's maximum, and the seven comparisons place it between
// the grid's midpoints (strict at a midpoint whose lower neighbour has the
// even code, inclusive where the upper one does).
__device__ __forceinline__ uint32_t e2m1_code(float x, uint32_t s) {
  const float a = ldexpf(fabsf(x), 127 - (int)s);
  const uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                     (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                     (uint32_t)(a > 5.0f);
  return c | (x < 0.f ? 8u : 0u);
}

// Value of E2M1 code c under scale byte s (exact in float32).
__device__ __forceinline__ float e2m1_value(uint32_t c, uint32_t s) {
  const uint32_t k = c & 7u;
  const float mag = k < 2u ? 0.5f * (float)k : ldexpf(1.0f + 0.5f * (float)(k & 1u), (int)(k >> 1) - 1);
  const float v = mag * mx_scale_value(s);
  return (c & 8u) ? -v : v;
}

// Eight channels (one code dword) to bf16 MFMA operand lanes: byte i gives
// channels 2i (low nibble) and 2i + 1, scaled by 2^(s-127) in the hardware
// conversion.
__device__ __forceinline__ bf16x8_t fp4x8_to_bf16(uint32_t codes, float scale) {
  const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 0);
  const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 1);
  const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 2);
  const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 3);
  return bf16x8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// ------------------------------------------------------ MX FP8 KV entries
// KV entries in mixed precision: the R RoPE channels in bfloat16, the other
// D - R channels in the OCP Microscaling FP8 format (E4M3 elements: sign bit
// 7, exponent field bits 3-6 with bias 7, mantissa bits 0-2, exponent field
// 0 subnormal in units of 2^-9, largest finite magnitude 448; one E8M0 scale
// byte s = 2^(s - 127) per 32 channels, s = floor(log2 amax) - 8).  Packed
// row: D - R code bytes, then the 2R bytes of the bfloat16 channels, then the
// (D - R) / 32 scale bytes zero-padded to a multiple of 16.

__device__ __forceinline__ int kv_fp8_scale_pad(int D, int R) {
  return 16 * ((((D - R) / 32) + 15) / 16);
}

// E8M0 scale byte of a block with largest magnitude amax (finite, >= 0):
// the exponent field minus 8, at least 0.
__device__ __forceinline__ uint32_t mx8_scale_byte(float amax) {
  const uint32_t ef = __float_as_uint(amax) >> 23;
  return ef > 8u ? ef - 8u : 0u;
}

// E4M3 code of x under scale byte s: a = |x| / 2^(s-127) lies below 512.
// With e = max(floor(log2 a), -6) (-6: the subnormal range shares the
// smallest normal exponent's step), a * 2^(3-e) is exact and its rounding to
// an integer q in [0, 16] (nearest, ties to even) is the rounding of the
// mantissa to 3 bits; the code is 8 (e + 7) + q - 8, which carries into the
// exponent when q = 16 and equals q itself in the subnormal range.  Codes
// above 0x7E (448) saturate there.
__device__ __forceinline__ uint32_t e4m3_code(float x, uint32_t s) {
  const float a = ldexpf(fabsf(x), 127 - (int)s);
  const int e = max((int)(__float_as_uint(a) >> 23) - 127, -6);
  const float q = rintf(ldexpf(a, 3 - e));
  const uint32_t c = min((uint32_t)(8 * (e + 7) + (int)q - 8), 126u);
  return c | (x < 0.f ? 0x80u : 0u);
}

}  // namespace csa
