// Internal interface of the grouped output projection (oproj.hip) for the
// C ABI layer.
#pragma once

#include "kernels.h"

namespace csa {

// ---------------------------------------------------- grouped output projection
constexpr int kOprojMaxTokens = 16;
struct OprojArgs {
  int T, H, D, G, r, d;
  const void* o;     // [T, H, D] bf16
  const void* w_a;   // [G, r, (H/G) D] bf16
  const void* w_b;   // [d, G r] bf16
  void* mid;         // [T, G r] bf16
  void* out;         // [T, d] bf16
};
bool out_proj_supported(const OprojArgs& a);
hipError_t launch_out_proj(const OprojArgs& a, hipStream_t stream);

}  // namespace csa
