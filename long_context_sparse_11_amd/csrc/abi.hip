// C ABI of the library (declarations and contracts in include/csa.h):
// argument validation, workspace sizing and dispatch to the kernels.  No
// call allocates, frees or synchronises.
#include "../../include/csa.h"
#include "kernels.h"
#include "oproj.h"

#include <math.h>

#include <mutex>

#define CSA_EXPORT extern "C" __attribute__((visibility("default")))

using namespace csa;

namespace {

inline bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
inline int status_of(hipError_t e) { return e == hipSuccess ? CSA_OK : CSA_ERR_HIP; }

// Candidate lists of the two-level selection for rows longer than kTopkCap.
inline int topk_chunks(int N_cap) { return N_cap > kTopkCap ? (N_cap + kTopkCap - 1) / kTopkCap : 0; }

}  // namespace

CSA_EXPORT const char* csa_status_string(int status) {
  switch (status) {
    case CSA_OK: return "CSA_OK";
    case CSA_ERR_ARG: return "CSA_ERR_ARG: invalid argument";
    case CSA_ERR_UNSUPPORTED: return "CSA_ERR_UNSUPPORTED: shape not implemented";
    case CSA_ERR_WORKSPACE: return "CSA_ERR_WORKSPACE: workspace missing or too small";
    case CSA_ERR_HIP: return "CSA_ERR_HIP: kernel launch failed";
    case CSA_ERR_SCRATCH:
      return "CSA_ERR_SCRATCH: the call needs more than the library's scratch "
             "(CSA_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown csa_status";
  }
}

// ---------------------------------------------------------------- compressor
namespace {

// Checks one compressor's arguments and fills its launch arguments.
// Returns CSA_OK, an error, or 1 for "nothing to do" (B or T zero).
// out_fp8: entries as packed mixed BF16 / FP8 rows (out_bstride in bytes).
bool kv_fp8_shape_ok(int D, int R) { return D == 512 && R >= 0 && R <= D && R % 32 == 0; }

int compress_args(int dt, int B, int T, int D, int m, int overlap, const void* c_a,
                  const void* z_a, const void* c_b, const void* z_b, const void* prev_c_b,
                  const void* prev_z_b, const float* bias_a, const float* bias_b,
                  const float* gain, float eps, int rope_dims, double rope_base,
                  const int64_t* pos0, void* out, int64_t out_bstride, CompressArgs& a,
                  int out_fp8 = 0) {
  if (dt != CSA_F32 && dt != CSA_BF16) return CSA_ERR_ARG;
  if (B < 0 || T < 0 || D <= 0 || m <= 0) return CSA_ERR_ARG;
  if (B == 0 || T == 0) return 1;
  if (!c_a || !out) return CSA_ERR_ARG;
  if (overlap) {
    if (!c_b || !z_b) return CSA_ERR_ARG;
    if ((prev_c_b == nullptr) != (prev_z_b == nullptr)) return CSA_ERR_ARG;
  } else if (c_b || z_b || prev_c_b || prev_z_b) {
    return CSA_ERR_ARG;
  }
  if (rope_dims < 0 || rope_dims > D || (rope_dims & 1)) return CSA_ERR_ARG;
  if (rope_dims > 0 && (!pos0 || !(rope_base > 0.0))) return CSA_ERR_ARG;
  if (gain && !(eps >= 0.f)) return CSA_ERR_ARG;
  const int n_out = (T + m - 1) / m;
  if (out_fp8 && !kv_fp8_shape_ok(D, rope_dims)) return CSA_ERR_UNSUPPORTED;
  const int64_t row = out_fp8 ? kv_fp8_row_bytes_host(D, rope_dims) : D;
  if (out_bstride != 0 && out_bstride < (int64_t)n_out * row) return CSA_ERR_ARG;
  if (m > 1024 || !is_pow2(D) || D > 1024 || D < (dt == CSA_BF16 ? 8 : 4)) return CSA_ERR_UNSUPPORTED;
  const double theta1 = rope_dims > 0 ? pow(rope_base, -2.0 / rope_dims) : 0.0;
  a = CompressArgs{dt, B, T, D, m, overlap ? 1 : 0, n_out, c_a, z_a, c_b, z_b, prev_c_b, prev_z_b,
                   bias_a, bias_b, gain, eps, rope_dims, theta1, pos0, out, out_bstride,
                   1, nullptr, 0};
  a.out_fp8_row = out_fp8 ? (int)row : 0;
  return CSA_OK;
}

}  // namespace

CSA_EXPORT int csa_compress(int dt, int B, int T, int D, int m, int overlap, const void* c_a,
                            const void* z_a, const void* c_b, const void* z_b,
                            const void* prev_c_b, const void* prev_z_b, const float* bias_a,
                            const float* bias_b, const float* gain, float eps, int rope_dims,
                            double rope_base, const int64_t* pos0, void* out,
                            int64_t out_bstride, void* ws, size_t ws_bytes, void* stream) {
  CompressArgs a;
  const int st = compress_args(dt, B, T, D, m, overlap, c_a, z_a, c_b, z_b, prev_c_b, prev_z_b,
                               bias_a, bias_b, gain, eps, rope_dims, rope_base, pos0, out,
                               out_bstride, a);
  if (st == 1) return CSA_OK;
  if (st != CSA_OK) return st;
  if (ws && ws_bytes < compress_ws_bytes(dt, B, a.n_out, D, m * (overlap ? 2 : 1)))
    return CSA_ERR_WORKSPACE;
  a.ws_y = (float*)ws;
  a.ws_bytes = ws ? ws_bytes : 0;
  return status_of(launch_compress(a, (hipStream_t)stream));
}

CSA_EXPORT int csa_compress_kvfp8(int dt, int B, int T, int D, int m, int overlap,
                                  const void* c_a, const void* z_a, const void* c_b,
                                  const void* z_b, const void* prev_c_b, const void* prev_z_b,
                                  const float* bias_a, const float* bias_b, const float* gain,
                                  float eps, int rope_dims, double rope_base, const int64_t* pos0,
                                  void* out, int64_t out_bstride, void* ws, size_t ws_bytes,
                                  void* stream) {
  CompressArgs a;
  const int st = compress_args(dt, B, T, D, m, overlap, c_a, z_a, c_b, z_b, prev_c_b, prev_z_b,
                               bias_a, bias_b, gain, eps, rope_dims, rope_base, pos0, out,
                               out_bstride, a, 1);
  if (st == 1) return CSA_OK;
  if (st != CSA_OK) return st;
  if (ws && ws_bytes < compress_ws_bytes(dt, B, a.n_out, D, m * (overlap ? 2 : 1)))
    return CSA_ERR_WORKSPACE;
  a.ws_y = (float*)ws;
  a.ws_bytes = ws ? ws_bytes : 0;
  return status_of(launch_compress(a, (hipStream_t)stream));
}

CSA_EXPORT int csa_compress_batch(int dt, int B, int T, int m, int overlap, const int64_t* pos0,
                                  const csa_compress_job* jobs, int n_jobs, void* stream) {
  if (n_jobs < 1 || n_jobs > 2 || !jobs) return CSA_ERR_ARG;
  CompressArgs a[2];
  int nothing = 0;
  for (int k = 0; k < n_jobs; ++k) {
    const csa_compress_job& j = jobs[k];
    const int st = compress_args(dt, B, T, j.D, m, overlap, j.c_a, j.z_a, j.c_b, j.z_b,
                                 j.prev_c_b, j.prev_z_b, j.bias_a, j.bias_b, j.gain, j.eps,
                                 j.rope_dims, j.rope_base, pos0, j.out, j.out_bstride, a[k],
                                 j.out_kv_fp8 ? 1 : 0);
    if (st == 1) nothing = 1;
    else if (st != CSA_OK) return st;
  }
  if (nothing) return CSA_OK;
  return status_of(launch_compress_batch(a, n_jobs, (hipStream_t)stream));
}

CSA_EXPORT size_t csa_compress_ws_bytes(int dt, int B, int T, int D, int m, int overlap) {
  if (B <= 0 || T <= 0 || D <= 0 || m <= 0) return 0;
  return compress_ws_bytes(dt, B, (T + m - 1) / m, D, m * (overlap ? 2 : 1));
}

// ------------------------------------------------------------- index + top-k
CSA_EXPORT size_t csa_index_topk_ws_bytes(int B, int Tq, int Hi, int N_cap, int K) {
  (void)Hi;
  if (B <= 0 || Tq <= 0 || N_cap <= 0 || K <= 0) return 0;
  const size_t q = (size_t)B * Tq;
  size_t bytes = align256(q * N_cap * sizeof(float));
  const int nc = topk_chunks(N_cap);
  if (nc) bytes += 2 * align256(q * nc * K * sizeof(float));
  return bytes;
}

namespace {

// Indexer scores of every visible entry, optionally preceded by the
// fresh-entry compressors of a decode step (fused into the indexer launch
// when its kernel covers the shape, else a compressor launch first).
// Arguments already validated; N_cap > 0.
int index_scores_run(int dt, int B, int Tq, int Hi, int Di, int N_cap, int m, const void* q_idx,
                     const float* w_idx, const void* k_idx, const uint8_t* k_scales,
                     const int32_t* n_entries, const int64_t* q_pos0, float* scores,
                     const FreshJobs* fresh, hipStream_t s) {
  IndexArgs ia{dt, B, Tq, Hi, Di, N_cap, m, q_idx, w_idx, k_idx, n_entries, q_pos0, scores,
               k_scales};
  hipError_t e;
  const bool fused = fresh && index_fresh_fused(ia, *fresh);
  // FP4 fresh keys are written only by the fused launch
  if (fresh && !fused && fresh->job[0].out_scales) return CSA_ERR_UNSUPPORTED;
  if (fused) {
    e = launch_index_fresh(ia, *fresh, s);
  } else {
    e = fresh ? launch_compress_batch(fresh->job, min(fresh->n_jobs, 2), s) : hipSuccess;
    if (e == hipSuccess && fresh && fresh->n_jobs == 3) e = launch_compress(fresh->job[2], s);
    if (e == hipSuccess) e = launch_index_scores(ia, s);
  }
  return status_of(e);
}

// Indexer scores and top-K, optionally preceded by the fresh-entry
// compressors of a decode step (index_scores_run), then the selection.
int index_topk_run(int dt, int B, int Tq, int Hi, int Di, int N_cap, int K, int m,
                   const void* q_idx, const float* w_idx, const void* k_idx,
                   const uint8_t* k_scales, const int32_t* n_entries, const int64_t* q_pos0, int32_t* idx_out,
                   float* score_out, float* all_scores, void* ws, size_t ws_bytes,
                   const FreshJobs* fresh, hipStream_t s) {
  if (dt != CSA_F32 && dt != CSA_BF16) return CSA_ERR_ARG;
  if (B < 0 || Tq < 0 || Hi <= 0 || Di <= 0 || N_cap < 0 || K <= 0 || m <= 0) return CSA_ERR_ARG;
  if (B == 0 || Tq == 0) return CSA_OK;
  if (!q_idx || !w_idx || !n_entries || !q_pos0 || !idx_out) return CSA_ERR_ARG;
  if (N_cap > 0 && !k_idx) return CSA_ERR_ARG;
  if (k_scales && (dt != CSA_BF16 || Di % 32)) return CSA_ERR_ARG;
  if (Hi > 64 || Di > 256 || Hi * Di > 8192 || K > 4096 || N_cap > (1 << 26))
    return CSA_ERR_UNSUPPORTED;
  if ((int64_t)topk_chunks(N_cap) * K > kTopkCap) return CSA_ERR_UNSUPPORTED;
  const size_t need = csa_index_topk_ws_bytes(B, Tq, Hi, N_cap, K);
  if (N_cap > 0 && (!ws || ws_bytes < need)) return CSA_ERR_WORKSPACE;
  const size_t q = (size_t)B * Tq;
  char* w = (char*)ws;
  float* scores = all_scores ? all_scores : (float*)w;
  w += align256(q * (size_t)N_cap * sizeof(float));

  if (N_cap > 0) {
    const int st = index_scores_run(dt, B, Tq, Hi, Di, N_cap, m, q_idx, w_idx, k_idx, k_scales,
                                    n_entries, q_pos0, scores, fresh, s);
    if (st != CSA_OK) return st;
  }
  const int nc = topk_chunks(N_cap);
  TopkArgs ta{};
  ta.B = B; ta.Tq = Tq; ta.N_cap = N_cap; ta.m = m; ta.K = K;
  ta.n_entries = n_entries; ta.q_pos0 = q_pos0;
  if (nc == 0) {
    ta.mode = 0;
    ta.nchunks = 1;
    ta.scores = scores;
    ta.out_idx = idx_out;
    ta.out_scores = score_out;
    return status_of(launch_topk(ta, (int)q, s));
  }
  float* cand_s = (float*)w;
  int32_t* cand_i = (int32_t*)(w + align256(q * nc * K * sizeof(float)));
  ta.mode = 1;
  ta.nchunks = nc;
  ta.chunk = kTopkCap;
  ta.scores = scores;
  ta.out_idx = cand_i;
  ta.out_scores = cand_s;
  hipError_t e = launch_topk(ta, (int)(q * nc), s);
  if (e != hipSuccess) return CSA_ERR_HIP;
  TopkArgs tb = ta;
  tb.mode = 2;
  tb.scores = cand_s;
  tb.in_idx = cand_i;
  tb.out_idx = idx_out;
  tb.out_scores = score_out;
  return status_of(launch_topk(tb, (int)q, s));
}

}  // namespace

CSA_EXPORT int csa_index_topk(int dt, int B, int Tq, int Hi, int Di, int N_cap, int K, int m,
                              const void* q_idx, const float* w_idx, const void* k_idx,
                              const int32_t* n_entries, const int64_t* q_pos0, int32_t* idx_out,
                              float* score_out, float* all_scores, void* ws, size_t ws_bytes,
                              void* stream) {
  return index_topk_run(dt, B, Tq, Hi, Di, N_cap, K, m, q_idx, w_idx, k_idx, nullptr, n_entries,
                        q_pos0, idx_out, score_out, all_scores, ws, ws_bytes, nullptr,
                        (hipStream_t)stream);
}

CSA_EXPORT int csa_index_topk_mxfp4(int B, int Tq, int Hi, int Di, int N_cap, int K, int m,
                                    const void* q_idx, const float* w_idx, const uint8_t* k_codes,
                                    const uint8_t* k_scales, const int32_t* n_entries,
                                    const int64_t* q_pos0, int32_t* idx_out, float* score_out,
                                    float* all_scores, void* ws, size_t ws_bytes, void* stream) {
  if (N_cap > 0 && !k_scales) return CSA_ERR_ARG;
  if (Di <= 0 || Di % 32) return CSA_ERR_ARG;
  return index_topk_run(CSA_BF16, B, Tq, Hi, Di, N_cap, K, m, q_idx, w_idx, k_codes,
                        N_cap > 0 ? k_scales : nullptr, n_entries, q_pos0, idx_out, score_out,
                        all_scores, ws, ws_bytes, nullptr, (hipStream_t)stream);
}

namespace {

// The fresh-entry jobs of a decode step; key_codes/key_scales replace job
// 0's output when the indexer keys are stored as MX FP4.  Returns a status.
int decode_jobs(int dt, int B, int Tq, int N_cap, int m, int overlap, const int64_t* block_pos0,
                const csa_compress_job* jobs, int n_jobs, uint8_t* key_codes,
                uint8_t* key_scales, const int32_t* n_entries, const int64_t* q_pos0,
                FreshJobs& f) {
  f = FreshJobs{};
  f.n_jobs = n_jobs;
  for (int k = 0; k < n_jobs; ++k) {
    const csa_compress_job& j = jobs[k];
    if (k == 2) {  // the step token's window row: m = 1, ring slot q_pos0[b] % L_win
      if (Tq != 1 || !q_pos0 || j.D <= 0 || j.out_bstride <= 0 || j.out_bstride % j.D ||
          j.out_kv_fp8)
        return CSA_ERR_ARG;
      const int st = compress_args(dt, B, 1, j.D, 1, 0, j.c_a, j.z_a, j.c_b, j.z_b, j.prev_c_b,
                                   j.prev_z_b, j.bias_a, j.bias_b, j.gain, j.eps, j.rope_dims,
                                   j.rope_base, q_pos0, j.out, j.out_bstride, f.job[2]);
      if (st != CSA_OK) return st == 1 ? CSA_ERR_ARG : st;
      f.job[2].ring_len = (int)(j.out_bstride / j.D);
      f.job[2].slices = 1;
      continue;
    }
    // the KV job (jobs[1]) may store packed mixed BF16 / FP8 rows
    if (j.out_kv_fp8 && k != 1) return CSA_ERR_ARG;
    if (j.out_kv_fp8 && !kv_fp8_shape_ok(j.D, j.rope_dims)) return CSA_ERR_UNSUPPORTED;
    const int64_t pool_stride =
        (int64_t)N_cap * (j.out_kv_fp8 ? kv_fp8_row_bytes_host(j.D, j.rope_dims) : j.D);
    if (j.out_bstride != 0 && j.out_bstride != pool_stride) return CSA_ERR_ARG;
    void* out = (k == 0 && key_codes) ? key_codes : j.out;
    const int st = compress_args(dt, B, m, j.D, m, overlap, j.c_a, j.z_a, j.c_b, j.z_b,
                                 j.prev_c_b, j.prev_z_b, j.bias_a, j.bias_b, j.gain, j.eps,
                                 j.rope_dims, j.rope_base, block_pos0, out, pool_stride, f.job[k],
                                 j.out_kv_fp8 ? 1 : 0);
    if (st != CSA_OK) return st == 1 ? CSA_ERR_ARG : st;
    f.job[k].rows_at = n_entries;
    f.job[k].rows_cap = N_cap;
    f.job[k].slices = 1;
    if (k == 0 && key_codes) f.job[k].out_scales = key_scales;
  }
  return CSA_OK;
}

}  // namespace

CSA_EXPORT int csa_decode_index_topk(int dt, int B, int Tq, int Hi, int Di, int N_cap, int K,
                                     int m, int overlap, const int64_t* block_pos0,
                                     const csa_compress_job* jobs, int n_jobs, const void* q_idx,
                                     const float* w_idx, const int32_t* n_entries,
                                     const int64_t* q_pos0, int32_t* idx_out, float* score_out,
                                     float* all_scores, void* ws, size_t ws_bytes,
                                     void* stream) {
  if (n_jobs < 1 || n_jobs > 3 || !jobs) return CSA_ERR_ARG;
  if (B < 0 || Tq < 0 || N_cap < 0 || m <= 0) return CSA_ERR_ARG;
  if (jobs[0].D != Di) return CSA_ERR_ARG;
  if (B == 0 || Tq == 0) return CSA_OK;
  if (N_cap == 0) return CSA_ERR_ARG;  // the fresh entries need a row
  FreshJobs f;
  const int st = decode_jobs(dt, B, Tq, N_cap, m, overlap, block_pos0, jobs, n_jobs, nullptr,
                             nullptr, n_entries, q_pos0, f);
  if (st != CSA_OK) return st;
  return index_topk_run(dt, B, Tq, Hi, Di, N_cap, K, m, q_idx, w_idx, jobs[0].out, nullptr,
                        n_entries, q_pos0, idx_out, score_out, all_scores, ws, ws_bytes, &f,
                        (hipStream_t)stream);
}

CSA_EXPORT int csa_decode_index_topk_mxfp4(int B, int Tq, int Hi, int Di, int N_cap, int K, int m,
                                           int overlap, const int64_t* block_pos0,
                                           const csa_compress_job* jobs, int n_jobs,
                                           const void* q_idx, const float* w_idx,
                                           uint8_t* k_codes, uint8_t* k_scales,
                                           const int32_t* n_entries, const int64_t* q_pos0,
                                           int32_t* idx_out, float* score_out, float* all_scores,
                                           void* ws, size_t ws_bytes, void* stream) {
  if (n_jobs < 1 || n_jobs > 3 || !jobs) return CSA_ERR_ARG;
  if (B < 0 || Tq < 0 || N_cap < 0 || m <= 0) return CSA_ERR_ARG;
  if (jobs[0].D != Di || Di <= 0 || Di % 32) return CSA_ERR_ARG;
  if (jobs[0].out || jobs[0].out_bstride) return CSA_ERR_ARG;  // the key job writes k_codes
  if (B == 0 || Tq == 0) return CSA_OK;
  if (N_cap == 0 || !k_codes || !k_scales) return CSA_ERR_ARG;
  FreshJobs f;
  const int st = decode_jobs(CSA_BF16, B, Tq, N_cap, m, overlap, block_pos0, jobs, n_jobs,
                             k_codes, k_scales, n_entries, q_pos0, f);
  if (st != CSA_OK) return st;
  return index_topk_run(CSA_BF16, B, Tq, Hi, Di, N_cap, K, m, q_idx, w_idx, k_codes, k_scales,
                        n_entries, q_pos0, idx_out, score_out, all_scores, ws, ws_bytes, &f,
                        (hipStream_t)stream);
}

// ------------------------------------------------- no-allocation decode call
// The scratch of csa_decode_index_topk_noalloc: a file-scope device array
// (one copy on every device the library runs on, allocated with the code
// object).  In host code `scratch` is a host-side stand-in, not a device
// address; the device address comes from hipGetSymbolAddress, once per
// device, and only that address is passed to kernels.
static __device__ __align__(256) unsigned char scratch[CSA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address (looked up on its first use), or
// nullptr if the lookup fails.
void* device_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

CSA_EXPORT int csa_decode_index_topk_noalloc(int dt, int B, int Tq, int Hi, int Di, int N_cap,
                                             int K, int m, int overlap,
                                             const int64_t* block_pos0,
                                             const csa_compress_job* jobs, int n_jobs,
                                             const void* q_idx, const float* w_idx,
                                             const int32_t* n_entries, const int64_t* q_pos0,
                                             int32_t* idx_out, float* score_out,
                                             float* all_scores, void* stream) {
  if (B < 0 || Tq < 0 || Hi <= 0 || N_cap < 0 || K <= 0) return CSA_ERR_ARG;
  const size_t need = csa_index_topk_ws_bytes(B, Tq, Hi, N_cap, K);
  if (need > (size_t)CSA_NOALLOC_SCRATCH_BYTES) return CSA_ERR_SCRATCH;
  void* ws = nullptr;
  if (need > 0) {
    ws = device_scratch();
    if (!ws) return CSA_ERR_HIP;
  }
  return csa_decode_index_topk(dt, B, Tq, Hi, Di, N_cap, K, m, overlap, block_pos0, jobs, n_jobs,
                               q_idx, w_idx, n_entries, q_pos0, idx_out, score_out, all_scores,
                               ws, need > 0 ? (size_t)CSA_NOALLOC_SCRATCH_BYTES : 0, stream);
}

namespace {

// Shape and pointer checks shared by the two decode-scores calls.
int decode_scores_args(int B, int Tq, int Hi, int Di, int N_cap, int m, const void* q_idx,
                       const float* w_idx, const int32_t* n_entries, const int64_t* q_pos0,
                       const float* scores) {
  if (B < 0 || Tq < 0 || Hi <= 0 || Di <= 0 || N_cap < 0 || m <= 0) return CSA_ERR_ARG;
  if (B == 0 || Tq == 0) return 1;
  if (N_cap == 0) return CSA_ERR_ARG;  // the fresh entries need a row
  if (!q_idx || !w_idx || !n_entries || !q_pos0 || !scores) return CSA_ERR_ARG;
  if (Hi > 64 || Di > 256 || Hi * Di > 8192 || N_cap > (1 << 26)) return CSA_ERR_UNSUPPORTED;
  return CSA_OK;
}

}  // namespace

CSA_EXPORT int csa_decode_index_scores(int dt, int B, int Tq, int Hi, int Di, int N_cap, int m,
                                       int overlap, const int64_t* block_pos0,
                                       const csa_compress_job* jobs, int n_jobs,
                                       const void* q_idx, const float* w_idx,
                                       const int32_t* n_entries, const int64_t* q_pos0,
                                       float* scores, void* stream) {
  if (dt != CSA_F32 && dt != CSA_BF16) return CSA_ERR_ARG;
  if (n_jobs < 1 || n_jobs > 3 || !jobs) return CSA_ERR_ARG;
  if (jobs[0].D != Di) return CSA_ERR_ARG;
  const int st0 = decode_scores_args(B, Tq, Hi, Di, N_cap, m, q_idx, w_idx, n_entries, q_pos0,
                                     scores);
  if (st0 != CSA_OK) return st0 == 1 ? CSA_OK : st0;
  FreshJobs f;
  const int st = decode_jobs(dt, B, Tq, N_cap, m, overlap, block_pos0, jobs, n_jobs, nullptr,
                             nullptr, n_entries, q_pos0, f);
  if (st != CSA_OK) return st;
  return index_scores_run(dt, B, Tq, Hi, Di, N_cap, m, q_idx, w_idx, jobs[0].out, nullptr,
                          n_entries, q_pos0, scores, &f, (hipStream_t)stream);
}

CSA_EXPORT int csa_decode_index_scores_mxfp4(int B, int Tq, int Hi, int Di, int N_cap, int m,
                                             int overlap, const int64_t* block_pos0,
                                             const csa_compress_job* jobs, int n_jobs,
                                             const void* q_idx, const float* w_idx,
                                             uint8_t* k_codes, uint8_t* k_scales,
                                             const int32_t* n_entries, const int64_t* q_pos0,
                                             float* scores, void* stream) {
  if (n_jobs < 1 || n_jobs > 3 || !jobs) return CSA_ERR_ARG;
  if (jobs[0].D != Di || Di <= 0 || Di % 32) return CSA_ERR_ARG;
  if (jobs[0].out || jobs[0].out_bstride) return CSA_ERR_ARG;  // the key job writes k_codes
  const int st0 = decode_scores_args(B, Tq, Hi, Di, N_cap, m, q_idx, w_idx, n_entries, q_pos0,
                                     scores);
  if (st0 != CSA_OK) return st0 == 1 ? CSA_OK : st0;
  if (!k_codes || !k_scales) return CSA_ERR_ARG;
  FreshJobs f;
  const int st = decode_jobs(CSA_BF16, B, Tq, N_cap, m, overlap, block_pos0, jobs, n_jobs,
                             k_codes, k_scales, n_entries, q_pos0, f);
  if (st != CSA_OK) return st;
  return index_scores_run(CSA_BF16, B, Tq, Hi, Di, N_cap, m, q_idx, w_idx, k_codes, k_scales,
                          n_entries, q_pos0, scores, &f, (hipStream_t)stream);
}

CSA_EXPORT int csa_index_scores(int dt, int B, int Tq, int Hi, int Di, int N_cap, int m,
                                const void* q_idx, const float* w_idx, const void* k_idx,
                                const int32_t* n_entries, const int64_t* q_pos0, float* scores,
                                void* stream) {
  if (dt != CSA_F32 && dt != CSA_BF16) return CSA_ERR_ARG;
  if (B < 0 || Tq < 0 || Hi <= 0 || Di <= 0 || N_cap < 0 || m <= 0) return CSA_ERR_ARG;
  if (B == 0 || Tq == 0 || N_cap == 0) return CSA_OK;
  if (!q_idx || !w_idx || !k_idx || !n_entries || !q_pos0 || !scores) return CSA_ERR_ARG;
  if (Hi > 64 || Di > 256 || Hi * Di > 8192 || N_cap > (1 << 26)) return CSA_ERR_UNSUPPORTED;
  IndexArgs ia{dt, B, Tq, Hi, Di, N_cap, m, q_idx, w_idx, k_idx, n_entries, q_pos0, scores};
  return status_of(launch_index_scores(ia, (hipStream_t)stream));
}

CSA_EXPORT int csa_index_scores_mxfp4(int B, int Tq, int Hi, int Di, int N_cap, int m,
                                      const void* q_idx, const float* w_idx,
                                      const uint8_t* k_codes, const uint8_t* k_scales,
                                      const int32_t* n_entries, const int64_t* q_pos0,
                                      float* scores, void* stream) {
  if (B < 0 || Tq < 0 || Hi <= 0 || Di <= 0 || Di % 32 || N_cap < 0 || m <= 0) return CSA_ERR_ARG;
  if (B == 0 || Tq == 0 || N_cap == 0) return CSA_OK;
  if (!q_idx || !w_idx || !k_codes || !k_scales || !n_entries || !q_pos0 || !scores)
    return CSA_ERR_ARG;
  if (Hi > 64 || Di > 256 || Hi * Di > 8192 || N_cap > (1 << 26)) return CSA_ERR_UNSUPPORTED;
  IndexArgs ia{CSA_BF16, B, Tq, Hi, Di, N_cap, m, q_idx, w_idx, k_codes, n_entries, q_pos0,
               scores, k_scales};
  return status_of(launch_index_scores(ia, (hipStream_t)stream));
}

// ------------------------------------------------------------- decode state
CSA_EXPORT int csa_window_row(int dt, int B, int D, const void* kv, const float* gain, float eps,
                              int rope_dims, double rope_base, const int64_t* pos, void* win,
                              int L_win, void* stream) {
  if (B < 0 || D <= 0 || L_win <= 0) return CSA_ERR_ARG;
  if (B == 0) return CSA_OK;
  if (!pos) return CSA_ERR_ARG;
  CompressArgs a;
  const int st = compress_args(dt, B, 1, D, 1, 0, kv, nullptr, nullptr, nullptr, nullptr, nullptr,
                               nullptr, nullptr, gain, eps, rope_dims, rope_base, pos, win,
                               (int64_t)L_win * D, a);
  if (st != CSA_OK) return st == 1 ? CSA_OK : st;
  a.ring_len = L_win;
  a.ws_y = nullptr;
  a.ws_bytes = 0;
  return status_of(launch_compress(a, (hipStream_t)stream));
}

CSA_EXPORT int csa_decode_advance(int B, int m, int N_cap, int64_t* q_pos, int32_t* n_entries,
                                  int64_t* block_pos0, void* stream) {
  if (B < 0 || m <= 0 || N_cap < 0) return CSA_ERR_ARG;
  if (B == 0) return CSA_OK;
  if (!q_pos || !n_entries || !block_pos0) return CSA_ERR_ARG;
  return status_of(launch_decode_advance(B, m, N_cap, q_pos, n_entries, block_pos0,
                                         (hipStream_t)stream));
}

// -------------------------------------------------- grouped output projection
CSA_EXPORT int csa_output_proj(int T, int H, int D, int G, int r, int d_model, const void* o,
                               const void* w_a, const void* w_b, void* mid, void* out,
                               void* stream) {
  if (T < 0 || H <= 0 || D <= 0 || G <= 0 || r <= 0 || d_model <= 0 || H % G) return CSA_ERR_ARG;
  if (T == 0) return CSA_OK;
  if (!o || !w_a || !w_b || !mid || !out) return CSA_ERR_ARG;
  OprojArgs a{T, H, D, G, r, d_model, o, w_a, w_b, mid, out};
  if (!out_proj_supported(a)) return CSA_ERR_UNSUPPORTED;
  return status_of(launch_out_proj(a, (hipStream_t)stream));
}

// ------------------------------------------------------------------ MX FP4
CSA_EXPORT int csa_quantize_mxfp4(int dt, int64_t rows, int D, const void* x, uint8_t* codes,
                                  uint8_t* scales, void* stream) {
  if (dt != CSA_F32 && dt != CSA_BF16) return CSA_ERR_ARG;
  if (rows < 0 || D <= 0 || D % 32) return CSA_ERR_ARG;
  if (rows == 0) return CSA_OK;
  if (!x || !codes || !scales) return CSA_ERR_ARG;
  if (rows > ((int64_t)1 << 39) / D) return CSA_ERR_UNSUPPORTED;  // grid bound
  return status_of(launch_mxfp4_quantize(dt, rows, D, x, codes, scales, (hipStream_t)stream));
}

// -------------------------------------------------- mixed BF16 / FP8 KV rows
CSA_EXPORT size_t csa_kv_fp8_row_bytes(int D, int rope_dims) {
  if (!kv_fp8_shape_ok(D, rope_dims)) return 0;
  return (size_t)kv_fp8_row_bytes_host(D, rope_dims);
}

CSA_EXPORT int csa_quantize_kv_fp8(int dt, int64_t rows, int D, int rope_dims, const void* x,
                                   void* out, void* stream) {
  if (dt != CSA_F32 && dt != CSA_BF16) return CSA_ERR_ARG;
  if (rows < 0 || D <= 0 || rope_dims < 0 || rope_dims > D) return CSA_ERR_ARG;
  if (!kv_fp8_shape_ok(D, rope_dims)) return CSA_ERR_UNSUPPORTED;
  if (rows == 0) return CSA_OK;
  if (!x || !out) return CSA_ERR_ARG;
  if (rows > ((int64_t)1 << 39) / D) return CSA_ERR_UNSUPPORTED;  // grid bound
  return status_of(launch_kv_fp8_quantize(dt, rows, D, rope_dims, x, out, (hipStream_t)stream));
}

CSA_EXPORT int csa_dequantize_kv_fp8(int64_t rows, int D, int rope_dims, const void* rows_in,
                                     void* out, void* stream) {
  if (rows < 0 || D <= 0 || rope_dims < 0 || rope_dims > D) return CSA_ERR_ARG;
  if (!kv_fp8_shape_ok(D, rope_dims)) return CSA_ERR_UNSUPPORTED;
  if (rows == 0) return CSA_OK;
  if (!rows_in || !out) return CSA_ERR_ARG;
  if (rows > ((int64_t)1 << 39) / D) return CSA_ERR_UNSUPPORTED;
  return status_of(launch_kv_fp8_dequantize(rows, D, rope_dims, rows_in, out,
                                            (hipStream_t)stream));
}

// ------------------------------------------------------------------ attention
CSA_EXPORT size_t csa_attn_ws_bytes(int B, int Tq, int H, int D, int keys_per_query) {
  if (B <= 0 || Tq <= 0 || H <= 0 || D <= 0 || keys_per_query <= 0) return 0;
  return attn_ws_bytes(CSA_BF16, B, Tq, H, D, keys_per_query);
}

namespace {

int attn_common(AttnArgs& a, double rope_base, int keys_per_query, void* ws, size_t ws_bytes,
                hipStream_t s) {
  if (a.dt != CSA_F32 && a.dt != CSA_BF16) return CSA_ERR_ARG;
  if (a.B < 0 || a.Tq < 0 || a.H <= 0 || a.D <= 0 || a.N_cap < 0 || a.W < 0 || a.L_win < 0)
    return CSA_ERR_ARG;
  if (a.B == 0 || a.Tq == 0) return CSA_OK;
  if (!a.q || !a.sink || !a.q_pos0 || !a.out) return CSA_ERR_ARG;
  if (a.N_cap > 0 && !a.pool) return CSA_ERR_ARG;
  if (a.W > 0 && a.L_win > 0 && !a.win) return CSA_ERR_ARG;
  if (a.W > 0 && a.L_win > 0 && !a.win_pos0 && a.L_win < a.W) return CSA_ERR_ARG;  // ring
  if (a.R < 0 || a.R > a.D || (a.R & 1) || (a.R > 0 && !(rope_base > 0.0))) return CSA_ERR_ARG;
  if (a.D > 1024 || a.H > 128 || (a.D & 1)) return CSA_ERR_UNSUPPORTED;
  a.rope_theta1 = a.R > 0 ? pow(rope_base, -2.0 / a.R) : 0.0;
  // packed mixed BF16 / FP8 pool rows: the bf16 MFMA kernels only
  if (a.pool_row_bytes > 0 &&
      (!attn_uses_mfma(a.dt, a.H, a.D, a.R) || !kv_fp8_shape_ok(a.D, a.R)))
    return CSA_ERR_UNSUPPORTED;
  if (attn_uses_mfma(a.dt, a.H, a.D, a.R)) {
    if (a.csa && (int64_t)keys_per_query > attn_max_csa_keys()) return CSA_ERR_UNSUPPORTED;
    a.splits = a.fresh ? attn_fresh_splits(a.B, a.H, a.D, keys_per_query)
                       : attn_splits(a.dt, a.B, a.Tq, a.H, a.D, keys_per_query);
    if (a.splits > 1) {
      const size_t need = a.fresh ? attn_fresh_ws_bytes(a.B, a.H, a.D, keys_per_query)
                                  : attn_ws_bytes(a.dt, a.B, a.Tq, a.H, a.D, keys_per_query);
      if (!ws || ws_bytes < need) return CSA_ERR_WORKSPACE;
      a.part_ml = (float*)ws;
      a.part_o = (bf16_t*)(a.part_ml + (size_t)a.B * a.Tq * a.splits * a.H * 2);
    }
  } else {
    a.splits = 1;
  }
  return status_of(launch_attn(a, s));
}

}  // namespace

CSA_EXPORT int csa_sparse_attn(int dt, int B, int Tq, int H, int D, int rope_dims,
                               double rope_base, float scale, const void* q, const void* pool,
                               int N_cap, const int32_t* idx, int K, const void* win, int L_win,
                               const int64_t* win_pos0, int W, const float* sink,
                               const int64_t* q_pos0, void* out, float* lse, void* ws,
                               size_t ws_bytes, void* stream) {
  if (K < 0) return CSA_ERR_ARG;
  if (K > 0 && !idx) return CSA_ERR_ARG;
  AttnArgs a{};
  a.dt = dt; a.B = B; a.Tq = Tq; a.H = H; a.D = D; a.R = rope_dims;
  a.scale = scale;
  a.q = q; a.pool = pool; a.N_cap = N_cap; a.csa = 1; a.idx = idx; a.K = K;
  a.n_entries = nullptr; a.m = 1;
  a.win = win; a.L_win = L_win; a.win_pos0 = win_pos0; a.W = W;
  a.sink = sink; a.q_pos0 = q_pos0; a.out = out; a.lse = lse;
  return attn_common(a, rope_base, K + W, ws, ws_bytes, (hipStream_t)stream);
}

CSA_EXPORT int csa_sparse_attn_kvfp8(int B, int Tq, int H, int D, int rope_dims,
                                     double rope_base, float scale, const void* q,
                                     const void* pool, int N_cap, const int32_t* idx, int K,
                                     const void* win, int L_win, const int64_t* win_pos0, int W,
                                     const float* sink, const int64_t* q_pos0, void* out,
                                     float* lse, void* ws, size_t ws_bytes, void* stream) {
  if (K < 0) return CSA_ERR_ARG;
  if (K > 0 && !idx) return CSA_ERR_ARG;
  if (!kv_fp8_shape_ok(D, rope_dims)) return CSA_ERR_UNSUPPORTED;
  AttnArgs a{};
  a.dt = CSA_BF16; a.B = B; a.Tq = Tq; a.H = H; a.D = D; a.R = rope_dims;
  a.scale = scale;
  a.q = q; a.pool = pool; a.N_cap = N_cap; a.csa = 1; a.idx = idx; a.K = K;
  a.n_entries = nullptr; a.m = 1;
  a.win = win; a.L_win = L_win; a.win_pos0 = win_pos0; a.W = W;
  a.sink = sink; a.q_pos0 = q_pos0; a.out = out; a.lse = lse;
  a.pool_row_bytes = kv_fp8_row_bytes_host(D, rope_dims);
  return attn_common(a, rope_base, K + W, ws, ws_bytes, (hipStream_t)stream);
}

CSA_EXPORT int hca_attn_kvfp8(int B, int Tq, int H, int D, int rope_dims, double rope_base,
                              float scale, const void* q, const void* pool, int N_cap,
                              const int32_t* n_entries, int m, const void* win, int L_win,
                              const int64_t* win_pos0, int W, const float* sink,
                              const int64_t* q_pos0, void* out, float* lse, void* ws,
                              size_t ws_bytes, void* stream) {
  if (m <= 0 || !n_entries) return CSA_ERR_ARG;
  if (!kv_fp8_shape_ok(D, rope_dims)) return CSA_ERR_UNSUPPORTED;
  AttnArgs a{};
  a.dt = CSA_BF16; a.B = B; a.Tq = Tq; a.H = H; a.D = D; a.R = rope_dims;
  a.scale = scale;
  a.q = q; a.pool = pool; a.N_cap = N_cap; a.csa = 0; a.idx = nullptr; a.K = 0;
  a.n_entries = n_entries; a.m = m;
  a.win = win; a.L_win = L_win; a.win_pos0 = win_pos0; a.W = W;
  a.sink = sink; a.q_pos0 = q_pos0; a.out = out; a.lse = lse;
  a.pool_row_bytes = kv_fp8_row_bytes_host(D, rope_dims);
  return attn_common(a, rope_base, N_cap + W, ws, ws_bytes, (hipStream_t)stream);
}

CSA_EXPORT int hca_attn(int dt, int B, int Tq, int H, int D, int rope_dims, double rope_base,
                        float scale, const void* q, const void* pool, int N_cap,
                        const int32_t* n_entries, int m, const void* win, int L_win,
                        const int64_t* win_pos0, int W, const float* sink, const int64_t* q_pos0,
                        void* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  if (m <= 0 || !n_entries) return CSA_ERR_ARG;
  AttnArgs a{};
  a.dt = dt; a.B = B; a.Tq = Tq; a.H = H; a.D = D; a.R = rope_dims;
  a.scale = scale;
  a.q = q; a.pool = pool; a.N_cap = N_cap; a.csa = 0; a.idx = nullptr; a.K = 0;
  a.n_entries = n_entries; a.m = m;
  a.win = win; a.L_win = L_win; a.win_pos0 = win_pos0; a.W = W;
  a.sink = sink; a.q_pos0 = q_pos0; a.out = out; a.lse = lse;
  return attn_common(a, rope_base, N_cap + W, ws, ws_bytes, (hipStream_t)stream);
}

CSA_EXPORT size_t hca_decode_attn_ws_bytes(int B, int H, int D, int keys_per_query) {
  if (B <= 0 || keys_per_query <= 0 || !attn_uses_mfma(CSA_BF16, H, D, 0)) return 0;
  return attn_fresh_ws_bytes(B, H, D, keys_per_query);
}

namespace {

int hca_decode_common(int B, int H, int D, int rope_dims, double rope_base, float scale,
                      const void* q, void* pool, int N_cap, const int32_t* n_entries, int m,
                      const void* c, const void* z, const float* bias, const float* gain,
                      float eps, const int64_t* block_pos0, const void* win, int L_win,
                      const int64_t* win_pos0, int W, const float* sink, const int64_t* q_pos0,
                      void* out, float* lse, void* ws, size_t ws_bytes, hipStream_t stream,
                      bool fp8) {
  if (m <= 0 || !n_entries || !block_pos0 || !c) return CSA_ERR_ARG;
  if (gain && !(eps >= 0.f)) return CSA_ERR_ARG;
  if (rope_dims < 0 || rope_dims > D || (rope_dims & 1)) return CSA_ERR_ARG;
  if (!attn_uses_mfma(CSA_BF16, H, D, rope_dims) || m > 1024) return CSA_ERR_UNSUPPORTED;
  if (fp8 && !kv_fp8_shape_ok(D, rope_dims)) return CSA_ERR_UNSUPPORTED;
  AttnArgs a{};
  a.dt = CSA_BF16; a.B = B; a.Tq = 1; a.H = H; a.D = D; a.R = rope_dims;
  a.scale = scale;
  a.q = q; a.pool = pool; a.N_cap = N_cap; a.csa = 0; a.idx = nullptr; a.K = 0;
  a.n_entries = n_entries; a.m = m;
  a.win = win; a.L_win = L_win; a.win_pos0 = win_pos0; a.W = W;
  a.sink = sink; a.q_pos0 = q_pos0; a.out = out; a.lse = lse;
  if (fp8) a.pool_row_bytes = kv_fp8_row_bytes_host(D, rope_dims);
  a.fresh = 1;
  a.fj.dt = CSA_BF16; a.fj.B = B; a.fj.T = m; a.fj.D = D; a.fj.m = m; a.fj.n_out = 1;
  a.fj.c_a = c; a.fj.z_a = z; a.fj.bias_a = bias; a.fj.gain = gain; a.fj.eps = eps;
  a.fj.rope_dims = rope_dims; a.fj.pos0 = block_pos0;
  return attn_common(a, rope_base, N_cap + W, ws, ws_bytes, stream);
}

}  // namespace

CSA_EXPORT int hca_decode_attn(int B, int H, int D, int rope_dims, double rope_base, float scale,
                               const void* q, void* pool, int N_cap, const int32_t* n_entries,
                               int m, const void* c, const void* z, const float* bias,
                               const float* gain, float eps, const int64_t* block_pos0,
                               const void* win, int L_win, const int64_t* win_pos0, int W,
                               const float* sink, const int64_t* q_pos0, void* out, float* lse,
                               void* ws, size_t ws_bytes, void* stream) {
  return hca_decode_common(B, H, D, rope_dims, rope_base, scale, q, pool, N_cap, n_entries, m, c,
                           z, bias, gain, eps, block_pos0, win, L_win, win_pos0, W, sink, q_pos0,
                           out, lse, ws, ws_bytes, (hipStream_t)stream, false);
}

CSA_EXPORT int hca_decode_attn_kvfp8(int B, int H, int D, int rope_dims, double rope_base,
                                     float scale, const void* q, void* pool, int N_cap,
                                     const int32_t* n_entries, int m, const void* c,
                                     const void* z, const float* bias, const float* gain,
                                     float eps, const int64_t* block_pos0, const void* win,
                                     int L_win, const int64_t* win_pos0, int W, const float* sink,
                                     const int64_t* q_pos0, void* out, float* lse, void* ws,
                                     size_t ws_bytes, void* stream) {
  return hca_decode_common(B, H, D, rope_dims, rope_base, scale, q, pool, N_cap, n_entries, m, c,
                           z, bias, gain, eps, block_pos0, win, L_win, win_pos0, W, sink, q_pos0,
                           out, lse, ws, ws_bytes, (hipStream_t)stream, true);
}

// The window-only decode step in one call: the query token's window row
// (the compressor with m = 1) and the attention over the window, through
// the kernels of the HCA path (no pool, no selected indices: with csa set,
// the key list is the K = 0 selection plus the window).
CSA_EXPORT size_t swa_decode_attn_ws_bytes(int B, int H, int D, int W) {
  if (B <= 0 || W <= 0 || !attn_uses_mfma(CSA_BF16, H, D, 0)) return 0;
  return attn_fresh_ws_bytes(B, H, D, W);
}

CSA_EXPORT int swa_decode_attn(int B, int H, int D, int rope_dims, double rope_base, float scale,
                               const void* q, const void* kv, const float* gain, float eps,
                               void* win, int L_win, const int64_t* win_pos0, int W,
                               const float* sink, const int64_t* q_pos0, void* out, float* lse,
                               void* ws, size_t ws_bytes, void* stream) {
  if (!kv || !win || L_win <= 0 || W <= 0) return CSA_ERR_ARG;
  if (gain && !(eps >= 0.f)) return CSA_ERR_ARG;
  if (rope_dims < 0 || rope_dims > D || (rope_dims & 1)) return CSA_ERR_ARG;
  if (!win_pos0 && L_win < W) return CSA_ERR_ARG;  // a ring holds the whole window
  if (!attn_uses_mfma(CSA_BF16, H, D, rope_dims)) return CSA_ERR_UNSUPPORTED;
  AttnArgs a{};
  a.dt = CSA_BF16; a.B = B; a.Tq = 1; a.H = H; a.D = D; a.R = rope_dims;
  a.scale = scale;
  a.q = q; a.pool = nullptr; a.N_cap = 0; a.csa = 1; a.idx = nullptr; a.K = 0;
  a.n_entries = nullptr; a.m = 1;
  a.win = win; a.L_win = L_win; a.win_pos0 = win_pos0; a.W = W;
  a.sink = sink; a.q_pos0 = q_pos0; a.out = out; a.lse = lse;
  a.fresh = 2;
  a.fj.dt = CSA_BF16; a.fj.B = B; a.fj.T = 1; a.fj.D = D; a.fj.m = 1; a.fj.n_out = 1;
  a.fj.c_a = kv; a.fj.gain = gain; a.fj.eps = eps; a.fj.rope_dims = rope_dims;
  a.fj.pos0 = q_pos0;
  return attn_common(a, rope_base, W, ws, ws_bytes, (hipStream_t)stream);
}
