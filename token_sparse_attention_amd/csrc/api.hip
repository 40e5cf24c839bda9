// C ABI of libmcs: argument validation, workspace sizing and launches.
// Validation happens before any HIP call, so a rejected call enqueues nothing.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/mcs.h"
#include "mcs_internal.h"

namespace {

thread_local char g_err[512] = "";

mcs_status fail(mcs_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
mcs_status fail(mcs_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

mcs_status ok() {
  g_err[0] = '\0';
  return MCS_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define REQUIRE_PTR(p)                                                         \
  do {                                                                         \
    if ((p) == nullptr) return fail(MCS_E_NULL, "%s: %s is NULL", fn, #p);     \
    if (!aligned16(p)) return fail(MCS_E_ALIGN, "%s: %s is not 16-byte aligned", fn, #p); \
  } while (0)

#define OPTIONAL_PTR(p)                                                        \
  do {                                                                         \
    if ((p) != nullptr && !aligned16(p))                                       \
      return fail(MCS_E_ALIGN, "%s: %s is not 16-byte aligned", fn, #p);       \
  } while (0)

mcs_status check_dims(const char* fn, mcs_dims d) {
  if (d.B < 1 || d.H < 1 || d.N < 1)
    return fail(MCS_E_SHAPE, "%s: B, H, N must be >= 1 (got %d, %d, %d)", fn, d.B, d.H, d.N);
  if (d.D != 64 && d.D != 128) return fail(MCS_E_HEAD_DIM, "%s: D must be 64 or 128 (got %d)", fn, d.D);
  const int64_t bh = (int64_t)d.B * d.H;
  if (bh > 65535) return fail(MCS_E_SHAPE, "%s: B*H = %lld exceeds 65535", fn, (long long)bh);
  if (bh * d.N > INT32_MAX)
    return fail(MCS_E_SHAPE, "%s: B*H*N = %lld exceeds 2^31-1", fn, (long long)(bh * d.N));
  if ((int64_t)d.N * d.D * 2 > INT32_MAX)
    return fail(MCS_E_SHAPE, "%s: one head's K (N*D*2 bytes) exceeds 2^31-1", fn);
  return MCS_OK;
}

mcs_status check_group_size(const char* fn, int32_t C) {
  if (C != 64 && C != 128) return fail(MCS_E_GROUP_SIZE, "%s: C must be 64 or 128 (got %d)", fn, C);
  return MCS_OK;
}

mcs_status check_budget(const char* fn, mcs_dims d, int32_t C, int32_t K) {
  if (K < 1 || K > d.N) return fail(MCS_E_BUDGET, "%s: K must be in [1, N=%d] (got %d)", fn, d.N, K);
  const int64_t G = (d.N + (int64_t)C - 1) / C;
  if ((int64_t)d.B * d.H * G * K > INT64_MAX / 8)
    return fail(MCS_E_SHAPE, "%s: kv_idx size overflows", fn);
  return MCS_OK;
}

mcs_status check_scale(const char* fn, float scale) {
  if (!(scale > 0.f) || !isfinite(scale))
    return fail(MCS_E_SCALE, "%s: scale must be finite and > 0 (got %g)", fn, (double)scale);
  return MCS_OK;
}

mcs_status launched(const char* fn, hipError_t e) {
  if (e != hipSuccess) return fail(MCS_E_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

size_t select_ws_per_head(mcs_dims d, int32_t C) {
  const size_t G = ((size_t)d.N + C - 1) / C;
  return G * (size_t)d.N * sizeof(float);
}

}  // namespace

// Scratch of mcs_group_noalloc: a static device array, so that call needs no
// allocation.  Each device the library's code is loaded on holds its own
// copy until the process ends.  Host code never uses the symbol itself (its
// host-side name is a stand-in, not a device address): the device address
// comes from hipGetSymbolAddress, looked up once per device.
constexpr size_t kGroupScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kGroupScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the calling thread's current device.
hipError_t group_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

static mcs_status dense_common(const char* fn, const uint16_t* q, const uint16_t* k,
                               const uint16_t* v, void* o, bool out_f32, float* lse, mcs_dims d,
                               float scale, void* stream) {
  REQUIRE_PTR(q);
  REQUIRE_PTR(k);
  REQUIRE_PTR(v);
  REQUIRE_PTR(o);
  OPTIONAL_PTR(lse);
  mcs_status st;
  if ((st = check_dims(fn, d)) != MCS_OK) return st;
  if ((st = check_scale(fn, scale)) != MCS_OK) return st;
  const int C = 128;   // query rows per workgroup
  return launched(fn, mcs::run_attention(q, k, v, nullptr, nullptr, nullptr, nullptr, o, out_f32, lse,
                                         d.B, d.H, d.N, d.D, C, d.N, scale, (hipStream_t)stream));
}

mcs_status mcs_dense_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                          float* lse, mcs_dims d, float scale, void* stream) {
  return dense_common("mcs_dense_attn", q, k, v, o, false, lse, d, scale, stream);
}

mcs_status mcs_dense_attn_f32out(const uint16_t* q, const uint16_t* k, const uint16_t* v, float* o,
                                 float* lse, mcs_dims d, float scale, void* stream) {
  return dense_common("mcs_dense_attn_f32out", q, k, v, o, true, lse, d, scale, stream);
}

static mcs_status sparse_common(const char* fn, const uint16_t* q, const uint16_t* k,
                                const uint16_t* v, const int32_t* perm, const int32_t* kv_idx,
                                const int32_t* kv_count, const uint16_t* residual, void* o,
                                bool out_f32, float* lse, mcs_dims d, int32_t C, int32_t K,
                                float scale, void* stream) {
  REQUIRE_PTR(q);
  REQUIRE_PTR(k);
  REQUIRE_PTR(v);
  REQUIRE_PTR(perm);
  REQUIRE_PTR(kv_idx);
  OPTIONAL_PTR(kv_count);
  OPTIONAL_PTR(residual);
  OPTIONAL_PTR(lse);
  REQUIRE_PTR(o);
  mcs_status st;
  if ((st = check_dims(fn, d)) != MCS_OK) return st;
  if ((st = check_group_size(fn, C)) != MCS_OK) return st;
  if ((st = check_budget(fn, d, C, K)) != MCS_OK) return st;
  if ((st = check_scale(fn, scale)) != MCS_OK) return st;
  if (residual != nullptr && lse != nullptr)
    return fail(MCS_E_ARG, "%s: residual and lse cannot both be given", fn);
  return launched(fn, mcs::run_attention(q, k, v, perm, kv_idx, kv_count, residual, o, out_f32, lse,
                                         d.B, d.H, d.N, d.D, C, K, scale, (hipStream_t)stream));
}

mcs_status mcs_sparse_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                           const int32_t* perm, const int32_t* kv_idx, const uint16_t* residual,
                           uint16_t* o, mcs_dims d, int32_t C, int32_t K, float scale,
                           void* stream) {
  return sparse_common("mcs_sparse_attn", q, k, v, perm, kv_idx, nullptr, residual, o, false, nullptr,
                       d, C, K, scale, stream);
}

mcs_status mcs_sparse_attn_f32out(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                  const int32_t* perm, const int32_t* kv_idx,
                                  const uint16_t* residual, float* o, mcs_dims d, int32_t C,
                                  int32_t K, float scale, void* stream) {
  return sparse_common("mcs_sparse_attn_f32out", q, k, v, perm, kv_idx, nullptr, residual, o, true,
                       nullptr, d, C, K, scale, stream);
}

mcs_status mcs_sparse_attn_ex(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              const int32_t* perm, const int32_t* kv_idx, const int32_t* kv_count,
                              const uint16_t* residual, void* o, int32_t o_f32, float* lse,
                              mcs_dims d, int32_t C, int32_t K, float scale, void* stream) {
  return sparse_common("mcs_sparse_attn_ex", q, k, v, perm, kv_idx, kv_count, residual, o, o_f32 != 0,
                       lse, d, C, K, scale, stream);
}

mcs_status mcs_residual_update(const uint16_t* o_dense, const uint16_t* o_sparse,
                               uint16_t* residual, int64_t n_elems, void* stream) {
  const char* fn = "mcs_residual_update";
  REQUIRE_PTR(o_dense);
  REQUIRE_PTR(o_sparse);
  REQUIRE_PTR(residual);
  if (n_elems < 1) return fail(MCS_E_SHAPE, "%s: n_elems must be >= 1 (got %lld)", fn, (long long)n_elems);
  return launched(fn, mcs::run_residual(o_dense, o_sparse, residual, n_elems, (hipStream_t)stream));
}

size_t mcs_select_workspace(mcs_dims d, int32_t C, int32_t K) {
  (void)K;
  if (d.N < 1 || (C != 64 && C != 128)) return 0;
  return select_ws_per_head(d, C);
}

size_t mcs_select_workspace_all_heads(mcs_dims d, int32_t C, int32_t K) {
  (void)K;
  if (d.N < 1 || d.B < 1 || d.H < 1 || (C != 64 && C != 128)) return 0;
  return select_ws_per_head(d, C) * (size_t)d.B * (size_t)d.H;
}

static mcs_status select_impl(const char* fn, bool fused, const uint16_t* q, const uint16_t* k,
                              const float* lse, const int32_t* perm, int32_t* kv_idx, mcs_dims d,
                              int32_t C, int32_t K, float scale, void* ws, size_t ws_bytes,
                              void* stream) {
  REQUIRE_PTR(q);
  REQUIRE_PTR(k);
  REQUIRE_PTR(lse);
  REQUIRE_PTR(perm);
  REQUIRE_PTR(kv_idx);
  mcs_status st;
  if ((st = check_dims(fn, d)) != MCS_OK) return st;
  if ((st = check_group_size(fn, C)) != MCS_OK) return st;
  if ((st = check_budget(fn, d, C, K)) != MCS_OK) return st;
  if ((st = check_scale(fn, scale)) != MCS_OK) return st;
  const size_t per_head = select_ws_per_head(d, C);
  if (ws == nullptr || ws_bytes < per_head)
    return fail(MCS_E_WORKSPACE, "%s: workspace of %zu bytes given, at least %zu needed", fn,
                ws == nullptr ? (size_t)0 : ws_bytes, per_head);
  if (!aligned16(ws)) return fail(MCS_E_ALIGN, "%s: ws is not 16-byte aligned", fn);
  const int BH = d.B * d.H;
  const int G = (d.N + C - 1) / C;
  size_t fit = ws_bytes / per_head;
  int chunk = fit >= (size_t)BH ? BH : (int)fit;
  hipStream_t s = (hipStream_t)stream;
  float* mass = static_cast<float*>(ws);
  for (int bh0 = 0; bh0 < BH; bh0 += chunk) {
    const int nh = BH - bh0 < chunk ? BH - bh0 : chunk;
    int32_t* idx = kv_idx + (size_t)bh0 * G * K;
    hipError_t e;
    if (fused) {
      e = mcs::run_select_fused(q, k, lse, perm, mass, idx, bh0, nh, d.N, d.D, C, K, scale, s);
    } else {
      e = mcs::run_group_mass(q, k, lse, perm, mass, bh0, nh, d.N, d.D, C, scale, s);
      if (e == hipSuccess) e = mcs::run_topk(mass, idx, (int64_t)nh * G, d.N, K, s);
    }
    if (e != hipSuccess) return launched(fn, e);
  }
  return ok();
}

mcs_status mcs_select(const uint16_t* q, const uint16_t* k, const float* lse, const int32_t* perm,
                      int32_t* kv_idx, mcs_dims d, int32_t C, int32_t K, float scale, void* ws,
                      size_t ws_bytes, void* stream) {
  const bool fused = d.N >= 1 && (d.D == 64 || d.D == 128) && (C == 64 || C == 128) &&
                     mcs::select_fused_fits(d.N, d.D, C);
  return select_impl("mcs_select", fused, q, k, lse, perm, kv_idx, d, C, K, scale, ws, ws_bytes,
                     stream);
}

mcs_status mcs_select_two_pass(const uint16_t* q, const uint16_t* k, const float* lse,
                               const int32_t* perm, int32_t* kv_idx, mcs_dims d, int32_t C,
                               int32_t K, float scale, void* ws, size_t ws_bytes, void* stream) {
  return select_impl("mcs_select_two_pass", false, q, k, lse, perm, kv_idx, d, C, K, scale, ws,
                     ws_bytes, stream);
}

mcs_status mcs_topk(const float* scores, int32_t* idx, int64_t rows, int32_t n, int32_t K,
                    void* stream) {
  const char* fn = "mcs_topk";
  REQUIRE_PTR(scores);
  REQUIRE_PTR(idx);
  if (rows < 1 || n < 1) return fail(MCS_E_SHAPE, "%s: rows and n must be >= 1", fn);
  if (K < 1 || K > n) return fail(MCS_E_BUDGET, "%s: K must be in [1, n=%d] (got %d)", fn, n, K);
  return launched(fn, mcs::run_topk(scores, idx, rows, n, K, (hipStream_t)stream));
}

size_t mcs_group_workspace(mcs_dims d, int32_t C) {
  if (d.B < 1 || d.H < 1 || d.N < 1 || (d.D != 64 && d.D != 128) || (C != 64 && C != 128)) return 0;
  return mcs::plan_group(d.B * d.H, d.N, d.D, C).bytes;
}

mcs_status mcs_group(const uint16_t* q, int32_t* perm, mcs_dims d, int32_t C, int32_t lanczos_steps,
                     void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "mcs_group";
  REQUIRE_PTR(q);
  REQUIRE_PTR(perm);
  mcs_status st;
  if ((st = check_dims(fn, d)) != MCS_OK) return st;
  if ((st = check_group_size(fn, C)) != MCS_OK) return st;
  if (lanczos_steps > 64)
    return fail(MCS_E_ARG, "%s: lanczos_steps must be <= 64 (got %d)", fn, lanczos_steps);
  const mcs::GroupPlan plan = mcs::plan_group(d.B * d.H, d.N, d.D, C);
  if (ws == nullptr || ws_bytes < plan.bytes)
    return fail(MCS_E_WORKSPACE, "%s: workspace of %zu bytes given, at least %zu needed", fn,
                ws == nullptr ? (size_t)0 : ws_bytes, plan.bytes);
  if (!aligned16(ws)) return fail(MCS_E_ALIGN, "%s: ws is not 16-byte aligned", fn);
  return launched(fn, mcs::run_group(q, perm, d.B * d.H, d.N, d.D, C, lanczos_steps, ws, plan,
                                     (hipStream_t)stream));
}

mcs_status mcs_group_noalloc(const uint16_t* q, int32_t* perm, mcs_dims d, int32_t C,
                             int32_t lanczos_steps, void* stream) {
  const char* fn = "mcs_group_noalloc";
  REQUIRE_PTR(q);
  REQUIRE_PTR(perm);
  mcs_status st;
  if ((st = check_dims(fn, d)) != MCS_OK) return st;
  if ((st = check_group_size(fn, C)) != MCS_OK) return st;
  if (lanczos_steps > 64)
    return fail(MCS_E_ARG, "%s: lanczos_steps must be <= 64 (got %d)", fn, lanczos_steps);
  const int BH = d.B * d.H;
  const size_t one = mcs::plan_group(1, d.N, d.D, C).bytes;
  if (one > kGroupScratchBytes)
    return fail(MCS_E_WORKSPACE, "%s: one head needs %zu bytes of scratch, more than the %zu the library holds",
                fn, one, kGroupScratchBytes);
  // heads per launch sequence: as many as the scratch holds
  int nh = (int)((size_t)BH < kGroupScratchBytes / one ? (size_t)BH : kGroupScratchBytes / one);
  while (nh > 1 && mcs::plan_group(nh, d.N, d.D, C).bytes > kGroupScratchBytes) --nh;
  void* ws = nullptr;
  hipError_t e = group_scratch(&ws);
  if (e != hipSuccess) return launched(fn, e);
  for (int bh0 = 0; bh0 < BH; bh0 += nh) {
    const int n = BH - bh0 < nh ? BH - bh0 : nh;
    const mcs::GroupPlan plan = mcs::plan_group(n, d.N, d.D, C);
    e = mcs::run_group(q + (size_t)bh0 * d.N * d.D, perm + (size_t)bh0 * d.N, n, d.N, d.D, C,
                       lanczos_steps, ws, plan, (hipStream_t)stream);
    if (e != hipSuccess) return launched(fn, e);
  }
  return ok();
}

size_t mcs_select_blocks_workspace(mcs_dims d) {
  if (d.B < 1 || d.H < 1 || d.N < 1 || (d.D != 64 && d.D != 128)) return 0;
  return mcs::block_select_ws_bytes(d.B * d.H, d.N, d.D);
}

mcs_status mcs_select_blocks(const uint16_t* q, const uint16_t* k, const int32_t* perm, int32_t* kv_idx,
                             int32_t* kv_count, mcs_dims d, int32_t C, int32_t K, float scale, void* ws,
                             size_t ws_bytes, void* stream) {
  const char* fn = "mcs_select_blocks";
  REQUIRE_PTR(q);
  REQUIRE_PTR(k);
  REQUIRE_PTR(perm);
  REQUIRE_PTR(kv_idx);
  REQUIRE_PTR(kv_count);
  mcs_status st;
  if ((st = check_dims(fn, d)) != MCS_OK) return st;
  if ((st = check_group_size(fn, C)) != MCS_OK) return st;
  if ((st = check_scale(fn, scale)) != MCS_OK) return st;
  const int64_t NB = ((int64_t)d.N + 63) / 64;
  if (NB > mcs::kMaxKeyBlocks)
    return fail(MCS_E_SHAPE, "%s: N = %d gives %lld key blocks, more than %d", fn, d.N, (long long)NB,
                mcs::kMaxKeyBlocks);
  if (K < 64 || K % 64 != 0 || K / 64 > NB)
    return fail(MCS_E_BUDGET, "%s: K must be a multiple of 64 in [64, 64 * %lld] (got %d)", fn,
                (long long)NB, K);
  const size_t need = mcs::block_select_ws_bytes(d.B * d.H, d.N, d.D);
  if (ws == nullptr || ws_bytes < need)
    return fail(MCS_E_WORKSPACE, "%s: workspace of %zu bytes given, at least %zu needed", fn,
                ws == nullptr ? (size_t)0 : ws_bytes, need);
  if (!aligned16(ws)) return fail(MCS_E_ALIGN, "%s: ws is not 16-byte aligned", fn);
  return launched(fn, mcs::run_block_select(q, k, perm, kv_idx, kv_count, d.B * d.H, d.N, d.D, C, K, scale,
                                            ws, (hipStream_t)stream));
}

mcs_status mcs_query_quality(const float* lse_dense, const float* lse_sparse, const float* o_dense,
                             const float* o_sparse, float* recall, float* l1, float* l1_ref, mcs_dims d,
                             void* stream) {
  const char* fn = "mcs_query_quality";
  REQUIRE_PTR(lse_dense);
  REQUIRE_PTR(lse_sparse);
  REQUIRE_PTR(o_dense);
  REQUIRE_PTR(o_sparse);
  REQUIRE_PTR(recall);
  REQUIRE_PTR(l1);
  REQUIRE_PTR(l1_ref);
  mcs_status st;
  if ((st = check_dims(fn, d)) != MCS_OK) return st;
  return launched(fn, mcs::run_query_quality(lse_dense, lse_sparse, o_dense, o_sparse, recall, l1, l1_ref,
                                             (int64_t)d.B * d.H * d.N, d.D, (hipStream_t)stream));
}

mcs_status mcs_row_sums(const float* x, double* out, int64_t rows, int64_t n, void* stream) {
  const char* fn = "mcs_row_sums";
  REQUIRE_PTR(x);
  REQUIRE_PTR(out);
  if (rows < 1 || n < 1 || rows > INT32_MAX)
    return fail(MCS_E_SHAPE, "%s: rows must be in [1, 2^31) and n >= 1 (got %lld, %lld)", fn, (long long)rows,
                (long long)n);
  return launched(fn, mcs::run_row_sums(x, out, rows, n, (hipStream_t)stream));
}

size_t mcs_kmeans_workspace(int32_t n, int32_t k) {
  if (n < 1 || k < 1) return 0;
  return mcs::kmeans_ws_bytes(n, k);
}

mcs_status mcs_kmeans(const uint16_t* x, const float* init, int32_t n, int32_t D, int32_t k, int32_t rounds,
                      int32_t* labels, float* centers, double* inertia, int32_t* sizes, void* ws,
                      size_t ws_bytes, void* stream) {
  const char* fn = "mcs_kmeans";
  REQUIRE_PTR(x);
  REQUIRE_PTR(init);
  REQUIRE_PTR(labels);
  REQUIRE_PTR(centers);
  REQUIRE_PTR(inertia);
  REQUIRE_PTR(sizes);
  if (D != 64 && D != 128) return fail(MCS_E_HEAD_DIM, "%s: D must be 64 or 128 (got %d)", fn, D);
  if (n < 1 || (int64_t)n * D > INT32_MAX)
    return fail(MCS_E_SHAPE, "%s: n must be >= 1 with n*D < 2^31 (got n = %d)", fn, n);
  if (k < 1 || k > n) return fail(MCS_E_ARG, "%s: k must be in [1, n=%d] (got %d)", fn, n, k);
  if (rounds < 1 || rounds > 10000) return fail(MCS_E_ARG, "%s: rounds must be in [1, 10000] (got %d)", fn, rounds);
  const size_t need = mcs::kmeans_ws_bytes(n, k);
  if (ws == nullptr || ws_bytes < need)
    return fail(MCS_E_WORKSPACE, "%s: workspace of %zu bytes given, at least %zu needed", fn,
                ws == nullptr ? (size_t)0 : ws_bytes, need);
  if (!aligned16(ws)) return fail(MCS_E_ALIGN, "%s: ws is not 16-byte aligned", fn);
  return launched(fn, mcs::run_kmeans(x, init, n, D, k, rounds, labels, centers, inertia, sizes, ws,
                                      (hipStream_t)stream));
}

const char* mcs_status_string(mcs_status s) {
  switch (s) {
    case MCS_OK: return "ok";
    case MCS_E_NULL: return "a required pointer is NULL";
    case MCS_E_SHAPE: return "invalid shape";
    case MCS_E_HEAD_DIM: return "head dimension must be 64 or 128";
    case MCS_E_GROUP_SIZE: return "group size must be 64 or 128";
    case MCS_E_BUDGET: return "KV budget K out of range";
    case MCS_E_SCALE: return "scale must be finite and > 0";
    case MCS_E_ALIGN: return "pointer not 16-byte aligned";
    case MCS_E_WORKSPACE: return "workspace missing or too small";
    case MCS_E_HIP: return "HIP launch failed";
    case MCS_E_ARG: return "argument out of range";
  }
  return "unknown status";
}

const char* mcs_last_error(void) { return g_err; }

int32_t mcs_version(void) { return MCS_VERSION; }

}  // extern "C"
