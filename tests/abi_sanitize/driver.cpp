// Drives every entry point of include/mcs.h through its argument checks (and
// its accepting path, which reaches the host stand-ins of stubs.cpp) in a
// build with AddressSanitizer and UndefinedBehaviorSanitizer on the host code.
// Pointers are fake device addresses: no call dereferences them on the host.
// Exits 0 and prints "sanitize ok" when every status is the expected one.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../../include/mcs.h"

namespace mcs {
extern int g_launches;
}

static int failures = 0;

static void expect(const char* what, mcs_status got, mcs_status want) {
  if (got != want) {
    ++failures;
    fprintf(stderr, "%s: status %d (%s), expected %d; last error: %s\n", what, (int)got, mcs_status_string(got),
            (int)want, mcs_last_error());
  }
}

int main() {
  const uintptr_t A = 0x10000, B = 0x20000, C = 0x30000, D = 0x40000, E = 0x50000, W = 0x80000;
  auto p16 = [](uintptr_t x) { return reinterpret_cast<uint16_t*>(x); };
  auto p32 = [](uintptr_t x) { return reinterpret_cast<int32_t*>(x); };
  auto pf = [](uintptr_t x) { return reinterpret_cast<float*>(x); };
  auto pv = [](uintptr_t x) { return reinterpret_cast<void*>(x); };
  const mcs_dims d = {1, 2, 1000, 128};
  const mcs_dims bad_d = {1, 2, 1000, 96};
  const mcs_dims bad_n = {1, 2, 0, 128};

  // dense
  expect("dense ok", mcs_dense_attn(p16(A), p16(B), p16(C), p16(D), pf(E), d, 0.1f, nullptr), MCS_OK);
  expect("dense null", mcs_dense_attn(nullptr, p16(B), p16(C), p16(D), nullptr, d, 0.1f, nullptr), MCS_E_NULL);
  expect("dense align", mcs_dense_attn(p16(A + 2), p16(B), p16(C), p16(D), nullptr, d, 0.1f, nullptr), MCS_E_ALIGN);
  expect("dense head dim", mcs_dense_attn(p16(A), p16(B), p16(C), p16(D), nullptr, bad_d, 0.1f, nullptr),
         MCS_E_HEAD_DIM);
  expect("dense shape", mcs_dense_attn(p16(A), p16(B), p16(C), p16(D), nullptr, bad_n, 0.1f, nullptr), MCS_E_SHAPE);
  expect("dense scale", mcs_dense_attn(p16(A), p16(B), p16(C), p16(D), nullptr, d, -1.f, nullptr), MCS_E_SCALE);
  expect("dense f32", mcs_dense_attn_f32out(p16(A), p16(B), p16(C), pf(D), nullptr, d, 0.1f, nullptr), MCS_OK);
  // sparse
  expect("sparse ok", mcs_sparse_attn(p16(A), p16(B), p16(C), p32(D), p32(E), nullptr, p16(W), d, 128, 100, 0.1f,
                                      nullptr), MCS_OK);
  expect("sparse budget", mcs_sparse_attn(p16(A), p16(B), p16(C), p32(D), p32(E), nullptr, p16(W), d, 128, 1001,
                                          0.1f, nullptr), MCS_E_BUDGET);
  expect("sparse group", mcs_sparse_attn(p16(A), p16(B), p16(C), p32(D), p32(E), nullptr, p16(W), d, 96, 100, 0.1f,
                                         nullptr), MCS_E_GROUP_SIZE);
  expect("sparse f32", mcs_sparse_attn_f32out(p16(A), p16(B), p16(C), p32(D), p32(E), p16(W), pf(W + 64), d, 128,
                                              100, 0.1f, nullptr), MCS_OK);
  expect("sparse ex ok", mcs_sparse_attn_ex(p16(A), p16(B), p16(C), p32(D), p32(E), p32(W), nullptr, pv(W + 64), 1,
                                            pf(W + 128), d, 128, 100, 0.1f, nullptr), MCS_OK);
  expect("sparse ex both", mcs_sparse_attn_ex(p16(A), p16(B), p16(C), p32(D), p32(E), nullptr, p16(W), pv(W + 64),
                                              0, pf(W + 128), d, 128, 100, 0.1f, nullptr), MCS_E_ARG);
  // residual
  expect("residual ok", mcs_residual_update(p16(A), p16(B), p16(C), 77, nullptr), MCS_OK);
  expect("residual n", mcs_residual_update(p16(A), p16(B), p16(C), 0, nullptr), MCS_E_SHAPE);
  // select
  const size_t ws = mcs_select_workspace(d, 128, 100);
  expect("select ok", mcs_select(p16(A), p16(B), pf(C), p32(D), p32(E), d, 128, 100, 0.1f, pv(W), ws, nullptr),
         MCS_OK);
  expect("select ws", mcs_select(p16(A), p16(B), pf(C), p32(D), p32(E), d, 128, 100, 0.1f, pv(W), ws - 1, nullptr),
         MCS_E_WORKSPACE);
  expect("select two pass", mcs_select_two_pass(p16(A), p16(B), pf(C), p32(D), p32(E), d, 128, 100, 0.1f, pv(W),
                                                mcs_select_workspace_all_heads(d, 128, 100), nullptr), MCS_OK);
  expect("topk ok", mcs_topk(pf(A), p32(B), 3, 10, 5, nullptr), MCS_OK);
  expect("topk K", mcs_topk(pf(A), p32(B), 3, 10, 11, nullptr), MCS_E_BUDGET);
  // group
  const size_t gws = mcs_group_workspace(d, 128);
  expect("group ok", mcs_group(p16(A), p32(B), d, 128, 0, pv(W), gws, nullptr), MCS_OK);
  expect("group steps", mcs_group(p16(A), p32(B), d, 128, 65, pv(W), gws, nullptr), MCS_E_ARG);
  expect("group ws", mcs_group(p16(A), p32(B), d, 128, 0, pv(W), gws - 1, nullptr), MCS_E_WORKSPACE);
  expect("noalloc steps", mcs_group_noalloc(p16(A), p32(B), d, 128, 65, nullptr), MCS_E_ARG);
  expect("noalloc null", mcs_group_noalloc(nullptr, p32(B), d, 128, 0, nullptr), MCS_E_NULL);
  // diagnostics, block selection, k-means
  const size_t bws = mcs_select_blocks_workspace(d);
  expect("blocks ok", mcs_select_blocks(p16(A), p16(B), p32(C), p32(D), p32(E), d, 128, 128, 0.1f, pv(W), bws,
                                        nullptr), MCS_OK);
  expect("blocks K", mcs_select_blocks(p16(A), p16(B), p32(C), p32(D), p32(E), d, 128, 100, 0.1f, pv(W), bws,
                                       nullptr), MCS_E_BUDGET);
  expect("quality ok", mcs_query_quality(pf(A), pf(B), pf(C), pf(D), pf(E), pf(W), pf(W + 64), d, nullptr), MCS_OK);
  expect("row sums ok", mcs_row_sums(pf(A), reinterpret_cast<double*>(B), 2, 9, nullptr), MCS_OK);
  expect("row sums shape", mcs_row_sums(pf(A), reinterpret_cast<double*>(B), 0, 9, nullptr), MCS_E_SHAPE);
  const size_t kws = mcs_kmeans_workspace(1000, 10);
  expect("kmeans ok", mcs_kmeans(p16(A), pf(B), 1000, 128, 10, 3, p32(C), pf(D), reinterpret_cast<double*>(E),
                                 p32(W), pv(W + 4096), kws, nullptr), MCS_OK);
  expect("kmeans k", mcs_kmeans(p16(A), pf(B), 1000, 128, 1001, 3, p32(C), pf(D), reinterpret_cast<double*>(E),
                                p32(W), pv(W + 4096), kws, nullptr), MCS_E_ARG);
  for (int s = 0; s <= 10; ++s)
    if (strlen(mcs_status_string((mcs_status)s)) == 0) ++failures;
  if (mcs_version() <= 0) ++failures;
  // accepted calls: 16 launcher calls (mcs_select with a one-head workspace
  // runs its 2 heads as 2 chunks; the two-pass select is 2 kernels)
  if (mcs::g_launches != 16) {
    ++failures;
    fprintf(stderr, "%d launches reached the stand-ins, expected 16\n", mcs::g_launches);
  }
  if (failures) return 1;
  printf("sanitize ok\n");
  return 0;
}
