// Host-only stand-ins for libmcs's launchers and sizing helpers, linked with
// the real C-ABI layer (api.hip) into a sanitizer build: every argument check
// of the C ABI then runs under AddressSanitizer and UndefinedBehaviorSanitizer
// on a machine without a GPU.  Each launcher counts its call and returns
// success; the sizing helpers return simple closed forms of the same shape.
#include "../../token_sparse_attention_amd/csrc/mcs_internal.h"

namespace mcs {

int g_launches = 0;

hipError_t run_attention(const uint16_t*, const uint16_t*, const uint16_t*, const int32_t*, const int32_t*,
                         const int32_t*, const uint16_t*, void*, bool, float*, int, int, int, int, int, int, float,
                         hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t run_residual(const uint16_t*, const uint16_t*, uint16_t*, int64_t, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t run_group_mass(const uint16_t*, const uint16_t*, const float*, const int32_t*, float*, int, int, int,
                          int, int, float, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
bool select_fused_fits(int N, int D, int) { return N <= (D == 128 ? 262144 : 131072); }
hipError_t run_select_fused(const uint16_t*, const uint16_t*, const float*, const int32_t*, float*, int32_t*, int,
                            int, int, int, int, int, float, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t run_topk(const float*, int32_t*, int64_t, int, int, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
size_t block_select_ws_bytes(int BH, int N, int D) { return (size_t)BH * ((N + 63) / 64) * D * 4; }
hipError_t run_block_select(const uint16_t*, const uint16_t*, const int32_t*, int32_t*, int32_t*, int, int, int,
                            int, int, float, void*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t run_query_quality(const float*, const float*, const float*, const float*, float*, float*, float*,
                             int64_t, int, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t run_row_sums(const float*, double*, int64_t, int64_t, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
size_t kmeans_ws_bytes(int n, int k) { return ((size_t)n + k) * 4 + 256; }
hipError_t run_kmeans(const uint16_t*, const float*, int, int, int, int, int32_t*, float*, double*, int32_t*,
                      void*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
GroupPlan plan_group(int BH, int N, int D, int C) {
  GroupPlan p{};
  p.levels = 1;
  p.max_slots = 0;
  p.max_nodes = 1;
  p.bytes = (size_t)BH * N * 8 + (size_t)BH * D * 4 * ((N + C - 1) / C);
  return p;
}
hipError_t run_group(const uint16_t*, int32_t*, int, int, int, int, int, void*, const GroupPlan&, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}

}  // namespace mcs
