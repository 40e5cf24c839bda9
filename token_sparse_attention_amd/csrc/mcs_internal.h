// Launchers behind the C ABI (arguments already validated by api.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mcs {

// Dense (kv_idx == nullptr, optional lse) or sparse (perm and kv_idx given,
// optional residual) attention.
hipError_t run_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         const int32_t* perm, const int32_t* kv_idx, const uint16_t* res,
                         void* o, bool out_f32, float* lse, int B, int H, int N, int D, int C,
                         int K, float scale, hipStream_t s);

hipError_t run_residual(const uint16_t* od, const uint16_t* osp, uint16_t* r, int64_t n,
                        hipStream_t s);

// Group mass rows of heads [bh0, bh0 + nh): mass[(h - bh0) * G + g][j], j < N.
hipError_t run_group_mass(const uint16_t* q, const uint16_t* k, const float* lse,
                          const int32_t* perm, float* mass, int bh0, int nh, int N, int D,
                          int C, float scale, hipStream_t s);

// Group mass rows as above, each followed in the same workgroup by its top-K
// (idx[(h - bh0) * G + g][0, K)); only where select_fused_fits(N, D, C).
bool select_fused_fits(int N, int D, int C);
hipError_t run_select_fused(const uint16_t* q, const uint16_t* k, const float* lse,
                            const int32_t* perm, float* mass, int32_t* idx, int bh0, int nh,
                            int N, int D, int C, int K, float scale, hipStream_t s);

// Top-K of non-negative rows (ties to the smaller id, ids ascending).
hipError_t run_topk(const float* scores, int32_t* idx, int64_t rows, int n, int K,
                    hipStream_t s);

// Median-split PDDP.
struct GroupPlan {
  int levels;        // number of split levels
  int max_slots;     // partial-moment slots per head (0 if no level needs them)
  int max_nodes;     // node slots of the deepest split level
  size_t proj_off, tmp_off, dir_off, part_off, bytes;
};
GroupPlan plan_group(int BH, int N, int D, int C);
hipError_t run_group(const uint16_t* q, int32_t* perm, int BH, int N, int D, int C, int iters,
                     void* ws, const GroupPlan& plan, hipStream_t s);

// Node geometry of the median-split tree: the node reached from the root by
// the top `level` bits of `slot` (most significant first, 0 = left).  Returns
// false when that node does not exist or is a leaf (<= one group).
__host__ __device__ inline bool node_geom(int N, int C, int level, int slot, int& off, int& n,
                                          int& g) {
  off = 0;
  n = N;
  g = (N + C - 1) / C;
  for (int i = 0; i < level; ++i) {
    if (g <= 1) return false;
    const int half = g / 2, nl = C * half;
    if (((slot >> (level - 1 - i)) & 1) == 0) {
      n = nl;
      g = half;
    } else {
      off += nl;
      n -= nl;
      g -= half;
    }
  }
  return g > 1;
}

}  // namespace mcs
