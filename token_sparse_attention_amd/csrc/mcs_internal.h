// Launchers behind the C ABI (arguments already validated by api.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mcs {

// Dense (kv_idx == nullptr, optional lse) or sparse (perm and kv_idx given,
// optional per-group key counts, optional residual or lse, not both) attention.
hipError_t run_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         const int32_t* perm, const int32_t* kv_idx, const int32_t* kv_count,
                         const uint16_t* res, void* o, bool out_f32, float* lse, int B, int H,
                         int N, int D, int C, int K, float scale, hipStream_t s);

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

// Selection diagnostics and the block-sparse comparison (diag.hip).
constexpr int kMaxKeyBlocks = 4096;   // 64-key blocks per head the block selector holds on chip
size_t block_select_ws_bytes(int BH, int N, int D);
hipError_t run_block_select(const uint16_t* q, const uint16_t* k, const int32_t* perm, int32_t* kv_idx,
                            int32_t* kv_count, int BH, int N, int D, int C, int K, float scale, void* ws,
                            hipStream_t s);
hipError_t run_query_quality(const float* lse_d, const float* lse_s, const float* od, const float* os,
                             float* recall, float* l1, float* l1ref, int64_t rows, int D, hipStream_t s);
hipError_t run_row_sums(const float* x, double* out, int64_t rows, int64_t n, hipStream_t s);

// Lloyd's k-means of n rows of D bf16 values (kmeans.hip).
size_t kmeans_ws_bytes(int n, int k);
hipError_t run_kmeans(const uint16_t* x, const float* init, int n, int D, int k, int rounds, int32_t* labels,
                      float* centers, double* inertia, int32_t* sizes, void* ws, hipStream_t s);

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

// Shape of the median-split tree.  A node of g > 1 groups has a left child of
// floor(g/2) groups (C*floor(g/2) queries) and a right child of the rest.
// Repeated halving leaves, d levels below a node of g groups, nodes of
// floor(g/2^d) or floor(g/2^d) + 1 groups, (g mod 2^d) of the latter; so the
// number of split nodes (> 1 group) there is closed-form.
__host__ __device__ inline int split_nodes_below(int g, int d) {
  const int q = g >> d, r = g & ((1 << d) - 1);
  return q >= 2 ? (1 << d) : (q == 1 ? r : 0);
}

// Number of split nodes at tree level `level` of a head of N queries.
__host__ __device__ inline int split_nodes_at(int N, int C, int level) {
  return split_nodes_below((N + C - 1) / C, level);
}

// The rank-th split node (left to right) at `level`: its offset in the head's
// perm row, its size n and group count g (> 1).  Returns false if rank is out
// of range.  Kernels launch one workgroup per split node, so consecutive
// workgroups (which the hardware deals to consecutive XCDs) always have work.
__host__ __device__ inline bool node_by_rank(int N, int C, int level, int rank, int& off, int& n,
                                             int& g) {
  off = 0;
  n = N;
  g = (N + C - 1) / C;
  if (rank < 0 || rank >= split_nodes_below(g, level)) return false;
  for (int i = 0; i < level; ++i) {
    const int half = g / 2, nl = C * half;
    const int left = split_nodes_below(half, level - 1 - i);
    if (rank < left) {
      n = nl;
      g = half;
    } else {
      rank -= left;
      off += nl;
      n -= nl;
      g -= half;
    }
  }
  return g > 1;
}

}  // namespace mcs
