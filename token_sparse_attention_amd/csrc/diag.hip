// Selection diagnostics and the block-sparse comparison, for gfx950.
//
// The ai.info page ("Methodology in Plain English", "Main Findings") and the
// wispaper.ai explainer ("Mean-pooled block scoring misses high-mass tokens")
// score a selection by attention recall (the dense attention mass it keeps)
// and by the relative L1 error of the output renormalised over the kept keys,
// and set the token selection against standard block-sparse attention, which
// keeps whole blocks of 64 consecutive keys chosen by the score of the query
// block's mean query against the key block's mean key.
//
//   block_means_kernel   mean key of every 64-key block of a head (fp32; the
//                        last block may be short);
//   block_select_kernel  one workgroup per query group: the group's mean
//                        query, its score against every key block, the
//                        nblk best blocks (radix select, equal scores to the
//                        smaller block id), written out as token ids of the
//                        blocks in ascending order with the number of real
//                        keys (only the last block can be short);
//   query_quality_kernel per query: recall = exp(lse_sparse - lse_dense) (the
//                        dense probability mass on the kept keys), the L1
//                        distance of the sparse output from the dense one and
//                        the L1 norm of the dense one;
//   row_sums_kernel      fp64 sums of rows in a fixed order.
#include "mcs_common.h"
#include "mcs_internal.h"
#include "mcs_radix.h"

namespace mcs {

constexpr int KVB = 64;      // keys per KV block
constexpr int BS_NT = 256;

template <int D>
__global__ __launch_bounds__(D) void block_means_kernel(const uint16_t* __restrict__ k, float* __restrict__ kbar,
                                                        int N, int NB) {
  const int b = blockIdx.x, bh = blockIdx.y, d = threadIdx.x;
  const uint16_t* kh = k + (size_t)bh * N * D;
  const int r0 = b * KVB, r1 = min(N, r0 + KVB);
  float s = 0.f;
  for (int r = r0; r < r1; ++r) s += __uint_as_float((uint32_t)kh[(size_t)r * D + d] << 16);
  kbar[((size_t)bh * NB + b) * D + d] = s / (float)(r1 - r0);
}

struct BlockSelParams {
  const uint16_t* q;
  const int32_t* perm;
  const float* kbar;
  int32_t* kv_idx;
  int32_t* kv_count;
  int32_t N, C, G, K, NB, nblk;
  float scale;
};

template <int D>
__global__ __launch_bounds__(BS_NT) void block_select_kernel(BlockSelParams p) {
  constexpr int PARTS = BS_NT / D;
  __shared__ float qbar[D];
  __shared__ float part[PARTS][D];
  __shared__ uint32_t keys[kMaxKeyBlocks];
  __shared__ RadixLds<BS_NT> L;
  __shared__ int last_selected;
  const int g = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const size_t head = (size_t)bh * p.N;
  const int m0 = g * p.C, m1 = min(p.N, m0 + p.C);
  if (tid == 0) last_selected = 0;
  // the group's mean query (members summed in a fixed order)
  {
    const int d = tid % D, pi = tid / D;
    float s = 0.f;
    for (int m = m0 + pi; m < m1; m += PARTS) {
      const int row = clamp_id(p.perm[head + m], p.N);
      s += __uint_as_float((uint32_t)p.q[(head + row) * D + d] << 16);
    }
    part[pi][d] = s;
  }
  __syncthreads();
  if (tid < D) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < PARTS; ++i) s += part[i][tid];
    qbar[tid] = s / (float)(m1 - m0);
  }
  __syncthreads();
  // scores of all key blocks, as selection keys: larger score, smaller key
  const float* __restrict__ kb = p.kbar + (size_t)bh * p.NB * D;
  for (int b = tid; b < p.NB; b += BS_NT) {
    const float4* kr = reinterpret_cast<const float4*>(kb + (size_t)b * D);
    float s = 0.f;
#pragma unroll 8
    for (int c = 0; c < D / 4; ++c) {
      const float4 v = kr[c];
      s = fmaf(qbar[4 * c], v.x, s);
      s = fmaf(qbar[4 * c + 1], v.y, s);
      s = fmaf(qbar[4 * c + 2], v.z, s);
      s = fmaf(qbar[4 * c + 3], v.w, s);
    }
    keys[b] = ~float_order_key(s * p.scale);
  }
  __syncthreads();
  auto key = [&](int i) -> uint32_t { return keys[i]; };
  uint32_t T;
  int need;
  radix_select_smallest<BS_NT>(key, p.NB, p.nblk, L, T, need);
  int32_t* __restrict__ out = p.kv_idx + ((size_t)bh * p.G + g) * p.K;
  ordered_compact<BS_NT>(key, p.NB, T, need, L, [&](int i, bool sel, int rank) {
    if (!sel) return;
    for (int r = 0; r < KVB; ++r) {
      const int id = i * KVB + r;
      out[rank * KVB + r] = id < p.N ? id : p.N - 1;   // past N: padding beyond the count
    }
    if (i == p.NB - 1) last_selected = 1;
  });
  __syncthreads();
  if (tid == 0) {
    const int tail = p.N - (p.NB - 1) * KVB;           // keys in the last block
    p.kv_count[(size_t)bh * p.G + g] = p.nblk * KVB - (last_selected ? KVB - tail : 0);
  }
}

template <int D>
__global__ __launch_bounds__(256) void query_quality_kernel(const float* __restrict__ lse_d,
                                                            const float* __restrict__ lse_s,
                                                            const float* __restrict__ od,
                                                            const float* __restrict__ os,
                                                            float* __restrict__ recall,
                                                            float* __restrict__ l1,
                                                            float* __restrict__ l1ref, int64_t rows) {
  constexpr int PER = D / 64;   // channels per lane
  const int lane = threadIdx.x & 63;
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
  for (int64_t r = wave; r < rows; r += nwaves) {
    float a = 0.f, b = 0.f;
#pragma unroll
    for (int c = 0; c < PER; ++c) {
      const float x = od[r * D + lane + 64 * c], y = os[r * D + lane + 64 * c];
      a += fabsf(y - x);
      b += fabsf(x);
    }
    a = wave_sum(a);
    b = wave_sum(b);
    if (lane == 0) {
      recall[r] = expf(lse_s[r] - lse_d[r]);
      l1[r] = a;
      l1ref[r] = b;
    }
  }
}

__global__ __launch_bounds__(256) void row_sums_kernel(const float* __restrict__ x, double* __restrict__ out,
                                                       int64_t n) {
  __shared__ double red[256];
  const int64_t row = blockIdx.x;
  const float* xr = x + row * n;
  double s = 0.0;
  for (int64_t i = threadIdx.x; i < n; i += 256) s += (double)xr[i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[row] = red[0];
}

size_t block_select_ws_bytes(int BH, int N, int D) {
  const size_t NB = ((size_t)N + KVB - 1) / KVB;
  return (size_t)BH * NB * D * sizeof(float);
}

hipError_t run_block_select(const uint16_t* q, const uint16_t* k, const int32_t* perm, int32_t* kv_idx,
                            int32_t* kv_count, int BH, int N, int D, int C, int K, float scale, void* ws,
                            hipStream_t s) {
  BlockSelParams p;
  p.q = q;
  p.perm = perm;
  p.kbar = static_cast<float*>(ws);
  p.kv_idx = kv_idx;
  p.kv_count = kv_count;
  p.N = N;
  p.C = C;
  p.G = (N + C - 1) / C;
  p.K = K;
  p.NB = (N + KVB - 1) / KVB;
  p.nblk = K / KVB;
  p.scale = scale;
  if (D == 128) {
    hipLaunchKernelGGL(block_means_kernel<128>, dim3(p.NB, BH), dim3(128), 0, s, k, static_cast<float*>(ws), N,
                       p.NB);
    hipLaunchKernelGGL(block_select_kernel<128>, dim3(p.G, BH), dim3(BS_NT), 0, s, p);
  } else {
    hipLaunchKernelGGL(block_means_kernel<64>, dim3(p.NB, BH), dim3(64), 0, s, k, static_cast<float*>(ws), N,
                       p.NB);
    hipLaunchKernelGGL(block_select_kernel<64>, dim3(p.G, BH), dim3(BS_NT), 0, s, p);
  }
  return hipGetLastError();
}

hipError_t run_query_quality(const float* lse_d, const float* lse_s, const float* od, const float* os,
                             float* recall, float* l1, float* l1ref, int64_t rows, int D, hipStream_t s) {
  int64_t blocks = (rows + 3) / 4;              // 4 waves (rows) per workgroup per pass
  if (blocks > 256 * 16) blocks = 256 * 16;
  if (D == 128)
    hipLaunchKernelGGL(query_quality_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, s, lse_d, lse_s, od, os,
                       recall, l1, l1ref, rows);
  else
    hipLaunchKernelGGL(query_quality_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, s, lse_d, lse_s, od, os,
                       recall, l1, l1ref, rows);
  return hipGetLastError();
}

hipError_t run_row_sums(const float* x, double* out, int64_t rows, int64_t n, hipStream_t s) {
  hipLaunchKernelGGL(row_sums_kernel, dim3((unsigned)rows), dim3(256), 0, s, x, out, n);
  return hipGetLastError();
}

}  // namespace mcs
