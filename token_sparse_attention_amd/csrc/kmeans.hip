// Lloyd's k-means of one head's query or key rows, for gfx950: the grouping
// the pages set against exactly-C PDDP groups (ai.info, "Main Findings": the
// alignment inflation of k-means clusters padded to whole tiles; wispaper.ai,
// "Token-level selection needs tile-aligned query groups").
//
// Each round: every point goes to its nearest centre (squared Euclidean
// distance, equal distances to the smaller centre id); the round's inertia is
// the sum of the squared distances to those centres; then every centre
// becomes the mean of its points (a centre without points keeps its place).
//
//   kmeans_assign_kernel  one thread per point, the point in registers; centre
//                         tiles of 32 with their squared norms stream through
//                         LDS (every lane reads the same centre: broadcasts);
//                         distance ranked as |c|^2 - 2 x.c, the first minimum
//                         kept; writes the label and |x - c|^2;
//   kmeans_update_kernel  one workgroup per cluster: scans the labels in
//                         order and adds its points in index order (no
//                         atomics, so the centres do not depend on timing);
//                         writes the mean and the size.
// The inertia of a round is the fixed-order fp64 sum of the per-point
// distances (run_row_sums).
#include "mcs_common.h"
#include "mcs_internal.h"

namespace mcs {

constexpr int KM_TC = 32;      // centres per LDS tile
constexpr int KM_NT = 256;

template <int D>
__global__ __launch_bounds__(KM_NT) void kmeans_norms_kernel(const float* __restrict__ cen, float* __restrict__ cc,
                                                             int k) {
  const int c = blockIdx.x * KM_NT + threadIdx.x;
  if (c >= k) return;
  float s = 0.f;
  for (int d = 0; d < D; ++d) s = fmaf(cen[(size_t)c * D + d], cen[(size_t)c * D + d], s);
  cc[c] = s;
}

template <int D>
__global__ __launch_bounds__(KM_NT) void kmeans_assign_kernel(const uint16_t* __restrict__ x,
                                                              const float* __restrict__ cen,
                                                              const float* __restrict__ cc, int n, int k,
                                                              int32_t* __restrict__ labels,
                                                              float* __restrict__ dist) {
  __shared__ __attribute__((aligned(16))) float tile[KM_TC][D];
  __shared__ float tnorm[KM_TC];
  const int i = blockIdx.x * KM_NT + threadIdx.x;
  const bool valid = i < n;
  float xr[D];
#pragma unroll
  for (int d = 0; d < D; d += 8) {
    const u32x4_t w = valid ? ldg16(x + (size_t)i * D + d) : zero_u32x4();
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      xr[d + 2 * e] = bf16_lo(w[e]);
      xr[d + 2 * e + 1] = bf16_hi(w[e]);
    }
  }
  float best = INFINITY;
  int bl = 0;
  for (int c0 = 0; c0 < k; c0 += KM_TC) {
    const int tc = min(KM_TC, k - c0);
    __syncthreads();
    for (int e = threadIdx.x; e < tc * D; e += KM_NT) tile[e / D][e % D] = cen[(size_t)c0 * D + e];
    if (threadIdx.x < tc) tnorm[threadIdx.x] = cc[c0 + threadIdx.x];
    __syncthreads();
    for (int c = 0; c < tc; ++c) {
      float dot0 = 0.f, dot1 = 0.f;
#pragma unroll
      for (int d = 0; d < D; d += 8) {
        const float4 a = *reinterpret_cast<const float4*>(&tile[c][d]);
        const float4 b = *reinterpret_cast<const float4*>(&tile[c][d + 4]);
        dot0 = fmaf(xr[d], a.x, dot0);
        dot1 = fmaf(xr[d + 1], a.y, dot1);
        dot0 = fmaf(xr[d + 2], a.z, dot0);
        dot1 = fmaf(xr[d + 3], a.w, dot1);
        dot0 = fmaf(xr[d + 4], b.x, dot0);
        dot1 = fmaf(xr[d + 5], b.y, dot1);
        dot0 = fmaf(xr[d + 6], b.z, dot0);
        dot1 = fmaf(xr[d + 7], b.w, dot1);
      }
      const float dd = fmaf(-2.f, dot0 + dot1, tnorm[c]);
      if (dd < best) {
        best = dd;
        bl = c0 + c;
      }
    }
  }
  if (!valid) return;
  labels[i] = bl;
  // squared distance to the chosen centre, computed directly
  const float* cr = cen + (size_t)bl * D;
  float s = 0.f;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    const float t = xr[d] - cr[d];
    s = fmaf(t, t, s);
  }
  dist[i] = s;
}

template <int D>
__global__ __launch_bounds__(KM_NT) void kmeans_update_kernel(const uint16_t* __restrict__ x,
                                                              const int32_t* __restrict__ labels, int n,
                                                              float* __restrict__ cen, int32_t* __restrict__ sizes) {
  constexpr int NW = KM_NT / 64;
  __shared__ uint64_t masks[NW];
  const int c = blockIdx.x, tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  float sum = 0.f;        // dimension tid (tid < D)
  int count = 0;
  for (int i0 = 0; i0 < n; i0 += KM_NT) {
    const int i = i0 + tid;
    const bool mine = i < n && labels[i] == c;
    const uint64_t m = __ballot(mine);
    if (lane == 0) masks[w] = m;
    __syncthreads();
    for (int ww = 0; ww < NW; ++ww) {
      uint64_t mm = masks[ww];
      while (mm) {
        const int b = __builtin_ctzll(mm);
        mm &= mm - 1;
        const int p = i0 + ww * 64 + b;
        if (tid < D) sum += __uint_as_float((uint32_t)x[(size_t)p * D + tid] << 16);
        ++count;
      }
    }
    __syncthreads();
  }
  if (tid < D && count > 0) cen[(size_t)c * D + tid] = sum / (float)count;
  if (tid == 0) sizes[c] = count;
}

__global__ __launch_bounds__(KM_NT) void copy_f32_kernel(const float* __restrict__ a, float* __restrict__ b,
                                                         int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * KM_NT + threadIdx.x;
  if (i < n) b[i] = a[i];
}

size_t kmeans_ws_bytes(int n, int k) { return ((size_t)n + k) * sizeof(float) + 256; }

hipError_t run_kmeans(const uint16_t* x, const float* init, int n, int D, int k, int rounds, int32_t* labels,
                      float* centers, double* inertia, int32_t* sizes, void* ws, hipStream_t s) {
  float* dist = static_cast<float*>(ws);
  float* cc = dist + n;
  const int64_t nc = (int64_t)k * D;
  hipLaunchKernelGGL(copy_f32_kernel, dim3((unsigned)((nc + KM_NT - 1) / KM_NT)), dim3(KM_NT), 0, s, init, centers, nc);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned pb = (unsigned)((n + KM_NT - 1) / KM_NT), cb = (unsigned)((k + KM_NT - 1) / KM_NT);
  for (int r = 0; r < rounds; ++r) {
    if (D == 128) {
      hipLaunchKernelGGL(kmeans_norms_kernel<128>, dim3(cb), dim3(KM_NT), 0, s, centers, cc, k);
      hipLaunchKernelGGL(kmeans_assign_kernel<128>, dim3(pb), dim3(KM_NT), 0, s, x, centers, cc, n, k, labels, dist);
    } else {
      hipLaunchKernelGGL(kmeans_norms_kernel<64>, dim3(cb), dim3(KM_NT), 0, s, centers, cc, k);
      hipLaunchKernelGGL(kmeans_assign_kernel<64>, dim3(pb), dim3(KM_NT), 0, s, x, centers, cc, n, k, labels, dist);
    }
    e = run_row_sums(dist, inertia + r, 1, n, s);
    if (e != hipSuccess) return e;
    if (D == 128)
      hipLaunchKernelGGL(kmeans_update_kernel<128>, dim3(k), dim3(KM_NT), 0, s, x, labels, n, centers, sizes);
    else
      hipLaunchKernelGGL(kmeans_update_kernel<64>, dim3(k), dim3(KM_NT), 0, s, x, labels, n, centers, sizes);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace mcs
