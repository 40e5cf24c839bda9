// Second pass of the exact selector for gfx950: group mass and top-K.
//
// The ai.info page ("Methodology in Plain English") describes the selection as
// a two-pass kernel: the first pass (the dense attention with row LSE) and a
// second pass that recomputes QK scores, recovers the attention probabilities
// from the LSE and aggregates them per query group before a top-K.  The
// agihunt.info method paragraphs state the objective: for each group, the K
// KV tokens with the largest summed attention weight.
//
// group_mass_kernel: one workgroup per (head, group).  The group's C queries
// (gathered by perm) stay in registers as MFMA A fragments; all N keys stream
// through LDS in tiles of 64 (double buffered).  S = Q K^T on MFMA leaves one
// key per lane column, so each lane sums exp2(s*scale*log2e - lse_i*log2e)
// over its 16 query rows, adds its partner lane's half, and the C/32 waves
// combine through LDS in a fixed order.  One fp32 mass row of N values per
// group goes to the workspace.
//
// topk_kernel: one 1024-thread workgroup per mass row: 4-pass radix select of
// the K-th largest value (8 bits per pass, per-wave LDS histograms), then an
// order-preserving compaction that writes the chosen ids in ascending order,
// equal values going to the smaller id.
#include "mcs_common.h"
#include "mcs_internal.h"
#include "mcs_radix.h"

namespace mcs {

constexpr int MKT = 64;  // keys per tile

struct MassParams {
  const uint16_t* q;
  const uint16_t* k;
  const float* lse;
  const int32_t* perm;
  float* mass;
  int32_t N, C, G, bh0, nh;
  float sl2;
};

// 16-byte chunk swizzle of a K row in LDS (64 banks of 4 bytes): 16
// consecutive rows reading one logical chunk hit 16 distinct bank groups.
template <int D>
__device__ __forceinline__ int mswz(int row) {
  if (D == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
  return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void group_mass_kernel(MassParams p) {
  constexpr int NT = NW * 64;
  constexpr int CH = D / 8;
  constexpr int KSTEPS = D / 16;
  constexpr int ROWS_PER_PASS = NT / CH;              // key rows loaded per pass
  constexpr int LIT = (MKT + ROWS_PER_PASS - 1) / ROWS_PER_PASS;

  __shared__ u32x4_t lds_k[2][MKT * CH];
  __shared__ float red[2][NW][MKT];

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, lq = lane & 31, hh = lane >> 5;
  const int lb = xcd_remap(blockIdx.x, p.nh * p.G);
  const int hl = lb / p.G, g = lb - hl * p.G;
  const size_t head = (size_t)(p.bh0 + hl) * p.N;
  const uint16_t* __restrict__ qh = p.q + head * D;
  const uint16_t* __restrict__ kh = p.k + head * D;

  // A fragments: row lq of the wave's 32-query block
  const int qpos = g * p.C + w * 32 + lq;
  bf16x8_t qf[KSTEPS];
  {
    const bool ok = qpos < p.N;
    const int row = ok ? clamp_id(p.perm[head + qpos], p.N) : 0;
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t)
      qf[t] = as_bf16x8(ok ? ldg16(qh + (size_t)row * D + 16 * t + 8 * hh) : zero_u32x4());
  }
  // log2-domain LSE of the accumulator rows 8j + 4*hh + i held by this lane
  float lse2[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int pos = g * p.C + w * 32 + 8 * (e >> 2) + 4 * hh + (e & 3);
    lse2[e] = pos < p.N ? p.lse[head + clamp_id(p.perm[head + pos], p.N)] * kLog2e : INFINITY;
  }

  const int ntiles = (p.N + MKT - 1) / MKT;
  const int chunk = tid % CH;
  const int rsub = tid / CH;
  u32x4_t kreg[LIT];
  auto load_tile = [&](int tile) {
#pragma unroll
    for (int it = 0; it < LIT; ++it) {
      const int r = rsub + it * ROWS_PER_PASS;
      const int key = tile * MKT + r;
      kreg[it] = (r < MKT && key < p.N) ? ldg16(kh + (size_t)key * D + chunk * 8) : zero_u32x4();
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int it = 0; it < LIT; ++it) {
      const int r = rsub + it * ROWS_PER_PASS;
      if (r < MKT) lds_k[buf][r * CH + (chunk ^ mswz<D>(r))] = kreg[it];
    }
  };

  float* __restrict__ mrow = p.mass + ((size_t)hl * p.G + g) * p.N;
  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) load_tile(t + 1);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16_t acc = zero16();
      const int row = kb * 32 + lq;
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        const bf16x8_t b = as_bf16x8(lds_k[buf][row * CH + ((2 * ks + hh) ^ mswz<D>(row))]);
        acc = mfma32x32x16(qf[ks], b, acc);
      }
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) part += fast_exp2(fmaf(acc[e], p.sl2, -lse2[e]));
      part = halves_sum(part);
      if (hh == 0) red[buf][w][kb * 32 + lq] = part;
    }
    if (t + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
    if (tid < MKT) {
      const int key = t * MKT + tid;
      if (key < p.N) {
        float s = 0.f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) s += red[buf][ww][tid];
        mrow[key] = s;
      }
    }
  }
}

hipError_t run_group_mass(const uint16_t* q, const uint16_t* k, const float* lse,
                          const int32_t* perm, float* mass, int bh0, int nh, int N, int D,
                          int C, float scale, hipStream_t s) {
  MassParams p;
  p.q = q; p.k = k; p.lse = lse; p.perm = perm; p.mass = mass;
  p.N = N; p.C = C; p.G = (N + C - 1) / C; p.bh0 = bh0; p.nh = nh;
  p.sl2 = scale * kLog2e;
  const dim3 grid(nh * p.G);
  if (D == 128) {
    if (C == 128) hipLaunchKernelGGL((group_mass_kernel<128, 4>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((group_mass_kernel<128, 2>), grid, dim3(128), 0, s, p);
  } else {
    if (C == 128) hipLaunchKernelGGL((group_mass_kernel<64, 4>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((group_mass_kernel<64, 2>), grid, dim3(128), 0, s, p);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------

constexpr int TOPK_NT = 1024;

__global__ __launch_bounds__(TOPK_NT) void topk_kernel(const float* __restrict__ scores,
                                                      int32_t* __restrict__ idx, int n, int K) {
  __shared__ RadixLds<TOPK_NT> L;
  const size_t row = blockIdx.x;
  const uint32_t* __restrict__ x = reinterpret_cast<const uint32_t*>(scores) + row * (size_t)n;
  int32_t* __restrict__ out = idx + row * (size_t)K;
  // larger score -> smaller key; -0.0 (and any negative, which is not allowed) -> as 0
  auto key = [&](int i) -> uint32_t {
    const uint32_t u = x[i];
    return ~((u & 0x80000000u) ? 0u : u);
  };
  uint32_t T;
  int need;
  radix_select_smallest<TOPK_NT>(key, n, K, L, T, need);
  ordered_compact<TOPK_NT>(key, n, T, need, L, [&](int i, bool sel, int rank) {
    if (sel && rank < K) out[rank] = i;   // rank < K by construction; kept as a bound
  });
}

hipError_t run_topk(const float* scores, int32_t* idx, int64_t rows, int n, int K,
                    hipStream_t s) {
  const int64_t max_grid = 1 << 30;
  for (int64_t r0 = 0; r0 < rows; r0 += max_grid) {
    const int64_t nr = rows - r0 < max_grid ? rows - r0 : max_grid;
    hipLaunchKernelGGL(topk_kernel, dim3((unsigned)nr), dim3(TOPK_NT), 0, s,
                       scores + r0 * (int64_t)n, idx + r0 * (int64_t)K, n, K);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace mcs
