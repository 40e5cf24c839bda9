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
#include <type_traits>

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

#ifndef MCS_MASS_VALU
#define MCS_MASS_VALU 3          // exponential-side VALU instructions after each MFMA of the next block
#endif

template <int D, int NW>
__global__ __launch_bounds__(NW * 64, 4) void group_mass_kernel(MassParams p) {
  constexpr int CH = D / 8;                 // 16-byte chunks per row
  constexpr int ROWB = D * 2;               // bytes per K row
  constexpr int KSTEPS = D / 16;
  constexpr int TILE_BYTES = MKT * ROWB;
  constexpr int INSTR = TILE_BYTES / 1024;  // 1 KiB DMA instructions per tile
  constexpr int IPW = INSTR / NW;
  constexpr int ROWS_PER_INSTR = 64 / CH;
  constexpr int RED_KEYS = MKT / NW;        // keys each wave reduces per tile
  static_assert(INSTR % NW == 0 && RED_KEYS <= 64, "tile split");

  __shared__ __attribute__((aligned(1024))) uint16_t lds_k[2][MKT * D];
  __shared__ float red[2][NW][MKT];
  char* const lbase = reinterpret_cast<char*>(&lds_k[0][0]);

  const int tid = threadIdx.x;
  const int lane = tid & 63, lq = lane & 31, hh = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lb = xcd_remap(blockIdx.x, p.nh * p.G);
  const int hl = lb / p.G, g = lb - hl * p.G;
  const size_t head = (size_t)(p.bh0 + hl) * p.N;
  const uint16_t* __restrict__ qh = p.q + head * D;
  const __amdgpu_buffer_rsrc_t rk = head_rsrc(p.k + head * D, (uint32_t)p.N * ROWB);

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
  // (+inf for rows past N, whose probabilities are then 0)
  float lse2[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int pos = g * p.C + w * 32 + 8 * (e >> 2) + 4 * hh + (e & 3);
    lse2[e] = pos < p.N ? p.lse[head + clamp_id(p.perm[head + pos], p.N)] * kLog2e : INFINITY;
  }

  // DMA plan: instruction j of this wave fills rows (w*IPW + j)*ROWS_PER_INSTR
  // + lane/CH of a tile, physical chunk lane%CH (the swizzle picks the
  // logical chunk); rows past N read as zeros and are never stored
  uint32_t coff[IPW];
#pragma unroll
  for (int j = 0; j < IPW; ++j) {
    const int r = (w * IPW + j) * ROWS_PER_INSTR + lane / CH;
    coff[j] = (uint32_t)(r * ROWB + (((lane % CH) ^ swz<D>(r)) << 4));
  }
  auto issue = [&](int tile, int buf) {
#pragma unroll
    for (int j = 0; j < IPW; ++j)
      dma16(rk, (uint32_t)tile * (uint32_t)TILE_BYTES + coff[j],
            lbase + buf * TILE_BYTES + (w * IPW + j) * 1024);
  };
  // B fragment of k-step ks for key column lq of a 32-key block
  uint32_t koff[KSTEPS];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks)
    koff[ks] = (uint32_t)(lq * ROWB + (((2 * ks + hh) ^ swz<D>(lq)) << 4));

  // mass of one 32-key block: sum over this lane's 16 query rows, then the
  // partner lane's 16; four partial sums keep the add chains short
  auto block_mass = [&](const f32x16_t& acc) {
    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
    for (int e = 0; e < 16; e += 4) {
      s0 += fast_exp2(fmaf(acc[e], p.sl2, -lse2[e]));
      s1 += fast_exp2(fmaf(acc[e + 1], p.sl2, -lse2[e + 1]));
      s2 += fast_exp2(fmaf(acc[e + 2], p.sl2, -lse2[e + 2]));
      s3 += fast_exp2(fmaf(acc[e + 3], p.sl2, -lse2[e + 3]));
    }
    return halves_sum((s0 + s1) + (s2 + s3));
  };

  float* __restrict__ mrow = p.mass + ((size_t)hl * p.G + g) * p.N;
  // the waves' partial masses of tile t, summed in wave order
  auto store_tile = [&](int t) {
    const int b = t & 1;
    const int kk = w * RED_KEYS + lane;
    const int key = t * MKT + kk;
    if (lane < RED_KEYS && key < p.N) {
      float s = red[b][0][kk];
#pragma unroll
      for (int ww = 1; ww < NW; ++ww) s += red[b][ww][kk];
      mrow[key] = s;
    }
  };

  // Step t: wait for K_t, barrier (K_{t-1} and the partial masses of tile
  // t-1 are then free / complete), gather K_{t+1} into the other buffer,
  // store tile t-1's mass, then S = Q K_t^T with the exponentials of the
  // first 32-key block interleaved with the MFMAs of the second.  The loop is
  // unrolled by the two buffers so all LDS offsets are immediates.
  const int ntiles = (p.N + MKT - 1) / MKT;
  auto step = [&](auto buf_c, int t) {
    constexpr int BUF = decltype(buf_c)::value;
    wait_vmem_all();
    __syncthreads();
    if (t + 1 < ntiles) issue(t + 1, BUF ^ 1);
    if (t > 0) store_tile(t - 1);
    const char* kt = lbase + BUF * TILE_BYTES;
    f32x16_t acc0 = zero16(), acc1 = zero16();
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
      acc0 = mfma32x32x16(qf[ks], as_bf16x8(*reinterpret_cast<const u32x4_t*>(kt + koff[ks])), acc0);
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
      acc1 = mfma32x32x16(qf[ks], as_bf16x8(*reinterpret_cast<const u32x4_t*>(kt + 32 * ROWB + koff[ks])), acc1);
    const float m0 = block_mass(acc0);
    const float m1 = block_mass(acc1);
    if (hh == 0) {
      red[BUF][w][lq] = m0;
      red[BUF][w][32 + lq] = m1;
    }
    // K fragment reads two MFMAs ahead; block 0's exponentials ride on
    // block 1's MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int i = 0; i < KSTEPS; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
#pragma unroll
    for (int i = 0; i < KSTEPS; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i + 2 < KSTEPS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, MCS_MASS_VALU, 0);
    }
  };
  issue(0, 0);
  int t = 0;
  for (; t + 1 < ntiles; t += 2) {
    step(std::integral_constant<int, 0>{}, t);
    step(std::integral_constant<int, 1>{}, t + 1);
  }
  if (t < ntiles) step(std::integral_constant<int, 0>{}, t);
  __syncthreads();
  store_tile(ntiles - 1);
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
