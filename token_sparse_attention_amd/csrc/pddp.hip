// Median-split Fast PDDP grouping for gfx950.
//
// The ai.info page ("Key Contributions", "Methodology in Plain English") and the
// wispaper.ai explainer ("Token-level selection needs tile-aligned query
// groups") describe the grouping: project each node's queries on the node's
// principal direction and split the ordered queries at the median, recursively,
// until every group holds exactly C queries; the GPU version runs batched power
// iteration over all heads at one tree depth at a time and passes only index
// arrays between depths.
//
// Tree shape.  A node of n queries forms g = ceil(n/C) groups; a node with
// g > 1 sends the first C*floor(g/2) queries (in projection order) left and the
// rest right.  The shape depends only on (N, C), so every kernel finds its node
// from (level, slot) by walking the split sizes down from the root
// (node_geom), and every node owns the contiguous range [off, off+n) of its
// head's perm row.  perm starts as the identity and every split is a stable
// partition, so inside every node the queries stay in ascending id order and a
// tie in projection is broken by query id simply by position.
//
// Per level, for all nodes of all heads at once:
//   pddp_moments   (large nodes only) chunks of 2048 queries -> partial
//                  sum(x) and sum(x x^T) on bf16 MFMA with fp32 accumulation;
//   pddp_direction one workgroup per node: moments (summed partials, or
//                  computed directly for small nodes) -> covariance -> power
//                  iteration -> unit direction v with its largest-magnitude
//                  component positive, and mu.v;
//   pddp_project   p_i = x_i.v - mu.v for every query of the node (fp32);
//   pddp_split     radix select of the rank-(C*floor(g/2)) projection and a
//                  stable partition of the node's perm range.
#include "mcs_common.h"
#include "mcs_internal.h"
#include "mcs_radix.h"

namespace mcs {

constexpr int PD_NT = 256;       // threads of the moment / direction / projection kernels
constexpr int CHUNK_M = 2048;    // queries per partial-moment chunk
constexpr int MSTEP = 64;        // queries staged in LDS per MFMA step
constexpr int DEFAULT_ITERS = 32;

__device__ __forceinline__ int swz_st(int d) { return (d >> 1) & 7; }

// Moments of queries [m0, m1) of the node at perm[off..]: each wave holds its
// share of sum(x x^T) as MFMA accumulators (NBLK 32x32 blocks), each thread a
// partial sum(x) of 8 dimensions of one 16-byte chunk.
template <int D>
struct MomentLds {
  u32x4_t st[2][D * (MSTEP / 8)];  // x^T: [D][64 queries], two buffers
};

template <int D>
__device__ void node_moments(const uint16_t* __restrict__ qh, const int32_t* __restrict__ ph,
                             int N, int m0, int m1, MomentLds<D>& L, f32x16_t* acc,
                             float* sumx) {
  constexpr int CH = D / 8;
  constexpr int NBLK = (D / 32) * (D / 32) / 4;
  constexpr int PAIRS = (MSTEP / 4) * CH;    // (quad of 4 queries, chunk)
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, lq = lane & 31, hh = lane >> 5;
  const bool loader = tid < PAIRS;
  const int quad = tid / CH, chunk = tid % CH;

#pragma unroll
  for (int b = 0; b < NBLK; ++b) acc[b] = zero16();
#pragma unroll
  for (int e = 0; e < 8; ++e) sumx[e] = 0.f;

  u32x4_t xr[4];
  auto load = [&](int base) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = base + quad * 4 + r;
      xr[r] = (loader && m < m1) ? ldg16(qh + (size_t)clamp_id(ph[m], N) * D + chunk * 8)
                                 : zero_u32x4();
    }
  };
  auto store = [&](int buf) {
    if (!loader) return;
    u32x2_t* st2 = reinterpret_cast<u32x2_t*>(&L.st[buf][0]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = chunk * 8 + e, word = e >> 1;
      u32x2_t pr;
      if (e & 1) {
        pr[0] = (xr[0][word] >> 16) | (xr[1][word] & 0xffff0000u);
        pr[1] = (xr[2][word] >> 16) | (xr[3][word] & 0xffff0000u);
      } else {
        pr[0] = (xr[0][word] & 0xffffu) | (xr[1][word] << 16);
        pr[1] = (xr[2][word] & 0xffffu) | (xr[3][word] << 16);
      }
      const int pos = quad * 4;  // query position inside the 64-query step
      st2[(d * (MSTEP / 8) + ((pos >> 3) ^ swz_st(d))) * 2 + ((pos >> 2) & 1)] = pr;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        sumx[2 * wd] += bf16_lo(xr[r][wd]);
        sumx[2 * wd + 1] += bf16_hi(xr[r][wd]);
      }
  };

  const int nsteps = (m1 - m0 + MSTEP - 1) / MSTEP;
  load(m0);
  store(0);
  __syncthreads();
  for (int st = 0; st < nsteps; ++st) {
    const int buf = st & 1;
    if (st + 1 < nsteps) load(m0 + (st + 1) * MSTEP);
#pragma unroll
    for (int b = 0; b < NBLK; ++b) {
      const int f = w * NBLK + b;
      const int rb = f / (D / 32), cb = f % (D / 32);
      const int d1 = rb * 32 + lq, d2 = cb * 32 + lq;
#pragma unroll
      for (int s = 0; s < MSTEP / 16; ++s) {
        const int c = 2 * s + hh;
        const bf16x8_t a = as_bf16x8(L.st[buf][d1 * (MSTEP / 8) + (c ^ swz_st(d1))]);
        const bf16x8_t bb = as_bf16x8(L.st[buf][d2 * (MSTEP / 8) + (c ^ swz_st(d2))]);
        acc[b] = mfma32x32x16(a, bb, acc[b]);
      }
    }
    if (st + 1 < nsteps) store(buf ^ 1);
    __syncthreads();
  }
}

struct PddpParams {
  const uint16_t* q;
  int32_t* perm;
  float* proj;
  int32_t* tmp;
  float* dir;    // [BH][nodes][D + 4]: v, then mu.v
  float* part;   // [BH][slots][D*D + D]
  int32_t N, C, level, cpn, iters, slots, nodes;
};

template <int D>
__global__ __launch_bounds__(PD_NT) void pddp_moments(PddpParams p) {
  constexpr int NBLK = (D / 32) * (D / 32) / 4;
  __shared__ MomentLds<D> L;
  __shared__ float sred[PD_NT / (D / 8)][D];
  const int c = blockIdx.x, slot = blockIdx.y, bh = blockIdx.z;
  int off, n, g;
  if (!node_geom(p.N, p.C, p.level, slot, off, n, g)) return;
  const int m0 = c * CHUNK_M;
  if (m0 >= n) return;
  const int m1 = min(n, m0 + CHUNK_M);
  const size_t head = (size_t)bh * p.N;
  f32x16_t acc[NBLK];
  float sumx[8];
  node_moments<D>(p.q + head * D, p.perm + head + off, p.N, m0, m1, L, acc, sumx);

  float* __restrict__ out = p.part + ((size_t)bh * p.slots + (size_t)slot * p.cpn + c) * (D * D + D);
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, lq = lane & 31, hh = lane >> 5;
#pragma unroll
  for (int b = 0; b < NBLK; ++b) {
    const int f = w * NBLK + b;
    const int rb = f / (D / 32), cb = f % (D / 32);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int r = rb * 32 + 8 * (e >> 2) + 4 * hh + (e & 3);
      out[(size_t)r * D + cb * 32 + lq] = acc[b][e];
    }
  }
  constexpr int CH = D / 8;
  constexpr int QUADS = PD_NT / CH;
  if (tid < (MSTEP / 4) * CH) {
#pragma unroll
    for (int e = 0; e < 8; ++e) sred[tid / CH][(tid % CH) * 8 + e] = sumx[e];
  }
  __syncthreads();
  if (tid < D) {
    float s = 0.f;
    for (int qd = 0; qd < (MSTEP / 4) && qd < QUADS; ++qd) s += sred[qd][tid];
    out[D * D + tid] = s;
  }
}

__device__ __forceinline__ float block_sum_256(float x, float* sh) {
  // sum over a 256-thread workgroup, fixed order
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  __syncthreads();
  if (lane == 0) sh[w] = x;
  __syncthreads();
  return sh[0] + sh[1] + sh[2] + sh[3];
}

template <int D>
__global__ __launch_bounds__(PD_NT) void pddp_direction(PddpParams p) {
  constexpr int NBLK = (D / 32) * (D / 32) / 4;
  constexpr int CH = D / 8;
  __shared__ float cov[D][D + 1];
  __shared__ float mu[D], vec[D], nv[D];
  __shared__ float sh[8];
  __shared__ int ish[2];
  __shared__ MomentLds<D> L;
  __shared__ float sred[MSTEP / 4][D];

  const int slot = blockIdx.x, bh = blockIdx.y;
  int off, n, g;
  if (!node_geom(p.N, p.C, p.level, slot, off, n, g)) return;
  const size_t head = (size_t)bh * p.N;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, lq = lane & 31, hh = lane >> 5;

  if (p.cpn > 1) {
    // sum the node's chunk partials in chunk order
    const int nch = (n + CHUNK_M - 1) / CHUNK_M;
    const float* __restrict__ base = p.part + ((size_t)bh * p.slots + (size_t)slot * p.cpn) * (D * D + D);
    for (int i = tid; i < D * D + D; i += PD_NT) {
      float s = 0.f;
      for (int c = 0; c < nch; ++c) s += base[(size_t)c * (D * D + D) + i];
      if (i < D * D) cov[i / D][i % D] = s;
      else mu[i - D * D] = s;
    }
  } else {
    f32x16_t acc[NBLK];
    float sumx[8];
    node_moments<D>(p.q + head * D, p.perm + head + off, p.N, 0, n, L, acc, sumx);
#pragma unroll
    for (int b = 0; b < NBLK; ++b) {
      const int f = w * NBLK + b;
      const int rb = f / (D / 32), cb = f % (D / 32);
#pragma unroll
      for (int e = 0; e < 16; ++e) cov[rb * 32 + 8 * (e >> 2) + 4 * hh + (e & 3)][cb * 32 + lq] = acc[b][e];
    }
    if (tid < (MSTEP / 4) * CH) {
#pragma unroll
      for (int e = 0; e < 8; ++e) sred[tid / CH][(tid % CH) * 8 + e] = sumx[e];
    }
    __syncthreads();
    if (tid < D) {
      float s = 0.f;
      for (int qd = 0; qd < MSTEP / 4; ++qd) s += sred[qd][tid];
      mu[tid] = s;
    }
  }
  __syncthreads();
  const float inv_n = 1.f / (float)n;
  if (tid < D) mu[tid] *= inv_n;
  __syncthreads();
  for (int i = tid; i < D * D; i += PD_NT) {
    const int a = i / D, b = i % D;
    cov[a][b] = cov[a][b] * inv_n - mu[a] * mu[b];
  }
  __syncthreads();

  // start: the covariance column of largest diagonal (first on ties)
  if (tid == 0) {
    int best = 0;
    float bv = cov[0][0];
    for (int d = 1; d < D; ++d)
      if (cov[d][d] > bv) {
        bv = cov[d][d];
        best = d;
      }
    ish[0] = best;
  }
  __syncthreads();
  float x = tid < D ? cov[tid][ish[0]] : 0.f;
  float nrm2 = block_sum_256(x * x, sh);
  if (tid < D) vec[tid] = nrm2 > 0.f ? x * rsqrtf(nrm2) : (tid == 0 ? 1.f : 0.f);
  __syncthreads();
  const int iters = p.iters > 0 ? p.iters : DEFAULT_ITERS;
  for (int it = 0; it < iters; ++it) {
    float y = 0.f;
    if (tid < D) {
#pragma unroll 8
      for (int e = 0; e < D; ++e) y = fmaf(cov[tid][e], vec[e], y);
    }
    const float s2 = block_sum_256(y * y, sh);
    if (s2 > 0.f && tid < D) nv[tid] = y * rsqrtf(s2);
    else if (tid < D) nv[tid] = vec[tid];
    __syncthreads();
    if (tid < D) vec[tid] = nv[tid];
    __syncthreads();
  }
  // sign: largest-magnitude component positive (first on ties)
  if (tid == 0) {
    int best = 0;
    float bv = fabsf(vec[0]);
    for (int d = 1; d < D; ++d)
      if (fabsf(vec[d]) > bv) {
        bv = fabsf(vec[d]);
        best = d;
      }
    ish[1] = vec[best] < 0.f ? 1 : 0;
  }
  __syncthreads();
  const float sgn = ish[1] ? -1.f : 1.f;
  const float vv = tid < D ? sgn * vec[tid] : 0.f;
  const float muv = block_sum_256(tid < D ? mu[tid] * vv : 0.f, sh);
  float* __restrict__ out = p.dir + ((size_t)bh * p.nodes + slot) * (D + 4);
  if (tid < D) out[tid] = vv;
  if (tid == 0) out[D] = muv;
}

template <int D>
__global__ __launch_bounds__(PD_NT) void pddp_project(PddpParams p) {
  constexpr int CH = D / 8;
  constexpr int RPP = PD_NT / CH;   // queries per pass
  const int c = blockIdx.x, slot = blockIdx.y, bh = blockIdx.z;
  int off, n, g;
  if (!node_geom(p.N, p.C, p.level, slot, off, n, g)) return;
  const int span = p.cpn > 1 ? CHUNK_M : n;
  const int m0 = c * span;
  if (m0 >= n) return;
  const int m1 = min(n, m0 + span);
  const size_t head = (size_t)bh * p.N;
  const float* __restrict__ dv = p.dir + ((size_t)bh * p.nodes + slot) * (D + 4);
  const int tid = threadIdx.x, chunk = tid % CH, sub = tid / CH;
  float vc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) vc[e] = dv[chunk * 8 + e];
  const float muv = dv[D];
  const uint16_t* __restrict__ qh = p.q + head * D;
  const int32_t* __restrict__ ph = p.perm + head + off;
  for (int base = m0; base < m1; base += RPP) {
    const int m = base + sub;
    const bool ok = m < m1;
    int id = 0;
    float part = 0.f;
    if (ok) {
      id = ph[m];
      const u32x4_t x = ldg16(qh + (size_t)clamp_id(id, p.N) * D + chunk * 8);
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        part = fmaf(bf16_lo(x[wd]), vc[2 * wd], part);
        part = fmaf(bf16_hi(x[wd]), vc[2 * wd + 1], part);
      }
    }
#pragma unroll
    for (int o = CH / 2; o >= 1; o >>= 1) part += __shfl_xor(part, o);
    if (ok && chunk == 0) {
      p.proj[head + off + m] = part - muv;
      p.tmp[head + off + m] = id;
    }
  }
}

__global__ __launch_bounds__(PD_NT) void pddp_split(PddpParams p) {
  __shared__ RadixLds<PD_NT> L;
  const int slot = blockIdx.x, bh = blockIdx.y;
  int off, n, g;
  if (!node_geom(p.N, p.C, p.level, slot, off, n, g)) return;
  const int r = p.C * (g / 2);
  const size_t head = (size_t)bh * p.N;
  const float* __restrict__ pr = p.proj + head + off;
  const int32_t* __restrict__ ids = p.tmp + head + off;
  int32_t* __restrict__ out = p.perm + head + off;
  auto key = [&](int i) -> uint32_t { return float_order_key(pr[i]); };
  uint32_t T;
  int need;
  radix_select_smallest<PD_NT>(key, n, r, L, T, need);
  ordered_compact<PD_NT>(key, n, T, need, L, [&](int i, bool sel, int rank) {
    const int pos = sel ? rank : r + rank;   // < n by construction; kept as a bound
    if (pos < n) out[pos] = ids[i];
  });
}

__global__ void pddp_init(int32_t* perm, int N, int64_t total) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < total) perm[i] = (int32_t)(i % N);
}

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

GroupPlan plan_group(int BH, int N, int D, int C) {
  GroupPlan pl;
  const int G = (N + C - 1) / C;
  int L = 0;
  while ((1 << L) < G) ++L;
  pl.levels = L;
  pl.max_slots = 0;
  pl.max_nodes = L > 0 ? (1 << (L - 1)) : 1;
  for (int lv = 0; lv < L; ++lv) {
    int maxn = 0;
    for (int s = 0; s < (1 << lv); ++s) {
      int off, n, g;
      if (node_geom(N, C, lv, s, off, n, g) && n > maxn) maxn = n;
    }
    const int cpn = (maxn + CHUNK_M - 1) / CHUNK_M;
    if (cpn > 1 && (1 << lv) * cpn > pl.max_slots) pl.max_slots = (1 << lv) * cpn;
  }
  size_t o = 0;
  pl.proj_off = o;
  o = align256(o + (size_t)BH * N * 4);
  pl.tmp_off = o;
  o = align256(o + (size_t)BH * N * 4);
  pl.dir_off = o;
  o = align256(o + (size_t)BH * pl.max_nodes * (D + 4) * 4);
  pl.part_off = o;
  o = align256(o + (size_t)BH * pl.max_slots * ((size_t)D * D + D) * 4);
  pl.bytes = o;
  return pl;
}

template <int D>
static hipError_t group_levels(PddpParams p, int BH, const GroupPlan& pl, hipStream_t s) {
  for (int lv = 0; lv < pl.levels; ++lv) {
    int maxn = 0;
    for (int sl = 0; sl < (1 << lv); ++sl) {
      int off, n, g;
      if (node_geom(p.N, p.C, lv, sl, off, n, g) && n > maxn) maxn = n;
    }
    p.level = lv;
    p.cpn = (maxn + CHUNK_M - 1) / CHUNK_M;
    const int nodes = 1 << lv;
    if (p.cpn > 1) {
      hipLaunchKernelGGL(pddp_moments<D>, dim3(p.cpn, nodes, BH), dim3(PD_NT), 0, s, p);
    }
    hipLaunchKernelGGL(pddp_direction<D>, dim3(nodes, BH), dim3(PD_NT), 0, s, p);
    hipLaunchKernelGGL(pddp_project<D>, dim3(p.cpn, nodes, BH), dim3(PD_NT), 0, s, p);
    hipLaunchKernelGGL(pddp_split, dim3(nodes, BH), dim3(PD_NT), 0, s, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t run_group(const uint16_t* q, int32_t* perm, int BH, int N, int D, int C, int iters,
                     void* ws, const GroupPlan& pl, hipStream_t s) {
  char* base = static_cast<char*>(ws);
  PddpParams p;
  p.q = q;
  p.perm = perm;
  p.proj = reinterpret_cast<float*>(base + pl.proj_off);
  p.tmp = reinterpret_cast<int32_t*>(base + pl.tmp_off);
  p.dir = reinterpret_cast<float*>(base + pl.dir_off);
  p.part = reinterpret_cast<float*>(base + pl.part_off);
  p.N = N;
  p.C = C;
  p.iters = iters;
  p.slots = pl.max_slots;
  p.nodes = pl.max_nodes;
  const int64_t total = (int64_t)BH * N;
  hipLaunchKernelGGL(pddp_init, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, perm, N, total);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return D == 128 ? group_levels<128>(p, BH, pl, s) : group_levels<64>(p, BH, pl, s);
}

}  // namespace mcs
