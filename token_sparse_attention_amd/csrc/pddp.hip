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

// Principal direction of one node per workgroup.  The node's second moments
// live in registers in the MFMA accumulator layout of node_moments: wave w,
// block b covers the 32x32 block (rb, cb) of sum(x x^T) with f = w*NBLK + b,
// rb = f / (D/32), cb = f % (D/32), and lane (lq, hh) holds element e of it at
// row rb*32 + 8*(e/4) + 4*hh + e%4, column cb*32 + lq.  The power iteration
// runs on that layout: since the covariance is symmetric, y = C v is
// y[c] = sum_r C[r][c] v[r], so every lane sums its 16 rows of one column,
// the two half-waves are added with one lane swap, and the row blocks meet in
// a small LDS array.  Two barriers per step; nothing D x D ever goes to LDS.
// FROM_PARTS: the node's moments are summed from pddp_moments partials (large
// nodes); otherwise the workgroup computes them itself.
template <int D, bool FROM_PARTS>
__global__ __launch_bounds__(PD_NT) void pddp_direction(PddpParams p) {
  constexpr int NBLK = (D / 32) * (D / 32) / 4;
  constexpr int RB = D / 32;
  constexpr int CH = D / 8;
  __shared__ MomentLds<D> L;
  __shared__ float sred[MSTEP / 4][D];
  __shared__ float part[2][RB][D];
  __shared__ float mu[D], vec[D];
  __shared__ int ish[2];
  const int slot = blockIdx.x, bh = blockIdx.y;
  int off, n, g;
  if (!node_geom(p.N, p.C, p.level, slot, off, n, g)) return;
  const size_t head = (size_t)bh * p.N;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, lq = lane & 31, hh = lane >> 5;

  f32x16_t acc[NBLK];
  if (FROM_PARTS) {
    // sum the node's chunk partials in chunk order, straight into the layout
    // (the chunk loop is outermost so every thread has 64 loads in flight)
    const int nch = (n + CHUNK_M - 1) / CHUNK_M;
    const float* __restrict__ base = p.part + ((size_t)bh * p.slots + (size_t)slot * p.cpn) * (D * D + D);
#pragma unroll
    for (int b = 0; b < NBLK; ++b) acc[b] = zero16();
    float msum = 0.f;
    for (int c = 0; c < nch; ++c) {
      const float* __restrict__ pc = base + (size_t)c * (D * D + D);
#pragma unroll
      for (int b = 0; b < NBLK; ++b) {
        const int f = w * NBLK + b, rb = f / RB, cb = f % RB;
#pragma unroll
        for (int e = 0; e < 16; ++e)
          acc[b][e] += pc[(size_t)(rb * 32 + 8 * (e >> 2) + 4 * hh + (e & 3)) * D + cb * 32 + lq];
      }
      if (tid < D) msum += pc[D * D + tid];
    }
    if (tid < D) mu[tid] = msum;
  } else {
    float sumx[8];
    node_moments<D>(p.q + head * D, p.perm + head + off, p.N, 0, n, L, acc, sumx);
    if (tid < (MSTEP / 4) * CH) {
#pragma unroll
      for (int e = 0; e < 8; ++e) sred[tid / CH][(tid % CH) * 8 + e] = sumx[e];
    }
    __syncthreads();
    if (tid < D) {
      float sacc = 0.f;
      for (int qd = 0; qd < MSTEP / 4; ++qd) sacc += sred[qd][tid];
      mu[tid] = sacc;
    }
  }
  __syncthreads();
  const float inv_n = 1.f / (float)n;
  if (tid < D) mu[tid] *= inv_n;
  __syncthreads();
  // covariance = sum(x x^T)/n - mu mu^T, in place
#pragma unroll
  for (int b = 0; b < NBLK; ++b) {
    const int f = w * NBLK + b, rb = f / RB, cb = f % RB;
    const float mc = mu[cb * 32 + lq];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int r = rb * 32 + 8 * (e >> 2) + 4 * hh + (e & 3);
      acc[b][e] = acc[b][e] * inv_n - mu[r] * mc;
    }
  }
  // start: the covariance column of largest diagonal (first on ties); the
  // diagonal goes through part[0]
#pragma unroll
  for (int b = 0; b < NBLK; ++b) {
    const int f = w * NBLK + b, rb = f / RB, cb = f % RB;
    if (rb == cb && hh == ((lq >> 2) & 1)) part[0][0][cb * 32 + lq] = acc[b][4 * (lq >> 3) + (lq & 3)];
  }
  __syncthreads();
  if (w == 0) {
    float bv = -INFINITY;
    int bi = 0;
#pragma unroll
    for (int k = 0; k < D / 64; ++k) {
      const float x = part[0][0][lane + 64 * k];
      if (x > bv) {
        bv = x;
        bi = lane + 64 * k;
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(bv, o);
      const int oi = __shfl_xor(bi, o);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (lane == 0) ish[0] = bi;
  }
  __syncthreads();
  {
    const int best = ish[0];
#pragma unroll
    for (int b = 0; b < NBLK; ++b) {
      const int f = w * NBLK + b, rb = f / RB, cb = f % RB;
      if (cb * 32 + lq == best) {
#pragma unroll
        for (int e = 0; e < 16; ++e) vec[rb * 32 + 8 * (e >> 2) + 4 * hh + (e & 3)] = acc[b][e];
      }
    }
  }
  __syncthreads();
  // normalise the start column (wave 0; a zero column gives e_0)
  if (w == 0) {
    float y[D / 64], s2 = 0.f;
#pragma unroll
    for (int k = 0; k < D / 64; ++k) {
      y[k] = vec[lane + 64 * k];
      s2 = fmaf(y[k], y[k], s2);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) s2 += __shfl_xor(s2, o);
#pragma unroll
    for (int k = 0; k < D / 64; ++k) {
      const int c = lane + 64 * k;
      vec[c] = s2 > 0.f ? y[k] * rsqrtf(s2) : (c == 0 ? 1.f : 0.f);
    }
  }
  __syncthreads();
  // Power iteration, one barrier per step: every wave forms y = C v from the
  // row-block partials (buffer it & 1), takes |y| itself, and writes the new v
  // only for the rows its own blocks read (vec rows are private to a wave from
  // here on; a zero y leaves v unchanged).
  const int iters = p.iters > 0 ? p.iters : DEFAULT_ITERS;
  const int myrb = (w * NBLK) / RB;       // row block of this wave's blocks
  for (int it = 0; it < iters; ++it) {
    const int pb = it & 1;
#pragma unroll
    for (int b = 0; b < NBLK; ++b) {
      const int f = w * NBLK + b, rb = f / RB, cb = f % RB;
      float y = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) y = fmaf(acc[b][e], vec[rb * 32 + 8 * (e >> 2) + 4 * hh + (e & 3)], y);
      y = halves_sum(y);
      if (hh == 0) part[pb][rb][cb * 32 + lq] = y;
    }
    __syncthreads();
    float y[D / 64], s2 = 0.f;
#pragma unroll
    for (int k = 0; k < D / 64; ++k) {
      float v = 0.f;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) v += part[pb][rb][lane + 64 * k];
      y[k] = v;
      s2 = fmaf(v, v, s2);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) s2 += __shfl_xor(s2, o);
    if (s2 > 0.f) {
      const float inv = rsqrtf(s2);
#pragma unroll
      for (int k = 0; k < D / 64; ++k) {
        const int c = lane + 64 * k;
        if ((c >> 5) == myrb) vec[c] = y[k] * inv;
      }
    }
  }
  // each row block of vec now holds v (written by the wave that owns it)
  __syncthreads();
  // sign: largest-magnitude component positive (first on ties); mu.v
  if (w == 0) {
    float bv = -1.f, mv = 0.f;
    int bi = 0;
    float sgnv = 0.f;
#pragma unroll
    for (int k = 0; k < D / 64; ++k) {
      const int c = lane + 64 * k;
      const float x = vec[c];
      if (fabsf(x) > bv) {
        bv = fabsf(x);
        bi = c;
        sgnv = x;
      }
      mv = fmaf(mu[c], x, mv);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(bv, o);
      const int oi = __shfl_xor(bi, o);
      const float os = __shfl_xor(sgnv, o);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
        sgnv = os;
      }
      mv += __shfl_xor(mv, o);
    }
    const float sgn = sgnv < 0.f ? -1.f : 1.f;
    float* __restrict__ out = p.dir + ((size_t)bh * p.nodes + slot) * (D + 4);
#pragma unroll
    for (int k = 0; k < D / 64; ++k) out[lane + 64 * k] = sgn * vec[lane + 64 * k];
    if (lane == 0) out[D] = sgn * mv;
  }
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
  // UR rows per thread and pass, their loads issued together
  constexpr int UR = 4;
  for (int base = m0; base < m1; base += RPP * UR) {
    int id[UR];
    u32x4_t x[UR];
#pragma unroll
    for (int u = 0; u < UR; ++u) {
      const int m = base + u * RPP + sub;
      id[u] = m < m1 ? ph[m] : 0;
    }
#pragma unroll
    for (int u = 0; u < UR; ++u) {
      const int m = base + u * RPP + sub;
      x[u] = m < m1 ? ldg16(qh + (size_t)clamp_id(id[u], p.N) * D + chunk * 8) : zero_u32x4();
    }
#pragma unroll
    for (int u = 0; u < UR; ++u) {
      const int m = base + u * RPP + sub;
      float part = 0.f;
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        part = fmaf(bf16_lo(x[u][wd]), vc[2 * wd], part);
        part = fmaf(bf16_hi(x[u][wd]), vc[2 * wd + 1], part);
      }
#pragma unroll
      for (int o = CH / 2; o >= 1; o >>= 1) part += __shfl_xor(part, o);
      if (m < m1 && chunk == 0) {
        p.proj[head + off + m] = part - muv;
        p.tmp[head + off + m] = id[u];
      }
    }
  }
}

template <int NT>
__global__ __launch_bounds__(NT) void pddp_split(PddpParams p) {
  __shared__ RadixLds<NT> L;
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
  radix_select_smallest<NT>(key, n, r, L, T, need);
  ordered_compact<NT>(key, n, T, need, L, [&](int i, bool sel, int rank) {
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
    if (p.cpn > 1) hipLaunchKernelGGL((pddp_direction<D, true>), dim3(nodes, BH), dim3(PD_NT), 0, s, p);
    else hipLaunchKernelGGL((pddp_direction<D, false>), dim3(nodes, BH), dim3(PD_NT), 0, s, p);
    hipLaunchKernelGGL(pddp_project<D>, dim3(p.cpn, nodes, BH), dim3(PD_NT), 0, s, p);
    // large nodes take a 1024-thread selection, small ones 256
    if (maxn > 8192) hipLaunchKernelGGL(pddp_split<1024>, dim3(nodes, BH), dim3(1024), 0, s, p);
    else hipLaunchKernelGGL(pddp_split<PD_NT>, dim3(nodes, BH), dim3(PD_NT), 0, s, p);
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
