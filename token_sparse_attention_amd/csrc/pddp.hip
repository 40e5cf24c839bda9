// Median-split Fast PDDP grouping for gfx950.
//
// The ai.info page ("Key Contributions", "Methodology in Plain English") and the
// wispaper.ai explainer ("Token-level selection needs tile-aligned query
// groups") describe the grouping: project each node's queries on the node's
// principal direction and split the ordered queries at the median, recursively,
// until every group holds exactly C queries; the GPU version finds the
// directions of all nodes of all heads at one tree depth at once (the pages'
// batched power iteration, here in its Krylov form: Lanczos on the same
// matrix-vector products, which converges where plain power steps stall on a
// small eigenvalue gap) and passes only index arrays between depths.
//
// Tree shape.  A node of n queries forms g = ceil(n/C) groups; a node with
// g > 1 sends the first C*floor(g/2) queries (in projection order) left and the
// rest right.  The shape depends only on (N, C), so the kernels of a level are
// launched over the level's split nodes only, and each workgroup finds its
// node from its rank by walking the split sizes down from the root
// (node_by_rank); every node owns the contiguous range [off, off+n) of its
// head's perm row.  perm starts as the identity and every split is a stable
// partition, so inside every node the queries stay in ascending id order and a
// tie in projection is broken by query id simply by position.
//
// Per level, for all nodes of all heads at once:
//   pddp_moments   (large nodes only) equal chunks of <= 2048 queries -> partial
//                  sum(x) and sum(x x^T) on bf16 MFMA with fp32 accumulation;
//   pddp_direction one workgroup per node: moments (summed partials, or
//                  computed directly for small nodes) -> covariance ->
//                  Lanczos (up to 32 steps, ending after 16 when the Ritz
//                  residual has converged) -> top eigenvector v of the
//                  covariance with its largest-magnitude component
//                  positive, and mu.v;
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
constexpr int DEFAULT_STEPS = 32;  // Lanczos steps (Krylov dimension) by default
constexpr int KRYLOV_MAX = 64;     // most Lanczos steps; the basis fills the moment staging LDS
// One convergence test of the Lanczos direction, after STOP_AT steps: the
// iteration ends there when the Ritz residual is below STOP_TOL times the
// Ritz value.  The test's eigenvalue bracket takes TEST_ROUNDS multisection
// rounds (about 1e-5 relative, plenty for the residual estimate); the final
// solve takes five.
constexpr int STOP_AT = 16;
constexpr double STOP_TOL = 1e-6;
constexpr int TEST_ROUNDS = 3;

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
                             int N, int m0, int m1, MomentLds<D>& L, int32_t* __restrict__ ids,
                             f32x16_t* acc, float* sumx) {
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

  // The ids of [m0, m1) (at most CHUNK_M) go to LDS first, so that every row
  // load below is a single global load (not an id load followed by a row
  // load); the rows of step st + 1 are loaded while step st is computed.
  for (int i = tid; i < m1 - m0; i += PD_NT) ids[i] = clamp_id(ph[m0 + i], N);
  __syncthreads();
  u32x4_t xr[4];
  auto load = [&](int base) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = base + quad * 4 + r;
      xr[r] = (loader && m < m1) ? ldg16(qh + (size_t)ids[m - m0] * D + chunk * 8) : zero_u32x4();
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
  // the per-thread sums of x, and before them the chunk's ids
  __shared__ float sred[PD_NT / (D / 8)][D];
  static_assert(PD_NT / (D / 8) * D >= CHUNK_M, "ids of a chunk fit");
  const int c = blockIdx.x, slot = blockIdx.y, bh = blockIdx.z;
  int off, n, g;
  if (!node_by_rank(p.N, p.C, p.level, slot, off, n, g)) return;
  // the node's ceil(n / CHUNK_M) chunks, of equal size up to one query
  const int nch = (n + CHUNK_M - 1) / CHUNK_M;
  const int span = (n + nch - 1) / nch;
  const int m0 = c * span;
  if (c >= nch || m0 >= n) return;
  const int m1 = min(n, m0 + span);
  const size_t head = (size_t)bh * p.N;
  f32x16_t acc[NBLK];
  float sumx[8];
  node_moments<D>(p.q + head * D, p.perm + head + off, p.N, m0, m1, L, reinterpret_cast<int32_t*>(&sred[0][0]),
                  acc, sumx);

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
// row rb*32 + 8*(e/4) + 4*hh + e%4, column cb*32 + lq.  The Lanczos products
// run on that layout: since the covariance is symmetric, y = C v is
// y[c] = sum_r C[r][c] v[r], so every lane sums its 16 rows of one column,
// the two half-waves are added with one lane swap, and the row blocks meet in
// a small LDS array.  One barrier per step; nothing D x D ever goes to LDS.
// The direction is the top eigenvector of the covariance (the node's
// principal direction), found by Lanczos with full reorthogonalisation: the
// top eigenpair of the small tridiagonal matrix (multisection on Sturm
// counts, then inverse iteration, in fp64) gives the Ritz vector.
// FROM_PARTS: the node's moments are summed from pddp_moments partials (large
// nodes); otherwise the workgroup computes them itself.
template <int D, bool FROM_PARTS>
__global__ __launch_bounds__(PD_NT) void pddp_direction(PddpParams p) {
  constexpr int NBLK = (D / 32) * (D / 32) / 4;
  constexpr int RB = D / 32;
  constexpr int CH = D / 8;
  __shared__ MomentLds<D> L;
  // the per-thread sums of x, and before them the ids of the node's queries
  // (nodes here hold at most CHUNK_M queries)
  __shared__ float sred[(MSTEP / 4) * D >= CHUNK_M ? MSTEP / 4 : CHUNK_M / D][D];
  __shared__ float part[2][RB][D];
  __shared__ float mu[D];
  // per wave: alpha, beta of the Lanczos recurrence (every wave holds the same
  // recurrence and runs the same convergence test, so all take the same stop
  // decision without a barrier); the final solve's pivots and vector (wave 0)
  constexpr int NWAVE = PD_NT / 64;
  __shared__ float tri[NWAVE][2][KRYLOV_MAX];
  __shared__ double tri_d[KRYLOV_MAX], tri_x[KRYLOV_MAX];
  __shared__ int ish[2];
  constexpr int NV = D / 64;                     // vector components per lane
  static_assert(sizeof(MomentLds<D>) >= sizeof(float) * KRYLOV_MAX * D, "basis must fit the staging LDS");
  const int slot = blockIdx.x, bh = blockIdx.y;
  int off, n, g;
  if (!node_by_rank(p.N, p.C, p.level, slot, off, n, g)) return;
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
    node_moments<D>(p.q + head * D, p.perm + head + off, p.N, 0, n, L, reinterpret_cast<int32_t*>(&sred[0][0]),
                    acc, sumx);
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
  // Lanczos basis vectors [KRYLOV_MAX][D] fp32, in the LDS of the moment
  // staging buffers (idle from here on)
  float* __restrict__ Vb = reinterpret_cast<float*>(&L);
  {
    const int best = ish[0];
#pragma unroll
    for (int b = 0; b < NBLK; ++b) {
      const int f = w * NBLK + b, rb = f / RB, cb = f % RB;
      if (cb * 32 + lq == best) {
#pragma unroll
        for (int e = 0; e < 16; ++e) Vb[rb * 32 + 8 * (e >> 2) + 4 * hh + (e & 3)] = acc[b][e];
      }
    }
  }
  __syncthreads();
  // normalise the start column (wave 0; a zero column gives e_0)
  if (w == 0) {
    float y[NV], s2 = 0.f;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      y[k] = Vb[lane + 64 * k];
      s2 = fmaf(y[k], y[k], s2);
    }
    s2 = wave_sum(s2);
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int c = lane + 64 * k;
      Vb[c] = s2 > 0.f ? y[k] * rsqrtf(s2) : (c == 0 ? 1.f : 0.f);
    }
  }
  __syncthreads();

  // Lanczos with full reorthogonalisation.  Every wave runs the three-term
  // recurrence on full-length vectors (lane holds components lane + 64*k),
  // with bitwise the same arithmetic in the same order, so all waves hold the
  // same alpha, beta and basis and leave the loop at the same step.  Only the
  // product C v needs the workgroup: each wave multiplies its row block (the
  // rows of v it reads are the ones it wrote itself), and the row-block
  // partials meet in LDS, one barrier per step.  The new vector is made
  // orthogonal to the whole basis by classical Gram-Schmidt, a second time
  // when the first pass removed more than half of its squared norm.
  const int steps = p.iters > 0 ? min(p.iters, KRYLOV_MAX) : DEFAULT_STEPS;
  const int myrb = (w * NBLK) / RB;       // row block of this wave's blocks
  float vj[NV], vprev[NV];
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    vj[k] = Vb[lane + 64 * k];
    vprev[k] = 0.f;
  }
  // One classical Gram-Schmidt pass against V[0..j]: h_i = V_i.w for all i
  // from the same w, then w -= sum h_i V_i.  The squared norm of w before the
  // pass is reduced in the same batch; the norm after it follows from
  // Pythagoras (V orthonormal), |w'|^2 = |w|^2 - sum h_i^2, returned in *after.
  auto reorth = [&](int j, float (&wv)[NV], float& before, float& after) {
    float dw[NV];
    float s2 = 0.f;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      dw[k] = 0.f;
      s2 = fmaf(wv[k], wv[k], s2);
    }
    before = 0.f;
    float hsq = 0.f;
    int i = 0;
    bool first = true;
    for (; i + 8 <= j + 1; i += 8) {
      float vv[8][NV], h[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        h[u] = 0.f;
#pragma unroll
        for (int k = 0; k < NV; ++k) {
          vv[u][k] = Vb[(i + u) * D + lane + 64 * k];
          h[u] = fmaf(vv[u][k], wv[k], h[u]);
        }
      }
      if (first) before = uniform_f(wave_sum(s2));
      first = false;
      wave_sum8(h);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        hsq = fmaf(h[u], h[u], hsq);
#pragma unroll
        for (int k = 0; k < NV; ++k) dw[k] = fmaf(h[u], vv[u][k], dw[k]);
      }
    }
    if (i <= j) {
      float vv[8][NV], h[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        h[u] = 0.f;
        if (i + u <= j) {
#pragma unroll
          for (int k = 0; k < NV; ++k) {
            vv[u][k] = Vb[(i + u) * D + lane + 64 * k];
            h[u] = fmaf(vv[u][k], wv[k], h[u]);
          }
        } else {
#pragma unroll
          for (int k = 0; k < NV; ++k) vv[u][k] = 0.f;
        }
      }
      if (first) before = uniform_f(wave_sum(s2));
      wave_sum8(h);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        hsq = fmaf(h[u], h[u], hsq);
#pragma unroll
        for (int k = 0; k < NV; ++k) dw[k] = fmaf(h[u], vv[u][k], dw[k]);
      }
    }
#pragma unroll
    for (int k = 0; k < NV; ++k) wv[k] -= dw[k];
    after = before - hsq;
  };
  // The small tridiagonal eigenproblem T = tridiag(beta, alpha, beta): the
  // recurrences are sequential in i and run on wave-uniform values, with
  // reciprocals from v_rcp_f64 refined by one Newton step (relative error
  // ~1e-14).
  float* const ta = tri[w][0];
  float* const tb = tri[w][1];
  double* const td = tri_d;
  double* const tx = tri_x;
  auto rcp64 = [](double d) {
    const double r = __builtin_amdgcn_rcp(d);
    return fma(r, fma(-d, r, 1.0), r);
  };
  // alpha_i and beta_i of this wave's arrays, one per lane, broadcast with readlane
  float al = 0.f, bl = 0.f;
  auto load_tri = [&](int mm) {
    al = lane < mm ? ta[lane] : 0.f;
    bl = lane < mm ? tb[lane] : 0.f;
  };
  auto a_at = [&](int i) { return (double)__int_as_float(__builtin_amdgcn_readlane(__float_as_int(al), i)); };
  auto b_at = [&](int i) { return (double)__int_as_float(__builtin_amdgcn_readlane(__float_as_int(bl), i)); };
  // Gershgorin interval, then multisection on Sturm counts: lane l counts the
  // eigenvalues below lo + (hi - lo) (l + 1) / 65, and the interval shrinks to
  // the two shifts around the largest eigenvalue, 5 times.  hi bounds it from
  // above.
  auto bracket = [&](int mm, int rounds, double& lo, double& hi) {
    load_tri(mm);
    lo = INFINITY;
    hi = -INFINITY;
    for (int i = 0; i < mm; ++i) {
      const double r = (i > 0 ? fabs(b_at(i - 1)) : 0.0) + (i + 1 < mm ? fabs(b_at(i)) : 0.0);
      lo = fmin(lo, a_at(i) - r);
      hi = fmax(hi, a_at(i) + r);
    }
    if (mm > 1 && hi > lo) {
      for (int round = 0; round < rounds; ++round) {
        const double x = lo + (hi - lo) * (double)(lane + 1) / 65.0;
        int cnt = 0;
        double d = 1.0;
        for (int i = 0; i < mm; ++i) {
          const double bb = i > 0 ? b_at(i - 1) : 0.0;
          d = (a_at(i) - x) - (i > 0 ? bb * bb * rcp64(d) : 0.0);
          if (d == 0.0) d = -1e-300;
          cnt += d < 0.0;
        }
        const uint64_t above = __builtin_amdgcn_ballot_w64(cnt >= mm);
        if (above == 0) {
          lo = lo + (hi - lo) * 64.0 / 65.0;
        } else {
          const int f = __builtin_ctzll(above);
          const double nhi = lo + (hi - lo) * (double)(f + 1) / 65.0;
          const double nlo = f > 0 ? lo + (hi - lo) * (double)f / 65.0 : lo;
          lo = nlo;
          hi = nhi;
        }
      }
    }
  };
  // |s_last| of the unit eigenvector of T for the eigenvalue th: rows mm-1
  // down to 1 of (T - th) s = 0 solved from the end with s_{mm-1} = 1.  For a
  // converged top pair the components grow towards the start, the stable
  // direction of this recurrence, and |s_last| = 1 / |s|.
  auto last_component = [&](int mm, double th) {
    double sp = 0.0, sc = 1.0, n2 = 1.0, last = 1.0;
    for (int i = mm - 1; i >= 1; --i) {
      const double bi = i + 1 < mm ? b_at(i) : 0.0;
      const double sn = -((a_at(i) - th) * sc + bi * sp) * rcp64(b_at(i - 1));
      sp = sc;
      sc = sn;
      n2 = fma(sn, sn, n2);
      if (n2 > 1e200) {                 // rescale the whole vector
        sp *= 1e-100;
        sc *= 1e-100;
        last *= 1e-100;
        n2 *= 1e-200;
      }
    }
    return last / sqrt(n2);
  };
  // The top eigenpair (theta, s) of the mm x mm tridiagonal in this wave's
  // arrays, for the final direction (wave 0): s goes to tx, theta (from above,
  // to the multisection's resolution) is returned.
  auto top_pair = [&](int mm) -> double {
    double lo, hi;
    bracket(mm, 5, lo, hi);
    if (mm == 1) {
      if (lane == 0) tx[0] = 1.0;
      return a_at(0);
    }
    // Inverse iteration with the shift sigma just above the largest
    // eigenvalue: sigma I - T is positive definite there, so its LU
    // factorisation needs no pivoting.  td holds the reciprocal pivots 1/d_i;
    // two sweeps from the all-ones vector.
    const double sigma = hi + fmax(hi - lo, 1e-9 * fabs(hi)) + 1e-300;
    {
      double rprev = 0.0;
      for (int i = 0; i < mm; ++i) {
        const double bb = i > 0 ? b_at(i - 1) : 0.0;
        const double dn = (sigma - a_at(i)) - (i > 0 ? bb * bb * rprev : 0.0);
        rprev = rcp64(dn);
        if (lane == 0) {
          td[i] = rprev;
          tx[i] = 1.0;
        }
      }
    }
    for (int iter = 0; iter < 2; ++iter) {
      double yprev = 0.0;
      for (int i = 0; i < mm; ++i) {       // forward: L y = x
        const double yi = tx[i] + (i > 0 ? b_at(i - 1) * td[i - 1] * yprev : 0.0);
        yprev = yi;
        if (lane == 0) tx[i] = yi;
      }
      double xnext = 0.0, s2 = 0.0;
      for (int i = mm - 1; i >= 0; --i) {  // back substitution: U x = y
        const double bb = i + 1 < mm ? b_at(i) : 0.0;
        const double xi = (tx[i] + bb * xnext) * td[i];
        xnext = xi;
        s2 += xi * xi;
        if (lane == 0) tx[i] = xi;
      }
      const double inv = 1.0 / sqrt(s2);
      for (int i = 0; i < mm; ++i)
        if (lane == 0) tx[i] *= inv;
    }
    return hi;
  };
  int m = 0;
  float bprev = 0.f;
  for (int j = 0; j < steps; ++j) {
    const int pb = j & 1;
    const float* __restrict__ vrow = Vb + j * D;
    {
      // the row block is the same for all of this wave's blocks, so the 16
      // entries of v are loaded once; two chains per block, all interleaved
      const int rb0 = (w * NBLK) / RB;
      float vr[16], ya[NBLK], yb[NBLK];
#pragma unroll
      for (int e = 0; e < 16; ++e) vr[e] = vrow[rb0 * 32 + 8 * (e >> 2) + 4 * hh + (e & 3)];
#pragma unroll
      for (int b = 0; b < NBLK; ++b) ya[b] = yb[b] = 0.f;
#pragma unroll
      for (int e = 0; e < 16; e += 2)
#pragma unroll
        for (int b = 0; b < NBLK; ++b) {
          ya[b] = fmaf(acc[b][e], vr[e], ya[b]);
          yb[b] = fmaf(acc[b][e + 1], vr[e + 1], yb[b]);
        }
#pragma unroll
      for (int b = 0; b < NBLK; ++b) {
        const int f = w * NBLK + b, rb = f / RB, cb = f % RB;
        const float y = halves_sum(ya[b] + yb[b]);
        if (hh == 0) part[pb][rb][cb * 32 + lq] = y;
      }
    }
    __syncthreads();
    float wv[NV], a = 0.f;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      float v = 0.f;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) v += part[pb][rb][lane + 64 * k];
      wv[k] = v;
      a = fmaf(vj[k], v, a);
    }
    a = uniform_f(wave_sum(a));
    if (lane == 0) ta[j] = a;
    m = j + 1;
    if (j + 1 >= steps) break;
#pragma unroll
    for (int k = 0; k < NV; ++k) wv[k] = fmaf(-bprev, vprev[k], fmaf(-a, vj[k], wv[k]));
    float n0, n1;
    reorth(j, wv, n0, n1);
    bool invariant = !(n0 > 0.f);
    if (!invariant && n1 <= 0.5f * n0) {
      // the pass removed more than half of the vector: the Pythagorean norm
      // is unreliable, and the vector is cleaned a second time
      float m1, m2;
      reorth(j, wv, m1, m2);
      // a vector a second pass still shrinks by half lies in the basis up to
      // rounding: the Krylov space is invariant and T already exact
      invariant = !(m1 > 0.f) || m2 <= 0.5f * m1;
      n1 = m2;
    }
    // the last pass removed less than half of the squared norm, so its
    // Pythagorean norm is accurate to a few ulps
    if (invariant) break;
    const float bnew = sqrtf(n1), inv = 1.f / bnew;
    if (lane == 0) tb[j] = bnew;
    // stop if the top Ritz pair of T (j + 1 steps) has converged: its
    // residual |C y - theta y| is beta_j |s_last|
    if (j + 1 == STOP_AT && j + 1 < steps) {
      double lo, hi;
      bracket(j + 1, TEST_ROUNDS, lo, hi);
      if ((double)bnew * last_component(j + 1, hi) <= STOP_TOL * fabs(hi)) break;
    }
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      vprev[k] = vj[k];
      vj[k] = wv[k] * inv;
      const int c = lane + 64 * k;
      if ((c >> 5) == myrb) Vb[(j + 1) * D + c] = vj[k];
    }
    bprev = bnew;
  }
  // From here on only wave 0 works (no further barriers): the top eigenpair
  // of the m x m tridiagonal, then the Ritz vector.  All of the basis is
  // visible: its last vector was written before the last step's barrier.
  if (w != 0) return;
  top_pair(m);
  // Ritz vector y = sum_j s_j V_j, normalised
  float y[NV], s2 = 0.f;
#pragma unroll
  for (int k = 0; k < NV; ++k) y[k] = 0.f;
  for (int j = 0; j < m; ++j) {
    const float sj = (float)tx[j];
#pragma unroll
    for (int k = 0; k < NV; ++k) y[k] = fmaf(sj, Vb[j * D + lane + 64 * k], y[k]);
  }
#pragma unroll
  for (int k = 0; k < NV; ++k) s2 = fmaf(y[k], y[k], s2);
  s2 = wave_sum(s2);
  const float yinv = s2 > 0.f ? rsqrtf(s2) : 0.f;
  // sign: largest-magnitude component positive (first on ties); mu.v
  {
    float bv = -1.f, mv = 0.f;
    int bi = 0;
    float sgnv = 0.f;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int c = lane + 64 * k;
      const float x = y[k] * yinv;
      y[k] = x;
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
    for (int k = 0; k < NV; ++k) out[lane + 64 * k] = sgn * y[k];
    if (lane == 0) out[D] = sgn * mv;
  }
}

template <int D>
__global__ __launch_bounds__(PD_NT) void pddp_project(PddpParams p) {
  constexpr int CH = D / 8;
  constexpr int RPP = PD_NT / CH;   // queries per pass
  const int c = blockIdx.x, slot = blockIdx.y, bh = blockIdx.z;
  int off, n, g;
  if (!node_by_rank(p.N, p.C, p.level, slot, off, n, g)) return;
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
  // UR rows per thread and pass, their loads issued together.  Pipelined:
  // the rows of the next pass are in flight while this pass is computed, and
  // the ids of the pass after that are loaded beside them.
  constexpr int UR = 4, STEP = RPP * UR;
  int id[UR], idn[UR] = {};
  u32x4_t x[UR], xn[UR];
#pragma unroll
  for (int u = 0; u < UR; ++u) xn[u] = zero_u32x4();
  auto load_ids = [&](int base, int (&ids)[UR]) {
#pragma unroll
    for (int u = 0; u < UR; ++u) {
      const int m = base + u * RPP + sub;
      ids[u] = m < m1 ? ph[m] : 0;
    }
  };
  auto load_rows = [&](int base, const int (&ids)[UR], u32x4_t (&xs)[UR]) {
#pragma unroll
    for (int u = 0; u < UR; ++u) {
      const int m = base + u * RPP + sub;
      xs[u] = m < m1 ? ldg16(qh + (size_t)clamp_id(ids[u], p.N) * D + chunk * 8) : zero_u32x4();
    }
  };
  load_ids(m0, id);
  load_rows(m0, id, x);
  if (m0 + STEP < m1) load_ids(m0 + STEP, idn);
  for (int base = m0; base < m1; base += STEP) {
    if (base + STEP < m1) load_rows(base + STEP, idn, xn);
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
#pragma unroll
    for (int u = 0; u < UR; ++u) {
      id[u] = idn[u];
      x[u] = xn[u];
    }
    if (base + 2 * STEP < m1) load_ids(base + 2 * STEP, idn);
  }
}

template <int NT>
__global__ __launch_bounds__(NT) void pddp_split(PddpParams p) {
  __shared__ RadixLds<NT> L;
  const int slot = blockIdx.x, bh = blockIdx.y;
  int off, n, g;
  if (!node_by_rank(p.N, p.C, p.level, slot, off, n, g)) return;
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

// Largest node (queries) at a level.  Only the rightmost node can be short
// (it holds the remainder group), and it is a split node whenever the level
// has any; every other node holds C * (its groups) queries, q or q + 1 groups
// with q = G >> level, and q + 1 occurs off the rightmost node when at least
// two nodes have it (G mod 2^level >= 2).
static int level_max_n(int N, int C, int lv) {
  const int G = (N + C - 1) / C;
  const int cnt = split_nodes_below(G, lv);
  if (cnt == 0) return 0;
  int off, n, g;
  node_by_rank(N, C, lv, cnt - 1, off, n, g);
  const int q = G >> lv, r = G & ((1 << lv) - 1);
  if (cnt >= 2) n = max(n, C * (r >= 2 ? q + 1 : q));
  return n;
}

GroupPlan plan_group(int BH, int N, int D, int C) {
  GroupPlan pl;
  const int G = (N + C - 1) / C;
  int L = 0;
  while ((1 << L) < G) ++L;
  pl.levels = L;
  pl.max_slots = 0;
  pl.max_nodes = 1;
  for (int lv = 0; lv < L; ++lv) {
    const int nodes = split_nodes_at(N, C, lv);
    if (nodes > pl.max_nodes) pl.max_nodes = nodes;
    const int cpn = (level_max_n(N, C, lv) + CHUNK_M - 1) / CHUNK_M;
    if (cpn > 1 && nodes * cpn > pl.max_slots) pl.max_slots = nodes * cpn;
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
    const int maxn = level_max_n(p.N, p.C, lv);
    const int nodes = split_nodes_at(p.N, p.C, lv);
    if (nodes == 0) continue;
    p.level = lv;
    p.cpn = (maxn + CHUNK_M - 1) / CHUNK_M;
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
