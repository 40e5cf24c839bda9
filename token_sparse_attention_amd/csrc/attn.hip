// Dense and token-sparse attention for gfx950.
//
// One workgroup owns one tile of C query rows: a query group (sparse: the rows
// perm[g*C ..] of its head, with the group's K selected KV rows gathered by
// id) or C consecutive rows (dense: all N keys in order).  This is the
// token-sparse attention of the wispaper.ai explainer ("Token-level selection
// needs tile-aligned query groups": every group of C queries shares one
// selection of individually gathered KV tokens, so the group fills one query
// tile) with the dense kernel as the same engine on contiguous rows.
//
// Tile engine (per workgroup, C/32 waves, each wave owns 32 queries):
//   * Q of the wave's 32 queries stays in registers as MFMA B fragments.
//   * KV tiles of 64 keys stream through LDS, double buffered: K row-major
//     (16-byte chunks XOR-swizzled by row) and V transposed to [D][64]
//     (keys permuted inside each 16-key block so that the 8 keys one lane
//     needs for a PV step are contiguous).  Gathered rows are 16-byte loads,
//     16 lanes per 256-byte row, issued one tile ahead of use.
//   * S^T = K Q^T on MFMA: each lane then holds 32 keys of one query, so the
//     online softmax is per lane, plus one exchange with lane L^32 for the
//     running maximum.  Softmax in base 2 with scale*log2(e) folded in.
//   * O^T += V^T P^T on MFMA, P^T taken straight from the S^T accumulators.
//   * Epilogue: O = O^T / l (+ residual), bf16, scattered to the query rows;
//     lse = (m + log2 l) * ln 2 for the dense pass.
#include "mcs_common.h"
#include "mcs_internal.h"

namespace mcs {

constexpr int KT = 64;  // keys per KV tile

struct AttnParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* perm;    // sparse only
  const int32_t* kv_idx;  // sparse only
  const uint16_t* res;    // optional residual
  void* o;                // bf16 or fp32 output
  float* lse;             // optional (dense)
  int32_t N, C, K, G, BH;
  float sl2;              // scale * log2(e)
};

// LDS chunk swizzles (16-byte chunks).
template <int D>
__device__ __forceinline__ int swz_k(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
__device__ __forceinline__ int swz_vt(int d) { return (d >> 1) & 7; }
// Position of key k (0..63) in a transposed V row: bits 2 and 3 swapped.
__device__ __forceinline__ int vt_pos(int k) {
  return (k & ~15) | (k & 3) | ((k & 4) << 1) | ((k & 8) >> 1);
}

template <int D, int NW, bool SPARSE, bool RES, bool LSE, bool OUTF32>
__global__ __launch_bounds__(NW * 64) void attn_kernel(AttnParams p) {
  constexpr int NT = NW * 64;
  constexpr int CH = D / 8;               // 16-byte chunks per row
  constexpr int KSTEPS = D / 16;          // MFMA k-steps of QK^T
  constexpr int DB = D / 32;              // 32-row blocks of O^T
  constexpr int PAIRS = (KT / 4) * CH;    // (4-key quad, chunk) load units per tile
  constexpr int LIT = (PAIRS + NT - 1) / NT;

  __shared__ u32x4_t lds_k[2][KT * CH];
  __shared__ u32x4_t lds_vt[2][D * (KT / 8)];

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, lq = lane & 31, hh = lane >> 5;

  const int total = p.BH * p.G;
  const int lb = xcd_remap(blockIdx.x, total);
  const int bh = lb / p.G, g = lb - bh * p.G;
  const size_t head = (size_t)bh * p.N;
  const uint16_t* __restrict__ qh = p.q + head * D;
  const uint16_t* __restrict__ kh = p.k + head * D;
  const uint16_t* __restrict__ vh = p.v + head * D;

  // ---- this lane's query (column lq of the wave's 32-query block) ----
  const int qpos = g * p.C + w * 32 + lq;
  const bool qvalid = qpos < p.N;
  int qrow = qvalid ? qpos : 0;
  if (SPARSE && qvalid) qrow = clamp_id(p.perm[head + qpos], p.N);
  bf16x8_t qf[KSTEPS];
#pragma unroll
  for (int t = 0; t < KSTEPS; ++t)
    qf[t] = as_bf16x8(qvalid ? ldg16(qh + (size_t)qrow * D + 16 * t + 8 * hh) : zero_u32x4());

  const int nkeys = SPARSE ? p.K : p.N;
  const int ntiles = (nkeys + KT - 1) / KT;
  const int32_t* __restrict__ ids = SPARSE ? p.kv_idx + ((size_t)bh * p.G + g) * p.K : nullptr;

  // ---- KV tile loader: thread -> (quad of 4 consecutive keys, 16-byte chunk) ----
  u32x4_t kreg[LIT][4], vreg[LIT][4];
  auto load_tile = [&](int tile) {
#pragma unroll
    for (int it = 0; it < LIT; ++it) {
      const int pp = tid + it * NT;
      if (PAIRS % NT != 0 && pp >= PAIRS) continue;
      const int quad = pp / CH, chunk = pp - (pp / CH) * CH;
      const int key0 = tile * KT + quad * 4;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kp = key0 + r;
        if (kp < nkeys) {
          const int row = SPARSE ? clamp_id(ids[kp], p.N) : kp;
          kreg[it][r] = ldg16(kh + (size_t)row * D + chunk * 8);
          vreg[it][r] = ldg16(vh + (size_t)row * D + chunk * 8);
        } else {
          kreg[it][r] = zero_u32x4();
          vreg[it][r] = zero_u32x4();
        }
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int it = 0; it < LIT; ++it) {
      const int pp = tid + it * NT;
      if (PAIRS % NT != 0 && pp >= PAIRS) continue;
      const int quad = pp / CH, chunk = pp - (pp / CH) * CH;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = quad * 4 + r;
        lds_k[buf][row * CH + (chunk ^ swz_k<D>(row))] = kreg[it][r];
      }
      const int kpos = vt_pos(quad * 4);
      u32x2_t* vt2 = reinterpret_cast<u32x2_t*>(&lds_vt[buf][0]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = chunk * 8 + e;
        const int word = e >> 1;
        uint32_t a0 = vreg[it][0][word], a1 = vreg[it][1][word];
        uint32_t a2 = vreg[it][2][word], a3 = vreg[it][3][word];
        u32x2_t pr;
        if (e & 1) {
          pr[0] = (a0 >> 16) | (a1 & 0xffff0000u);
          pr[1] = (a2 >> 16) | (a3 & 0xffff0000u);
        } else {
          pr[0] = (a0 & 0xffffu) | (a1 << 16);
          pr[1] = (a2 & 0xffffu) | (a3 << 16);
        }
        const int c = kpos >> 3;
        vt2[(d * (KT / 8) + (c ^ swz_vt(d))) * 2 + ((kpos >> 2) & 1)] = pr;
      }
    }
  };

  float m_run = -INFINITY, l_run = 0.f;
  f32x16_t oacc[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) oacc[b] = zero16();

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) load_tile(t + 1);

    // S^T = K Q^T for the two 32-key blocks of the tile
    f32x16_t sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sacc[kb] = zero16();
      const int row = kb * 32 + lq;
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        const bf16x8_t a = as_bf16x8(lds_k[buf][row * CH + ((2 * ks + hh) ^ swz_k<D>(row))]);
        sacc[kb] = mfma32x32x16(a, qf[ks], sacc[kb]);
      }
    }
    if ((t + 1) * KT > nkeys) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = t * KT + kb * 32 + 8 * (e >> 2) + 4 * hh + (e & 3);
          if (key >= nkeys) sacc[kb][e] = -INFINITY;
        }
    }

    // online softmax (base 2), one query per lane
    float mx = sacc[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[kb][e]);
    mx = halves_max(mx);
    const float m_new = fmaxf(m_run, mx * p.sl2);
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;

    bf16x8_t pf[KT / 16];
    float lsum = 0.f;
#pragma unroll
    for (int s = 0; s < KT / 16; ++s) {
      const int kb = s >> 1, e0 = 8 * (s & 1);
      u32x4_t pw;
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        const float x0 = fast_exp2(fmaf(sacc[kb][e0 + 2 * wd], p.sl2, -m_new));
        const float x1 = fast_exp2(fmaf(sacc[kb][e0 + 2 * wd + 1], p.sl2, -m_new));
        lsum += x0 + x1;
        pw[wd] = pack_bf16x2(x0, x1);
      }
      pf[s] = as_bf16x8(pw);
    }
    l_run = l_run * alpha + lsum;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[b][e] *= alpha;

    // O^T += V^T P^T
#pragma unroll
    for (int b = 0; b < DB; ++b) {
      const int d = b * 32 + lq;
#pragma unroll
      for (int s = 0; s < KT / 16; ++s) {
        const bf16x8_t a = as_bf16x8(lds_vt[buf][d * (KT / 8) + ((2 * s + hh) ^ swz_vt(d))]);
        oacc[b] = mfma32x32x16(a, pf[s], oacc[b]);
      }
    }

    if (t + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue ----
  const float l_tot = halves_sum(l_run);
  if (!qvalid) return;
  const float inv = 1.f / l_tot;
  uint16_t* orow = static_cast<uint16_t*>(p.o) + (head + qrow) * D;
  float* orow32 = static_cast<float*>(p.o) + (head + qrow) * D;
  const uint16_t* rrow = RES ? p.res + (head + qrow) * D : nullptr;
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d0 = b * 32 + 8 * j + 4 * hh;
      float y0 = oacc[b][4 * j + 0] * inv, y1 = oacc[b][4 * j + 1] * inv;
      float y2 = oacc[b][4 * j + 2] * inv, y3 = oacc[b][4 * j + 3] * inv;
      if (RES) {
        const u32x2_t r = *reinterpret_cast<const u32x2_t*>(rrow + d0);
        y0 += bf16_lo(r[0]);
        y1 += bf16_hi(r[0]);
        y2 += bf16_lo(r[1]);
        y3 += bf16_hi(r[1]);
      }
      if (OUTF32) {
        float4 out = {y0, y1, y2, y3};
        *reinterpret_cast<float4*>(orow32 + d0) = out;
      } else {
        u32x2_t out;
        out[0] = pack_bf16x2(y0, y1);
        out[1] = pack_bf16x2(y2, y3);
        *reinterpret_cast<u32x2_t*>(orow + d0) = out;
      }
    }
  if (LSE && hh == 0) p.lse[head + qrow] = (m_run + fast_log2(l_tot)) * kLn2;
}

template <int D, int NW, bool SPARSE, bool RES, bool LSE, bool OUTF32>
static hipError_t launch_attn(const AttnParams& p, hipStream_t s) {
  const int total = p.BH * p.G;
  hipLaunchKernelGGL((attn_kernel<D, NW, SPARSE, RES, LSE, OUTF32>), dim3(total), dim3(NW * 64), 0,
                     s, p);
  return hipGetLastError();
}

template <int D, int NW, bool OUTF32>
static hipError_t dispatch_attn(const AttnParams& p, bool sparse, bool res, bool lse, hipStream_t s) {
  if (sparse) {
    return res ? launch_attn<D, NW, true, true, false, OUTF32>(p, s)
               : launch_attn<D, NW, true, false, false, OUTF32>(p, s);
  }
  return lse ? launch_attn<D, NW, false, false, true, OUTF32>(p, s)
             : launch_attn<D, NW, false, false, false, OUTF32>(p, s);
}

template <bool OUTF32>
static hipError_t dispatch_shape(const AttnParams& p, int D, int C, bool sparse, bool res, bool lse,
                                 hipStream_t s) {
  if (D == 128) {
    return C == 128 ? dispatch_attn<128, 4, OUTF32>(p, sparse, res, lse, s)
                    : dispatch_attn<128, 2, OUTF32>(p, sparse, res, lse, s);
  }
  return C == 128 ? dispatch_attn<64, 4, OUTF32>(p, sparse, res, lse, s)
                  : dispatch_attn<64, 2, OUTF32>(p, sparse, res, lse, s);
}

hipError_t run_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         const int32_t* perm, const int32_t* kv_idx, const uint16_t* res,
                         void* o, bool out_f32, float* lse, int B, int H, int N, int D, int C, int K,
                         float scale, hipStream_t s) {
  AttnParams p;
  p.q = q; p.k = k; p.v = v; p.perm = perm; p.kv_idx = kv_idx; p.res = res;
  p.o = o; p.lse = lse;
  p.N = N; p.C = C; p.K = K; p.G = (N + C - 1) / C; p.BH = B * H;
  p.sl2 = scale * kLog2e;
  const bool sparse = kv_idx != nullptr;
  return out_f32 ? dispatch_shape<true>(p, D, C, sparse, res != nullptr, lse != nullptr, s)
                 : dispatch_shape<false>(p, D, C, sparse, res != nullptr, lse != nullptr, s);
}

}  // namespace mcs
