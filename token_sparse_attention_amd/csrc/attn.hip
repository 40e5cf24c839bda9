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
// Tile engine (per workgroup, C/32 waves, each wave owns 32 queries; two
// workgroups per CU, so two waves share each SIMD and one's softmax overlaps
// the other's MFMA work):
//   * Q of the wave's 32 queries stays in registers as MFMA B fragments.
//   * KV tiles of 64 keys are gathered straight into LDS by LDS-DMA
//     (global_load_lds_dwordx4: each lane moves one 16-byte chunk of a K or V
//     row, so rows are fetched by id with no staging registers), double
//     buffered: tile t+1 is in flight while tile t is computed.  K and V are
//     row-major with 16-byte chunks XOR-swizzled by row; the lane -> chunk
//     assignment of the DMA realises the swizzle.
//   * S^T = K Q^T on MFMA (v_mfma_f32_32x32x16_bf16): each lane then holds 32
//     keys of one query, so the online softmax is per lane plus one exchange
//     with lane L^32 for the running maximum.  Base-2 softmax with
//     scale*log2(e) folded into one FMA per score.  The running maximum is
//     only moved (and O rescaled) when a new score exceeds it by more than
//     2^8, so most tiles skip the rescale; P stays <= 256, exact in bf16
//     range, and the final division by the row sum cancels the offset.
//   * O^T += V^T P^T on MFMA, P^T taken straight from the S^T accumulators and
//     V^T fragments read with the LDS transpose load ds_read_b64_tr_b16.
//   * Epilogue: O = O^T / l (+ residual), bf16 or fp32, scattered to the query
//     rows; lse = (m + log2 l) * ln 2 for the dense pass.
#include "mcs_common.h"
#include "mcs_internal.h"

namespace mcs {

constexpr int KT = 64;          // keys per KV tile
constexpr float kRescaleSlack = 8.f;   // log2 of the largest unscaled P

typedef __attribute__((address_space(3))) void* lds_void_t;
typedef __attribute__((address_space(1))) void* gbl_void_t;
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4_t* lds_bf16x4_ptr;

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

// 16-byte chunk swizzle of a K/V row in LDS.
template <int D>
__device__ __forceinline__ int swz(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}

// One 16-byte LDS-DMA per lane: the wave writes 1 KiB at lds (wave-uniform).
__device__ __forceinline__ void dma16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds((gbl_void_t)g, (lds_void_t)lds, 16, 0, 0);
}

__device__ __forceinline__ void wait_vmem_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <int D, int NW, bool SPARSE, bool RES, bool LSE, bool OUTF32>
__global__ __launch_bounds__(NW * 64, 2) void attn_kernel(AttnParams p) {
  constexpr int NT = NW * 64;
  constexpr int CH = D / 8;                 // 16-byte chunks per row
  constexpr int KSTEPS = D / 16;            // MFMA k-steps of QK^T
  constexpr int DB = D / 32;                // 32-row blocks of O^T
  constexpr int TILE_BYTES = KT * D * 2;    // one K (or V) tile
  constexpr int INSTR = TILE_BYTES / 1024;  // 1 KiB DMA instructions per K tile
  constexpr int IPW = INSTR / NW;           // ... per wave
  constexpr int ROWS_PER_INSTR = 64 / CH;
  static_assert(INSTR % NW == 0, "tile must split evenly over the waves");

  // [stage][K | V][KT * D] bf16
  __shared__ __attribute__((aligned(1024))) uint16_t lds[2][2][KT * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63, lq = lane & 31, hh = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

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

  // ---- DMA plan: instruction j of this wave covers tile rows
  //      (w*IPW + j)*ROWS_PER_INSTR + lane/CH, one 16-byte chunk per lane ----
  const int lrow = lane / CH;
  const int pchunk = lane % CH;
  int rowid[IPW];        // kv row of each DMA instruction for the next tile to load
  auto fetch_ids = [&](int tile) {
#pragma unroll
    for (int j = 0; j < IPW; ++j) {
      int kp = tile * KT + (w * IPW + j) * ROWS_PER_INSTR + lrow;
      kp = kp < nkeys ? kp : nkeys - 1;   // rows past the end: a valid row, masked later
      rowid[j] = SPARSE ? clamp_id(ids[kp], p.N) : kp;
    }
  };
  auto issue_dma = [&](int stage) {
#pragma unroll
    for (int j = 0; j < IPW; ++j) {
      const int r = (w * IPW + j) * ROWS_PER_INSTR + lrow;
      const int c = pchunk ^ swz<D>(r);   // logical chunk stored at physical chunk pchunk
      const size_t goff = (size_t)rowid[j] * D + c * 8;
      char* kdst = reinterpret_cast<char*>(&lds[stage][0][0]) + (w * IPW + j) * 1024;
      char* vdst = reinterpret_cast<char*>(&lds[stage][1][0]) + (w * IPW + j) * 1024;
      dma16(kh + goff, kdst);
      dma16(vh + goff, vdst);
    }
  };

  float m_run = -INFINITY, l_run = 0.f;
  f32x16_t oacc[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) oacc[b] = zero16();

  fetch_ids(0);
  issue_dma(0);
  if (ntiles > 1) fetch_ids(1);

  for (int t = 0; t < ntiles; ++t) {
    const int st = t & 1;
    wait_vmem_all();
    __syncthreads();
    if (t + 1 < ntiles) {
      issue_dma(st ^ 1);
      if (t + 2 < ntiles) fetch_ids(t + 2);
    }
    const uint16_t* kt = &lds[st][0][0];
    const uint16_t* vt = &lds[st][1][0];

    // S^T = K Q^T for the two 32-key blocks of the tile
    f32x16_t sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sacc[kb] = zero16();
      const int row = kb * 32 + lq;
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        const bf16x8_t a = as_bf16x8(
            *reinterpret_cast<const u32x4_t*>(kt + row * D + ((2 * ks + hh) ^ swz<D>(row)) * 8));
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
    mx = halves_max(mx) * p.sl2;
    // move the reference maximum only when a score exceeds it by > 2^slack
    if (__builtin_amdgcn_ballot_w64(mx > m_run + kRescaleSlack) != 0) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = fast_exp2(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[b][e] *= alpha;
    }
    const float mneg = -m_run;

    bf16x8_t pf[KT / 16];
#pragma unroll
    for (int s = 0; s < KT / 16; ++s) {
      const int kb = s >> 1, e0 = 8 * (s & 1);
      u32x4_t pw;
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        const float x0 = fast_exp2(fmaf(sacc[kb][e0 + 2 * wd], p.sl2, mneg));
        const float x1 = fast_exp2(fmaf(sacc[kb][e0 + 2 * wd + 1], p.sl2, mneg));
        l_run += x0 + x1;
        pw[wd] = pack_bf16x2(x0, x1);
      }
      pf[s] = as_bf16x8(pw);
    }

    // O^T += V^T P^T; V^T fragments by LDS transpose reads: lane group
    // (lane/16) reads 4 consecutive key rows, lane i%16 gets column i
#pragma unroll
    for (int b = 0; b < DB; ++b) {
      const int dcol = b * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
      const int rsub = (lane & 15) >> 2;
#pragma unroll
      for (int s = 0; s < KT / 16; ++s) {
        const int r0 = 16 * s + 4 * hh + rsub;       // slots e = 0..3
        const int r1 = r0 + 8;                       // slots e = 4..7
        const uint16_t* a0p = vt + r0 * D + (((dcol >> 3) ^ swz<D>(r0)) << 3) + (dcol & 7);
        const uint16_t* a1p = vt + r1 * D + (((dcol >> 3) ^ swz<D>(r1)) << 3) + (dcol & 7);
        const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_ptr)(a0p));
        const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_ptr)(a1p));
        const bf16x8_t a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        oacc[b] = mfma32x32x16(a, pf[s], oacc[b]);
      }
    }
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
