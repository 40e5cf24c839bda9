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
//   * KV tiles of 64 keys are gathered straight into LDS by buffer loads
//     with the LDS destination (buffer_load_dwordx4 ... lds: each lane moves
//     one 16-byte chunk of a K or V row, so rows are fetched by id with no
//     staging registers; a per-head buffer descriptor bounds the reads and
//     returns zeros past the end), double buffered: tile t+1 is in flight
//     while tile t is computed.  K and V are row-major with 16-byte chunks
//     XOR-swizzled by row; the lane -> chunk assignment of the DMA realises
//     the swizzle.  All LDS read addresses are per-lane constants plus
//     immediates (the tile loop is unrolled by the two buffers).
//   * S^T = K Q^T on MFMA (v_mfma_f32_32x32x16_bf16): each lane then holds 32
//     keys of one query, so the online softmax is per lane plus one exchange
//     with lane L^32 for the running maximum.  Base-2 softmax with
//     scale*log2(e) folded into one FMA per score.  The running maximum is
//     only moved (and O rescaled) when a new score exceeds it by more than
//     2^8, so most tiles skip the rescale; P stays small (<= 2^13), well in
//     bf16 range, and the final division by the row sum cancels the offset.
//     Kernels without an LSE output defer even the row max: they take the
//     exponentials against the current maximum and let the tile's P sum
//     show the rare tile that must move it (that tile is then redone).
//   * O^T += V^T P^T on MFMA, P^T taken straight from the S^T accumulators and
//     V^T fragments read with the LDS transpose load ds_read_b64_tr_b16.  O
//     is normalised by the sum of the same bf16-rounded P that enter the
//     product (v_dot2c_f32_bf16 against (1, 1)), so its error scales with
//     |v_j - o| instead of |v_j|; the LSE uses the exact fp32 sum.
//   * Epilogue: O = O^T / l (+ residual), bf16 or fp32, scattered to the query
//     rows; lse = (m + log2 l) * ln 2 (the dense pass, or on request the
//     sparse one over its selected keys).
#include <type_traits>

#include "mcs_common.h"
#include "mcs_internal.h"

namespace mcs {

constexpr int KT = 64;          // keys per KV tile
#ifndef MCS_SCHED_LOOKAHEAD
#define MCS_SCHED_LOOKAHEAD 4        // LDS fragment reads issued ahead of their MFMA
#endif
#ifndef MCS_S_ALTERNATE
#define MCS_S_ALTERNATE 0            // interleave the two S accumulation chains
#endif
#ifndef MCS_SCHED_VALU
#define MCS_SCHED_VALU 4             // VALU instructions interleaved after each S MFMA
#endif
constexpr float kRescaleSlack = 8.f;   // log2 of the largest unscaled P
constexpr float kDeferredLimit = 8192.f;  // a lane's 32 values of one tile, each <= 2^8

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4_t* lds_bf16x4_ptr;

struct AttnParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* perm;    // sparse only
  const int32_t* kv_idx;  // sparse only
  const int32_t* kv_count;  // sparse, optional: keys used per group (first ids)
  const uint16_t* res;    // optional residual
  void* o;                // bf16 or fp32 output
  float* lse;             // optional (dense)
  int32_t N, C, K, G, BH;
  float sl2;              // scale * log2(e)
};

template <int V>
using ic = std::integral_constant<int, V>;

template <int D, int NW, bool SPARSE, bool RES, bool LSE, bool OUTF32>
__global__ __launch_bounds__(NW * 64, 2) void attn_kernel(AttnParams p) {
  constexpr int CH = D / 8;                 // 16-byte chunks per row
  constexpr int ROWB = D * 2;               // bytes per K/V row
  constexpr int KSTEPS = D / 16;            // MFMA k-steps of QK^T
  constexpr int DB = D / 32;                // 32-row blocks of O^T
  constexpr int TILE_BYTES = KT * ROWB;     // one K (or V) tile
  constexpr int STAGE_BYTES = 2 * TILE_BYTES;
  constexpr int INSTR = TILE_BYTES / 1024;  // 1 KiB DMA instructions per K tile
  constexpr int IPW = INSTR / NW;           // ... per wave
  constexpr int ROWS_PER_INSTR = 64 / CH;
  static_assert(INSTR % NW == 0, "tile must split evenly over the waves");

  // [stage][K | V][KT * D] bf16
  __shared__ __attribute__((aligned(1024))) uint16_t lds[2][2][KT * D];
  char* const lbase = reinterpret_cast<char*>(&lds[0][0][0]);
  // sparse: ring of kv ids, two halves of IDS_CHUNK tiles, refilled by DMA
  // a whole chunk ahead so id latency never reaches the tile loop (D = 64:
  // a half-size ring keeps the workgroup at 40 KB, four per CU)
  constexpr int IDS_CHUNK = D == 64 ? 16 : 32;        // tiles per ring half
  constexpr int RING_IDS = SPARSE ? 2 * IDS_CHUNK * KT : 4;
  __shared__ __attribute__((aligned(1024))) int32_t ring[RING_IDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63, lq = lane & 31, hh = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

  const int total = p.BH * p.G;
  const int lb = xcd_remap(blockIdx.x, total);
  const int bh = lb / p.G, g = lb - bh * p.G;
  const size_t head = (size_t)bh * p.N;
  const uint16_t* __restrict__ qh = p.q + head * D;
  const uint32_t head_bytes = (uint32_t)p.N * ROWB;
  const __amdgpu_buffer_rsrc_t rk = head_rsrc(p.k + head * D, head_bytes);
  const __amdgpu_buffer_rsrc_t rv = head_rsrc(p.v + head * D, head_bytes);

  // ---- this lane's query (column lq of the wave's 32-query block) ----
  const int qpos = g * p.C + w * 32 + lq;
  const bool qvalid = qpos < p.N;
  int qrow = qvalid ? qpos : 0;
  if (SPARSE && qvalid) qrow = clamp_id(p.perm[head + qpos], p.N);
  bf16x8_t qf[KSTEPS];
#pragma unroll
  for (int t = 0; t < KSTEPS; ++t)
    qf[t] = as_bf16x8(qvalid ? ldg16(qh + (size_t)qrow * D + 16 * t + 8 * hh) : zero_u32x4());

  int nkeys = SPARSE ? p.K : p.N;
  if (SPARSE && p.kv_count != nullptr) {
    const int c = __builtin_amdgcn_readfirstlane(p.kv_count[(size_t)bh * p.G + g]);
    nkeys = c < 1 ? 1 : (c > p.K ? p.K : c);
  }
  const int ntiles = (nkeys + KT - 1) / KT;
  const int32_t* __restrict__ ids = SPARSE ? p.kv_idx + ((size_t)bh * p.G + g) * p.K : nullptr;

  // ---- DMA plan: instruction j of this wave fills tile rows
  //      (w*IPW + j)*ROWS_PER_INSTR + lane/CH, physical chunk lane%CH ----
  const int lrow = lane / CH;
  const int pchunk = lane % CH;
  uint32_t coff[IPW];    // byte offset of this lane's logical chunk in its row, per instruction
#pragma unroll
  for (int j = 0; j < IPW; ++j) {
    const int r = (w * IPW + j) * ROWS_PER_INSTR + lrow;
    coff[j] = (uint32_t)((pchunk ^ swz<D>(r)) * 16);
  }
  // Sparse: ids come from the LDS ring; ring positions past K hold zeros (the
  // id buffer descriptor ends at K), and those keys are masked after QK^T.
  auto fetch_ids = [&](int tile, uint32_t (&rowoff)[IPW]) {
#pragma unroll
    for (int j = 0; j < IPW; ++j) {
      const int r = (w * IPW + j) * ROWS_PER_INSTR + lrow;
      const uint32_t row = (uint32_t)ring[(tile % (2 * IDS_CHUNK)) * KT + r];
      // an id outside [0, N) (negative ones included, as unsigned) is clamped
      // to N, whose offset lies past the descriptor's end (N*D*2 < 2^31), so
      // it reads a zero row; the product of a larger id could wrap
      rowoff[j] = __builtin_elementwise_min(row, (uint32_t)p.N) * (uint32_t)ROWB + coff[j];
    }
  };
  // Dense: a tile's rows are consecutive, so each load's offset is a per-lane
  // constant (its row in the tile and chunk) plus the tile's base, a scalar;
  // rows past N fall past the descriptor's end and read zeros.
  uint32_t doff[IPW];
#pragma unroll
  for (int j = 0; j < IPW; ++j) doff[j] = (uint32_t)(((w * IPW + j) * ROWS_PER_INSTR + lrow) * ROWB) + coff[j];
  // refill ring half (chunk & 1) with the ids of tiles [chunk*IDS_CHUNK, +IDS_CHUNK)
  __amdgpu_buffer_rsrc_t rids;
  if (SPARSE) rids = head_rsrc(ids, (uint32_t)p.K * 4u);
  auto refill_ids = [&](int chunk) {
    constexpr int BYTES = IDS_CHUNK * KT * 4;           // bytes per half
    constexpr int PER_WAVE = BYTES / 1024 / NW;
    char* half = reinterpret_cast<char*>(&ring[0]) + (chunk & 1) * BYTES;
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
      const int blk = w * PER_WAVE + j;                 // 1 KiB block of the half
      dma16(rids, (uint32_t)(chunk * BYTES + blk * 1024 + lane * 16), half + blk * 1024);
    }
  };
  // K tiles live in lds[*][0], V tiles in lds[*][1]; K runs one tile ahead of
  // V.  `tile` is the key tile the rows belong to (dense), rowoff the gathered
  // rows' offsets (sparse).
  auto issue_rows = [&](__amdgpu_buffer_rsrc_t r, const uint32_t (&rowoff)[IPW], int tile, char* dst) {
    if constexpr (SPARSE) {
#pragma unroll
      for (int j = 0; j < IPW; ++j) dma16(r, rowoff[j], dst + (w * IPW + j) * 1024);
    } else {
      const uint32_t soff = __builtin_amdgcn_readfirstlane((uint32_t)tile * (uint32_t)TILE_BYTES);
#pragma unroll
      for (int j = 0; j < IPW; ++j) dma16s(r, doff[j], soff, dst + (w * IPW + j) * 1024);
    }
  };
  auto issue_k = [&](auto buf_c, const uint32_t (&rowoff)[IPW], int tile) {
    constexpr int BUF = decltype(buf_c)::value;
    issue_rows(rk, rowoff, tile, lbase + BUF * STAGE_BYTES);
  };
  auto issue_v = [&](auto buf_c, const uint32_t (&rowoff)[IPW], int tile) {
    constexpr int BUF = decltype(buf_c)::value;
    issue_rows(rv, rowoff, tile, lbase + BUF * STAGE_BYTES + TILE_BYTES);
  };

  // ---- per-lane LDS read offsets (buffer, key block and k-step are immediates) ----
  uint32_t koff[KSTEPS];   // K fragment of k-step ks, key row lq
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks)
    koff[ks] = (uint32_t)(lq * ROWB + (((2 * ks + hh) ^ swz<D>(lq)) << 4));
  const int rsub = (lane & 15) >> 2;
  // transpose reads of d-block b: key rows 16s + 4*hh + rsub (slots 0..3) and
  // 16s + 8 + 4*hh + rsub (slots 4..7); the swizzle of a row depends on it
  // only through row mod 16, so s enters as an immediate
  uint32_t voff_tr[2][DB];
#pragma unroll
  for (int half = 0; half < 2; ++half)
#pragma unroll
    for (int b = 0; b < DB; ++b) {
      const int dcol = b * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
      const int r = 8 * half + 4 * hh + rsub;
      voff_tr[half][b] = (uint32_t)(r * ROWB + (((dcol >> 3) ^ swz<D>(r)) << 4) + (dcol & 7) * 2);
    }

  // l_run: row sum of the bf16-rounded P that enter PV (normalises O
  // consistently: errors then scale with |v_j - o| rather than |v_j|);
  // l_lse: the exact fp32 row sum, for the LSE output.
  float m_run = -INFINITY, l_run = 0.f, l_lse = 0.f;
  f32x16_t oacc[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) oacc[b] = zero16();

  // S^T = K Q^T for the two 32-key blocks of the K tile in buffer BUF
  auto compute_s = [&](auto buf_c, f32x16_t (&sacc)[2]) {
    constexpr int BUF = decltype(buf_c)::value;
    const char* kt = lbase + BUF * STAGE_BYTES;
    sacc[0] = zero16();
    sacc[1] = zero16();
#if MCS_S_ALTERNATE
    // the two 32-key blocks' accumulation chains alternate
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8_t a = as_bf16x8(*reinterpret_cast<const u32x4_t*>(kt + kb * 32 * ROWB + koff[ks]));
        sacc[kb] = mfma32x32x16(a, qf[ks], sacc[kb]);
      }
#else
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        const bf16x8_t a = as_bf16x8(*reinterpret_cast<const u32x4_t*>(kt + kb * 32 * ROWB + koff[ks]));
        sacc[kb] = mfma32x32x16(a, qf[ks], sacc[kb]);
      }
#endif
  };

  // ---- online softmax of one tile's scores (base 2), one query per lane ----
  // The reference maximum m_run moves, and O and the row sums are rescaled,
  // only when a score exceeds it by more than 2^8 (wave-uniform, rare).
  auto tile_max = [&](const f32x16_t (&sacc)[2]) {
    float mx = sacc[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[kb][e]);
    return halves_max(mx) * p.sl2;
  };
  auto move_max = [&](float mx) {
    const float m_new = fmaxf(m_run, mx);
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
    if (LSE) l_lse *= alpha;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[b][e] *= alpha;
  };
  // eager form (kernels with an LSE output, and the last tile): the row max
  // first, then the exponentials
  auto softmax_max = [&](f32x16_t (&sacc)[2]) {
    const float mx = tile_max(sacc);
    if (__builtin_amdgcn_ballot_w64(mx > m_run + kRescaleSlack) != 0) move_max(mx);
  };
  // P = exp2(s*scale*log2e - m) as bf16 MFMA fragments; lsum accumulates the
  // sum of the bf16-rounded P, l_lse (LSE kernels) the exact one
  auto softmax_p = [&](f32x16_t (&sacc)[2], bf16x8_t (&pf)[KT / 16], float& lsum) {
    const float mneg = -m_run;
#pragma unroll
    for (int s = 0; s < KT / 16; ++s) {
      const int kb = s >> 1, e0 = 8 * (s & 1);
      u32x4_t pw;
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        const float x0 = fast_exp2(fmaf(sacc[kb][e0 + 2 * wd], p.sl2, mneg));
        const float x1 = fast_exp2(fmaf(sacc[kb][e0 + 2 * wd + 1], p.sl2, mneg));
        pw[wd] = pack_bf16x2(x0, x1);
        lsum = add_bf16_pair(pw[wd], lsum);
        if (LSE) l_lse += x0 + x1;
      }
      pf[s] = as_bf16x8(pw);
    }
  };
  // deferred form (kernels without an LSE output): the exponentials are taken
  // against the current reference first, so no row max precedes them; the
  // tile's P sum then shows whether a score exceeded the reference by more
  // than 2^8 (sum above 32 * 2^8, an overflow, or the first tile, whose
  // reference is -inf), and only such a tile moves the maximum and takes its
  // exponentials again.  P stays <= 2^13.
  auto softmax_check = [&](f32x16_t (&sacc)[2], bf16x8_t (&pf)[KT / 16], float lt) {
    if (__builtin_amdgcn_ballot_w64(!(lt <= kDeferredLimit)) != 0) {
      move_max(tile_max(sacc));
      lt = 0.f;
      softmax_p(sacc, pf, lt);
    }
    l_run += lt;
  };
  // O^T += V^T P^T with the V tile in BUF; V^T fragments by LDS transpose
  // reads (lane group lane/16 reads 4 consecutive key rows, lane i%16 gets
  // column i)
  auto pv = [&](auto buf_c, const bf16x8_t (&pf)[KT / 16]) {
    constexpr int BUF = decltype(buf_c)::value;
    const char* vt = lbase + BUF * STAGE_BYTES + TILE_BYTES;
#pragma unroll
    for (int s = 0; s < KT / 16; ++s) {
#pragma unroll
      for (int b = 0; b < DB; ++b) {
        const char* a0p = vt + (16 * s) * ROWB + voff_tr[0][b];    // slots e = 0..3
        const char* a1p = vt + (16 * s) * ROWB + voff_tr[1][b];    // slots e = 4..7
        const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_ptr)(a0p));
        const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_ptr)(a1p));
        const bf16x8_t a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        oacc[b] = mfma32x32x16(a, pf[s], oacc[b]);
      }
    }
  };

  // Software pipeline.  Iteration t (buffer parity P = t & 1) waits for K_{t+1}
  // and V_t, issues the gathers of V_{t+1} (into V buffer P^1) and K_{t+2}
  // (into K buffer P), takes the row max of S_t (eager form only), then in
  // one branch-free block computes S_{t+1} = K_{t+1} Q^T on MFMA interleaved
  // with the exponentials of S_t on the VALU, and O += V_t P_t.  Only the
  // last tile can be partial; it is peeled off and masked.
  // Sparse: the gathered rows' offsets of tile t stay in offs[t & 1] from
  // its K gather (two steps ahead) to its V gather (one step ahead).
  uint32_t offs[2][IPW] = {};
  auto step_head = [&](auto par_c, int t) {
    constexpr int P = decltype(par_c)::value;
    wait_vmem_all();
    __syncthreads();
    if (SPARSE && t % IDS_CHUNK == 0 && t + IDS_CHUNK < ntiles) refill_ids(t / IDS_CHUNK + 1);
    if (t + 1 < ntiles) issue_v(ic<P ^ 1>{}, offs[P ^ 1], t + 1);
    if (t + 2 < ntiles) {
      if (SPARSE) fetch_ids(t + 2, offs[P]);
      issue_k(ic<P>{}, offs[P], t + 2);
    }
  };
  auto steady_step = [&](auto par_c, int t, f32x16_t (&s_cur)[2], f32x16_t (&s_nxt)[2]) {
    constexpr int P = decltype(par_c)::value;
    constexpr int LOOKAHEAD = MCS_SCHED_LOOKAHEAD;
    // K fragment reads run LOOKAHEAD MFMAs ahead; each S MFMA is followed by
    // a share of the exponentials' VALU work
    auto interleave_s = [&]() {
      __builtin_amdgcn_sched_group_barrier(0x100, LOOKAHEAD, 0);        // DS read
#pragma unroll
      for (int i = 0; i < 2 * KSTEPS; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);              // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, MCS_SCHED_VALU, 0); // VALU
        if (i + LOOKAHEAD < 2 * KSTEPS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    };
    step_head(par_c, t);
    bf16x8_t pf[KT / 16];
    if constexpr (LSE) {
      softmax_max(s_cur);
      softmax_p(s_cur, pf, l_run);
      compute_s(ic<P ^ 1>{}, s_nxt);
      pv(ic<P>{}, pf);
      interleave_s();
    } else {
      float lt = 0.f;
      softmax_p(s_cur, pf, lt);
      compute_s(ic<P ^ 1>{}, s_nxt);
      interleave_s();
      softmax_check(s_cur, pf, lt);
      pv(ic<P>{}, pf);
    }
    // then the PV MFMAs with their transpose reads, also run ahead
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * LOOKAHEAD, 0);    // DS read (transpose)
#pragma unroll
    for (int i = 0; i < (KT / 16) * DB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);              // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);              // VALU
      if (i + LOOKAHEAD < (KT / 16) * DB) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
  };
  auto last_step = [&](auto par_c, int t, f32x16_t (&s_cur)[2]) {
    constexpr int P = decltype(par_c)::value;
    step_head(par_c, t);
    if ((t + 1) * KT > nkeys) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = t * KT + kb * 32 + 8 * (e >> 2) + 4 * hh + (e & 3);
          if (key >= nkeys) s_cur[kb][e] = -INFINITY;
        }
    }
    softmax_max(s_cur);
    bf16x8_t pf[KT / 16];
    softmax_p(s_cur, pf, l_run);
    pv(ic<P>{}, pf);
  };

  if (SPARSE) {
    refill_ids(0);
    wait_vmem_all();
    __syncthreads();
  }
  if (SPARSE) fetch_ids(0, offs[0]);
  issue_k(ic<0>{}, offs[0], 0);
  issue_v(ic<0>{}, offs[0], 0);
  if (ntiles > 1) {
    if (SPARSE) fetch_ids(1, offs[1]);
    issue_k(ic<1>{}, offs[1], 1);
  }
  wait_vmem_all();
  __syncthreads();
  f32x16_t sa[2], sb[2];
  compute_s(ic<0>{}, sa);
  int t = 0;
  for (; t + 2 < ntiles; t += 2) {
    steady_step(ic<0>{}, t, sa, sb);
    steady_step(ic<1>{}, t + 1, sb, sa);
  }
  if (t + 1 < ntiles) {        // tiles t (full) and t + 1 (last) remain
    steady_step(ic<0>{}, t, sa, sb);
    last_step(ic<1>{}, t + 1, sb);
  } else {                     // tile t is the last
    last_step(ic<0>{}, t, sa);
  }

  // ---- epilogue ----
  const float l_tot = halves_sum(l_run);
  const float l_exact = LSE ? halves_sum(l_lse) : 0.f;
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
  if (LSE && hh == 0) p.lse[head + qrow] = (m_run + fast_log2(l_exact)) * kLn2;
}

template <int D, int NW, bool SPARSE, bool RES, bool LSE, bool OUTF32>
static hipError_t launch_attn(const AttnParams& p, hipStream_t s) {
  const int total = p.BH * p.G;
  hipLaunchKernelGGL((attn_kernel<D, NW, SPARSE, RES, LSE, OUTF32>), dim3(total), dim3(NW * 64), 0,
                     s, p);
  return hipGetLastError();
}

template <int D, int NW, bool OUTF32>
static hipError_t dispatch_sparse(const AttnParams& p, bool res, bool lse, hipStream_t s) {
  if (lse) return launch_attn<D, NW, true, false, true, OUTF32>(p, s);   // no residual (checked)
  return res ? launch_attn<D, NW, true, true, false, OUTF32>(p, s)
             : launch_attn<D, NW, true, false, false, OUTF32>(p, s);
}

// The dense pass has no query groups: it always runs workgroups of 128 query
// rows (four waves), so only those variants are built.
template <int D, bool OUTF32>
static hipError_t dispatch_dense(const AttnParams& p, bool lse, hipStream_t s) {
  return lse ? launch_attn<D, 4, false, false, true, OUTF32>(p, s)
             : launch_attn<D, 4, false, false, false, OUTF32>(p, s);
}

template <bool OUTF32>
static hipError_t dispatch_shape(const AttnParams& p, int D, int C, bool sparse, bool res, bool lse,
                                 hipStream_t s) {
  if (!sparse) {
    if (C != 128) return hipErrorInvalidValue;
    return D == 128 ? dispatch_dense<128, OUTF32>(p, lse, s) : dispatch_dense<64, OUTF32>(p, lse, s);
  }
  if (D == 128) {
    return C == 128 ? dispatch_sparse<128, 4, OUTF32>(p, res, lse, s)
                    : dispatch_sparse<128, 2, OUTF32>(p, res, lse, s);
  }
  return C == 128 ? dispatch_sparse<64, 4, OUTF32>(p, res, lse, s)
                  : dispatch_sparse<64, 2, OUTF32>(p, res, lse, s);
}

hipError_t run_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         const int32_t* perm, const int32_t* kv_idx, const int32_t* kv_count,
                         const uint16_t* res, void* o, bool out_f32, float* lse, int B, int H, int N,
                         int D, int C, int K, float scale, hipStream_t s) {
  AttnParams p;
  p.q = q; p.k = k; p.v = v; p.perm = perm; p.kv_idx = kv_idx; p.kv_count = kv_count; p.res = res;
  p.o = o; p.lse = lse;
  p.N = N; p.C = C; p.K = K; p.G = (N + C - 1) / C; p.BH = B * H;
  p.sl2 = scale * kLog2e;
  const bool sparse = kv_idx != nullptr;
  return out_f32 ? dispatch_shape<true>(p, D, C, sparse, res != nullptr, lse != nullptr, s)
                 : dispatch_shape<false>(p, D, C, sparse, res != nullptr, lse != nullptr, s);
}

}  // namespace mcs
