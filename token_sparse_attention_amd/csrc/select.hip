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
// through LDS in tiles of 64 (double buffered), starting at a tile taken from
// the clock so that concurrent workgroups share their K tiles in L2.  S = Q K^T on MFMA leaves one
// key per lane column, so each lane sums exp2(s*scale*log2e - lse_i*log2e)
// over its 16 query rows; the two half-waves' sums and the C/32 waves combine
// through LDS in a fixed order, one wave per tile in turn.  One fp32 mass row
// of N values per group goes to the workspace.  The fused form (aggregation and top-K in one
// kernel, as the ai.info page describes the second pass) also histograms the
// first digit of each finished mass during the sweep, then selects the K ids
// from the row it has just written, in the same workgroup: two more digit
// passes and the compaction read the row back (from cache while it is fresh),
// and the other workgroups' VALU-bound sweeps on the CU hide those reads.
//
// topk_reg_kernel: one 1024-thread workgroup per mass row of up to 81920
// values, held on chip (registers and LDS): radix select of the K-th largest
// value in passes of 12, 12 and 8 bits over one shared histogram (the finer
// passes over the keys that share the first digit, gathered into LDS), then an
// order-preserving compaction that writes the chosen ids in ascending order,
// equal values going to the smaller id.  topk_kernel: the same selection for
// longer rows, streaming the row from memory (four 8-bit passes with per-wave
// LDS histograms, then the compaction).
#include <type_traits>

#include "mcs_common.h"
#include "mcs_internal.h"
#include "mcs_radix.h"

namespace mcs {

constexpr int MKT = 64;  // keys per tile
// Sweep alignment: workgroups start their key sweep at the chunk of
// SWEEP_CHUNK tiles given by the 100 MHz clock, one chunk per SWEEP_TICKS
// (about the time a workgroup takes for a chunk at full occupancy: 4 waves
// per SIMD for C = 128, 2 for C = 64), so the workgroups resident on an XCD
// read the same K tiles at about the same time.  The masses do not depend on
// the order of the sweep.
constexpr int SWEEP_CHUNK = 32;
template <int NW>
constexpr int sweep_ticks() { return NW == 4 ? 7000 : 3500; }

struct MassParams {
  const uint16_t* q;
  const uint16_t* k;
  const float* lse;
  const int32_t* perm;
  float* mass;
  int32_t* idx;    // fused top-K: the chunk's [nh * G, K] ids
  int32_t N, C, G, bh0, nh, K;
  float sl2;
};

// Order key of a mass (a non-negative float): larger mass -> smaller key;
// -0.0 (and any negative value, which cannot occur) ranks as 0.  The full
// 32-bit key always has its top bit set, so 31 bits order the row.
__device__ __forceinline__ uint32_t mass_key31(uint32_t u) {
  return ~((u & 0x80000000u) ? 0u : u) & 0x7fffffffu;
}

template <int D, int NW, bool FUSED>
__global__ __launch_bounds__(NW * 64, 4) void group_mass_kernel(MassParams p) {
  constexpr int CH = D / 8;                 // 16-byte chunks per row
  constexpr int ROWB = D * 2;               // bytes per K row
  constexpr int KSTEPS = D / 16;
  constexpr int TILE_BYTES = MKT * ROWB;
  constexpr int INSTR = TILE_BYTES / 1024;  // 1 KiB DMA instructions per tile
  constexpr int IPW = INSTR / NW;
  constexpr int ROWS_PER_INSTR = 64 / CH;
  static_assert(INSTR % NW == 0 && MKT == 64 && (NW & (NW - 1)) == 0, "tile split");

  __shared__ __attribute__((aligned(1024))) uint16_t lds_k[2][MKT * D];
  // per tile buffer, wave and 32-key block: the 16-row partial sums of the
  // lanes, lane L holding key L % 32 of the block
  __shared__ float red[2][NW][2][64];
  // fused top-K: histogram of the first 9-bit digit of the keys, filled as
  // the masses are completed
  constexpr int H1 = 512;
  __shared__ uint32_t h1[FUSED ? H1 : 1];
  char* const lbase = reinterpret_cast<char*>(&lds_k[0][0]);

  const int tid = threadIdx.x;
  if (FUSED)
    for (int i = tid; i < H1; i += NW * 64) h1[i] = 0u;
  const int lane = tid & 63, lq = lane & 31, hh = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lb = xcd_remap(blockIdx.x, p.nh * p.G);
  const int hl = lb / p.G, g = lb - hl * p.G;
  const size_t head = (size_t)(p.bh0 + hl) * p.N;
  const uint16_t* __restrict__ qh = p.q + head * D;
  const __amdgpu_buffer_rsrc_t rk = head_rsrc_uniform(p.k + head * D, (uint32_t)p.N * ROWB);

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
    const uint32_t soff = __builtin_amdgcn_readfirstlane((uint32_t)tile * (uint32_t)TILE_BYTES);
#pragma unroll
    for (int j = 0; j < IPW; ++j) dma16s(rk, coff[j], soff, lbase + buf * TILE_BYTES + (w * IPW + j) * 1024);
  };
  // B fragment of k-step ks for key column lq of a 32-key block
  uint32_t koff[KSTEPS];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks)
    koff[ks] = (uint32_t)(lq * ROWB + (((2 * ks + hh) ^ swz<D>(lq)) << 4));

  // partial mass of one 32-key block: the sum over this lane's 16 query rows
  // (the partner lane L ^ 32 holds the other 16); four partial sums keep the
  // add chains short
  auto block_mass = [&](const f32x16_t& acc) {
    auto term = [&](int e) { return fast_exp2(fmaf(acc[e], p.sl2, -lse2[e])); };
    float s0 = term(0), s1 = term(1), s2 = term(2), s3 = term(3);
#pragma unroll
    for (int e = 4; e < 16; e += 4) {
      s0 += term(e);
      s1 += term(e + 1);
      s2 += term(e + 2);
      s3 += term(e + 3);
    }
    return (s0 + s1) + (s2 + s3);
  };

  float* __restrict__ mrow = p.mass + ((size_t)hl * p.G + g) * p.N;
  // the mass of key `lane` of tile t: per wave, the two half-wave partial
  // sums added, then the waves summed in order.  Wave t % NW does it, so the
  // work rotates over the SIMDs.
  const int ntiles = (p.N + MKT - 1) / MKT;
  // sweep order: iteration i handles tile (i + t0) mod ntiles, t0 taken from
  // the clock by one thread and shared
  int t0;
  {
    __shared__ int t0_sh;
    if (tid == 0) {
      const int nchunks = (ntiles + SWEEP_CHUNK - 1) / SWEEP_CHUNK;
      const uint64_t now = __builtin_amdgcn_s_memrealtime();
      t0_sh = (int)((now / (uint64_t)sweep_ticks<NW>()) % (uint64_t)nchunks) * SWEEP_CHUNK;
    }
    __syncthreads();
    t0 = __builtin_amdgcn_readfirstlane(t0_sh);
    if (t0 >= ntiles) t0 = 0;
  }
  auto tile_of = [&](int i) { const int t = i + t0; return t >= ntiles ? t - ntiles : t; };
  auto store_tile = [&](int i) {
    const int b = i & 1, blk = lane >> 5, lk = lane & 31;
    const int key = tile_of(i) * MKT + lane;
    if (w == (i & (NW - 1)) && key < p.N) {
      float s = red[b][0][blk][lk] + red[b][0][blk][32 + lk];
#pragma unroll
      for (int ww = 1; ww < NW; ++ww) s += red[b][ww][blk][lk] + red[b][ww][blk][32 + lk];
      mrow[key] = s;
      if (FUSED) atomicAdd(&h1[mass_key31(__float_as_uint(s)) >> 22], 1u);
    }
  };

  // Step t (tiles in sweep order): wait for K_t, barrier (K_{t-1} and the
  // partial masses of tile t-1 are then free / complete), gather K_{t+1} into
  // the other buffer, store tile t-1's mass, then S = Q K_t^T with the MFMA chains of the two
  // 32-key blocks alternating (independent accumulators back to back), then
  // the exponentials; the other waves on the SIMD fill the MFMA gaps.  The
  // loop is unrolled by the two buffers so all LDS offsets are immediates.
  auto step = [&](auto buf_c, int t) {
    constexpr int BUF = decltype(buf_c)::value;
    wait_vmem_all();
    __syncthreads();
    if (t + 1 < ntiles) issue(tile_of(t + 1), BUF ^ 1);
    if (t > 0) store_tile(t - 1);
    const char* kt = lbase + BUF * TILE_BYTES;
    f32x16_t acc0 = zero16(), acc1 = zero16();
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      acc0 = mfma32x32x16(qf[ks], as_bf16x8(*reinterpret_cast<const u32x4_t*>(kt + koff[ks])), acc0);
      acc1 = mfma32x32x16(qf[ks], as_bf16x8(*reinterpret_cast<const u32x4_t*>(kt + 32 * ROWB + koff[ks])), acc1);
    }
    red[BUF][w][0][lane] = block_mass(acc0);
    red[BUF][w][1][lane] = block_mass(acc1);
  };
  issue(tile_of(0), 0);
  int t = 0;
  for (; t + 1 < ntiles; t += 2) {
    step(std::integral_constant<int, 0>{}, t);
    step(std::integral_constant<int, 1>{}, t + 1);
  }
  if (t < ntiles) step(std::integral_constant<int, 0>{}, t);
  __syncthreads();
  store_tile(ntiles - 1);
  if (!FUSED) return;

  // ---- fused top-K over the group's own mass row, just written ----
  // Radix select of the K-th smallest 31-bit key in digits of 9 (histogram
  // built during the sweep), 11 and 11 bits, then the order-preserving
  // compaction (ties to the smaller id); the row is read back three times
  // (second digit; third digit with the counts; placing), or four when the
  // keys sharing the threshold's first 20 bits do not fit in LDS, in rounds
  // of NT * V positions with V consecutive keys per thread (one 16-byte load
  // when N % 4 == 0, so rows are 16-byte aligned; else V = 1).  Scratch
  // reuses the K tiles' LDS: an 11-bit histogram, the compaction's
  // per-(round, wave) counts and the gathered keys.
  constexpr int NT = NW * 64;
  constexpr int H2 = 2048;
  static_assert(sizeof(lds_k) >= H2 * 4, "scratch for the 11-bit histogram");
  __shared__ uint32_t wtot[NW];
  __shared__ uint32_t sel_digit, sel_below, cand_n;
  uint32_t* const sh = reinterpret_cast<uint32_t*>(lbase);
  const uint32_t* __restrict__ xr = reinterpret_cast<const uint32_t*>(mrow);
  int32_t* __restrict__ out = p.idx + ((size_t)hl * p.G + g) * p.K;
  const int N = p.N;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  __syncthreads();                           // row and first histogram complete

  // the bin of hist[0, NB) that holds the remaining-th smallest key: thread t
  // owns bins NB/NT * t ...; sets sel_digit and sel_below (keys in smaller bins)
  auto pick = [&](auto nb_c, const uint32_t* hist, uint32_t remaining) {
    constexpr int NB = decltype(nb_c)::value;
    constexpr int BPT = NB / NT;
    static_assert(NB % NT == 0, "bins split evenly over the threads");
    uint32_t c[BPT];
    uint32_t local = 0;
#pragma unroll
    for (int q = 0; q < BPT; ++q) {
      c[q] = hist[BPT * tid + q];
      local += c[q];
    }
    uint32_t incl = local;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    if (lane == 63) wtot[w] = incl;
    __syncthreads();
    uint32_t wbase = 0;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww)
      if (ww < w) wbase += wtot[ww];
    const uint32_t excl = wbase + incl - local;
    if (excl < remaining && remaining <= excl + local) {
      uint32_t acc = excl;
#pragma unroll
      for (int q = 0; q < BPT; ++q) {
        if (acc + c[q] >= remaining) {
          sel_digit = BPT * tid + q;
          sel_below = acc;
          break;
        }
        acc += c[q];
      }
    }
    __syncthreads();
  };

  auto select_row = [&](auto v_c) {
    constexpr int V = decltype(v_c)::value;
    constexpr int RB = 8;                    // rounds per batch of loads in flight
    const int rounds = (N + NT * V - 1) / (NT * V);   // the host keeps 2 * rounds * NW <= sh's size
    // f(round, first position, keys) for every round; positions past N hold
    // the key of a zero mass and are excluded by the callers
    auto walk = [&](auto f) {
      for (int r0 = 0; r0 < rounds; r0 += RB) {
        uint32_t u[RB][V];
#pragma unroll
        for (int j = 0; j < RB; ++j) {
          const int i = (r0 + j) * NT * V + V * tid;
          const bool ok = r0 + j < rounds && i < N;
          if (V == 4) {
            const u32x4_t x = ok ? *reinterpret_cast<const u32x4_t*>(xr + i) : zero_u32x4();
#pragma unroll
            for (int e = 0; e < V; ++e) u[j][e] = x[e];
          } else {
            u[j][0] = ok ? xr[i] : 0u;
          }
        }
#pragma unroll
        for (int j = 0; j < RB; ++j)
          if (r0 + j < rounds) f(r0 + j, (r0 + j) * NT * V + V * tid, u[j]);
      }
    };

    pick(std::integral_constant<int, H1>{}, h1, (uint32_t)p.K);
    uint32_t prefix = sel_digit << 22, pmask = 511u << 22;
    uint32_t remaining = (uint32_t)p.K - sel_below;
    // second digit (bits 21..11) among the keys that share the first
    for (int i = tid; i < H2; i += NT) sh[i] = 0u;
    __syncthreads();
    walk([&](int, int i0, const uint32_t (&u)[V]) {
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const uint32_t key = mass_key31(u[e]);
        if (i0 + e < N && (key & pmask) == prefix) atomicAdd(&sh[(key >> 11) & 2047u], 1u);
      }
    });
    __syncthreads();
    pick(std::integral_constant<int, H2>{}, sh, remaining);
    prefix |= sel_digit << 11;
    pmask |= 2047u << 11;
    remaining -= sel_below;

    // Third digit (bits 10..0).  The same read also counts, per round and
    // wave, the keys whose first 20 bits are below the threshold's (all of
    // them are below T) and gathers the few that share those bits, with their
    // positions: once T is known they complete the counts, so no separate
    // counting read is needed.  When the LDS has no room for them beside the
    // histogram and the counts, or they do not fit, the counting read runs.
    constexpr int WORDS = (int)(sizeof(lds_k) / 4);
    const int cap = (WORDS - H2 - 2 * rounds * NW) / 2;        // (key, position) pairs
    const bool merged = cap >= 64;
    uint32_t* const cnt_lt = merged ? sh + H2 : sh;
    uint32_t* const cnt_eq = cnt_lt + rounds * NW;
    uint32_t* const cand = cnt_eq + rounds * NW;
    for (int i = tid; i < H2; i += NT) sh[i] = 0u;
    if (tid == 0) cand_n = 0u;
    __syncthreads();
    walk([&](int r, int i0, const uint32_t (&u)[V]) {
      uint32_t nlt = 0;
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const uint32_t key = mass_key31(u[e]);
        const bool valid = i0 + e < N;
        const bool c = valid && (key & pmask) == prefix;
        if (c) atomicAdd(&sh[key & 2047u], 1u);
        if (merged) {
          nlt += (uint32_t)__popcll(__ballot(valid && (key & pmask) < prefix));
          const uint64_t bc = __ballot(c);
          uint32_t base = 0;
          if (lane == 0 && bc) base = atomicAdd(&cand_n, (uint32_t)__popcll(bc));
          base = __shfl(base, 0);
          const uint32_t at = base + (uint32_t)__popcll(bc & lt_mask);
          if (c && at < (uint32_t)cap) {
            cand[2 * at] = key;
            cand[2 * at + 1] = (uint32_t)(i0 + e);
          }
        }
      }
      if (merged && lane == 0) {
        cnt_lt[r * NW + w] = nlt;
        cnt_eq[r * NW + w] = 0u;
      }
    });
    __syncthreads();
    const uint32_t ncand = cand_n;
    pick(std::integral_constant<int, H2>{}, sh, remaining);
    const uint32_t T = prefix | sel_digit;
    const uint32_t need = remaining - sel_below;

    if (merged && ncand <= (uint32_t)cap) {
      // complete the counts with the gathered keys
      for (uint32_t j = tid; j < ncand; j += NT) {
        const uint32_t key = cand[2 * j], pos = cand[2 * j + 1];
        const uint32_t r = pos / (NT * V), ww = (pos % (NT * V)) / (64 * V);
        if (key < T) atomicAdd(&cnt_lt[r * NW + ww], 1u);
        else if (key == T) atomicAdd(&cnt_eq[r * NW + ww], 1u);
      }
    } else {
      // compaction, step 1 as its own read: per round and wave, the keys
      // below and equal to T
      walk([&](int r, int i0, const uint32_t (&u)[V]) {
        uint32_t nlt = 0, neq = 0;
#pragma unroll
        for (int e = 0; e < V; ++e) {
          const uint32_t key = mass_key31(u[e]);
          const bool valid = i0 + e < N;
          nlt += (uint32_t)__popcll(__ballot(valid && key < T));
          neq += (uint32_t)__popcll(__ballot(valid && key == T));
        }
        if (lane == 0) {
          cnt_lt[r * NW + w] = nlt;
          cnt_eq[r * NW + w] = neq;
        }
      });
    }
    __syncthreads();
    // step 2: exclusive scans of both count arrays in position order (wave 0
    // scans the lt counts, wave 1 the eq counts; each lane owns a contiguous run)
    if (w < 2) {
      uint32_t* c = w == 0 ? cnt_lt : cnt_eq;
      const int total = rounds * NW;
      const int per = (total + 63) / 64;
      const int b0 = lane * per, b1 = min(total, b0 + per);
      uint32_t local = 0;
      for (int j = b0; j < b1; ++j) local += c[j];
      uint32_t incl = local;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
      }
      uint32_t run = incl - local;
      for (int j = b0; j < b1; ++j) {
        const uint32_t v = c[j];
        c[j] = run;
        run += v;
      }
    }
    __syncthreads();
    // step 3: place every chosen id: rank = #(keys < T before it) +
    // min(#(keys == T before it), need); a wave's positions in a round are
    // contiguous, lane-major, V per lane
    walk([&](int r, int i0, const uint32_t (&u)[V]) {
      bool lt[V], eq[V];
      uint32_t lt_before = cnt_lt[r * NW + w], eq_before = cnt_eq[r * NW + w];
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const uint32_t key = mass_key31(u[e]);
        const bool valid = i0 + e < N;
        lt[e] = valid && key < T;
        eq[e] = valid && key == T;
        lt_before += (uint32_t)__popcll(__ballot(lt[e]) & lt_mask);
        eq_before += (uint32_t)__popcll(__ballot(eq[e]) & lt_mask);
      }
#pragma unroll
      for (int e = 0; e < V; ++e) {
        if (lt[e] || (eq[e] && eq_before < need)) {
          const uint32_t rank = lt_before + (eq_before < need ? eq_before : need);
          if (rank < (uint32_t)p.K) out[rank] = i0 + e;   // rank < K by construction; kept as a bound
        }
        lt_before += lt[e];
        eq_before += eq[e];
      }
    });
  };
  if ((N & 3) == 0) select_row(std::integral_constant<int, 4>{});
  else select_row(std::integral_constant<int, 1>{});
}

hipError_t run_group_mass(const uint16_t* q, const uint16_t* k, const float* lse,
                          const int32_t* perm, float* mass, int bh0, int nh, int N, int D,
                          int C, float scale, hipStream_t s) {
  MassParams p;
  p.q = q; p.k = k; p.lse = lse; p.perm = perm; p.mass = mass;
  p.N = N; p.C = C; p.G = (N + C - 1) / C; p.bh0 = bh0; p.nh = nh;
  p.sl2 = scale * kLog2e;
  p.idx = nullptr; p.K = 0;
  const dim3 grid(nh * p.G);
  if (D == 128) {
    if (C == 128) hipLaunchKernelGGL((group_mass_kernel<128, 4, false>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((group_mass_kernel<128, 2, false>), grid, dim3(128), 0, s, p);
  } else {
    if (C == 128) hipLaunchKernelGGL((group_mass_kernel<64, 4, false>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((group_mass_kernel<64, 2, false>), grid, dim3(128), 0, s, p);
  }
  return hipGetLastError();
}

// The fused kernel keeps its compaction counts (2 per round of C/32 * 64
// positions and wave) in the LDS of the K tiles: 64 * D * 2 * 2 bytes.
bool select_fused_fits(int N, int D, int C) {
  const int64_t nt = (C / 32) * 64;
  const int64_t rounds = ((int64_t)N + nt - 1) / nt;
  return 2 * rounds * (C / 32) * 4 <= (int64_t)MKT * D * 2 * 2;
}

hipError_t run_select_fused(const uint16_t* q, const uint16_t* k, const float* lse,
                            const int32_t* perm, float* mass, int32_t* idx, int bh0, int nh,
                            int N, int D, int C, int K, float scale, hipStream_t s) {
  if (!select_fused_fits(N, D, C)) return hipErrorInvalidValue;
  MassParams p;
  p.q = q; p.k = k; p.lse = lse; p.perm = perm; p.mass = mass; p.idx = idx;
  p.N = N; p.C = C; p.G = (N + C - 1) / C; p.bh0 = bh0; p.nh = nh; p.K = K;
  p.sl2 = scale * kLog2e;
  const dim3 grid(nh * p.G);
  if (D == 128) {
    if (C == 128) hipLaunchKernelGGL((group_mass_kernel<128, 4, true>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((group_mass_kernel<128, 2, true>), grid, dim3(128), 0, s, p);
  } else {
    if (C == 128) hipLaunchKernelGGL((group_mass_kernel<64, 4, true>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((group_mass_kernel<64, 2, true>), grid, dim3(128), 0, s, p);
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

// Adds one to hist[bin] for every active lane (one LDS atomic per lane).
// Grouping the lanes of a wave that share a bin (a leader per bin, one atomic
// for the lot) was measured slower on the mass rows than the plain atomics.
__device__ __forceinline__ void hist_add(uint32_t* hist, bool active, uint32_t bin) {
  if (active) atomicAdd(&hist[bin], 1u);
}

// The same selection with the whole row held on chip (element i of the row in
// slot i / TOPK_NT of thread i % TOPK_NT; the first RSLOTS slots in
// registers, the rest in LDS): the row is read from memory once instead of
// once per radix pass and once more for the compaction.  Rows of up to
// TOPK_NT * SLOTS values.  Slots past the row end hold the largest key (that
// of a zero score): they rank after every element of the row, so they never
// change the K-th key (K <= n); the compaction skips them.  Only the keys that
// share the first 12-bit digit with the K-th key matter to the two finer
// passes; when they fit (up to CAND_CAP) they are gathered into LDS first, so
// those passes cost no more than their number.  The compaction counts, per
// round of TOPK_NT positions and per wave, the keys below and equal to the
// threshold, scans those counts once in position order, and then places every
// chosen id without further synchronisation.
template <int SLOTS, int RSLOTS>
__global__ __launch_bounds__(TOPK_NT) void topk_reg_kernel(const float* __restrict__ scores,
                                                          int32_t* __restrict__ idx, int n, int K) {
  constexpr int NWV = TOPK_NT / 64;
  constexpr int HBINS = 4096;
  constexpr int CAND_CAP = 6080;             // candidate keys (the LDS left beside the row)
  static_assert(CAND_CAP >= 2 * SLOTS * NWV, "the count arrays live in the candidate area");
  __shared__ uint32_t hist[HBINS];
  __shared__ uint32_t wtot[NWV];
  __shared__ uint32_t sel_digit, sel_below, ncand;
  __shared__ uint32_t kl[SLOTS - RSLOTS][TOPK_NT];
  // candidate keys during the finer passes, then [lt | eq][round * NWV + wave]
  // counts of the compaction, scanned in place
  __shared__ uint32_t cand_area[CAND_CAP];
  uint32_t (*cnt)[SLOTS * NWV] = reinterpret_cast<uint32_t (*)[SLOTS * NWV]>(cand_area);
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const size_t row = blockIdx.x;
  const uint32_t* __restrict__ x = reinterpret_cast<const uint32_t*>(scores) + row * (size_t)n;
  int32_t* __restrict__ out = idx + row * (size_t)K;
  const int nslots = (n + TOPK_NT - 1) / TOPK_NT;
  // larger score -> smaller key; -0.0 (and any negative, which is not allowed) -> as 0
  auto to_key = [](uint32_t u) -> uint32_t { return ~((u & 0x80000000u) ? 0u : u); };
  // register slots first, so the first histogram pass can start on them while
  // the LDS slots arrive by DMA (raw score bits; reads past the row end give
  // 0, a zero score)
  uint32_t kv[RSLOTS];
#pragma unroll
  for (int k = 0; k < RSLOTS; ++k) {
    const int i = k * TOPK_NT + tid;
    kv[k] = to_key(i < n ? x[i] : 0u);
  }
  const __amdgpu_buffer_rsrc_t rrow = head_rsrc(x, (uint32_t)n * 4u);
  for (int k = RSLOTS; k < nslots; ++k)
    dma4(rrow, (uint32_t)(k * TOPK_NT + tid) * 4u, &kl[k - RSLOTS][w * 64]);
  for (int i = tid; i < HBINS; i += TOPK_NT) hist[i] = 0u;
  if (tid == 0) ncand = 0u;
  __syncthreads();
  auto lkey = [&](int k) -> uint32_t { return to_key(kl[k - RSLOTS][tid]); };

  // the bin holding the remaining-th key of the histogram: thread t owns bins
  // 4t .. 4t+3; sets sel_digit and sel_below (keys in smaller bins)
  auto pick = [&](int remaining) {
    uint32_t c[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) c[q] = hist[4 * tid + q];
    const uint32_t local = c[0] + c[1] + c[2] + c[3];
    uint32_t incl = local;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    if (lane == 63) wtot[w] = incl;
    __syncthreads();
    uint32_t wbase = 0;
#pragma unroll
    for (int ww = 0; ww < NWV; ++ww)
      if (ww < w) wbase += wtot[ww];
    const uint32_t excl = wbase + incl - local;
    if (excl < (uint32_t)remaining && (uint32_t)remaining <= excl + local) {
      uint32_t acc = excl;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (acc + c[q] >= (uint32_t)remaining) {
          sel_digit = 4 * tid + q;
          sel_below = acc;
          break;
        }
        acc += c[q];
      }
    }
    __syncthreads();
  };

  // radix select of the K-th smallest key in passes of 12, 12 and 8 bits.
  // Pass 1 over the whole row: every key is active.
#pragma unroll
  for (int k = 0; k < RSLOTS; ++k)
    if (k < nslots) hist_add(hist, true, kv[k] >> 20);
  wait_vmem_all();
  __syncthreads();
#pragma unroll 2
  for (int k = RSLOTS; k < nslots; ++k) hist_add(hist, true, lkey(k) >> 20);
  __syncthreads();
  pick(K);
  uint32_t prefix = sel_digit << 20, pmask = 4095u << 20;
  int remaining = K - (int)sel_below;
  const uint32_t nbin = hist[sel_digit];     // keys sharing the first digit
  __syncthreads();                            // everyone has read hist before it is cleared

  // Passes 2 and 3 look only at keys that share the first digit.  When they
  // fit, they are first gathered into the count array (order does not matter
  // to a histogram), so these passes cost no more than their number; else the
  // passes walk the row again.
  uint32_t* cand = cand_area;
  const bool gathered = nbin <= (uint32_t)CAND_CAP;
  if (gathered) {
    auto gather = [&](uint32_t key) {
      const bool m = (key & pmask) == prefix;
      const uint64_t b = __ballot(m);
      uint32_t base = 0;
      if (lane == 0 && b) base = atomicAdd(&ncand, (uint32_t)__popcll(b));
      base = __shfl(base, 0);
      const uint64_t below = (lane == 0) ? 0ull : (b & (~0ull >> (64 - lane)));
      const uint32_t at = base + (uint32_t)__popcll(below);
      if (m && at < (uint32_t)CAND_CAP) cand[at] = key;   // at < nbin <= CAND_CAP by construction
    };
#pragma unroll
    for (int k = 0; k < RSLOTS; ++k)
      if (k < nslots) gather(kv[k]);
    for (int k = RSLOTS; k < nslots; ++k) gather(lkey(k));
    __syncthreads();
  }
  const uint32_t nc = gathered ? ncand : 0u;
  for (int pass = 1; pass < 3; ++pass) {
    const int shift = pass == 1 ? 8 : 0;
    const uint32_t dmask = pass == 2 ? 255u : 4095u;
    for (int i = tid; i < HBINS; i += TOPK_NT) hist[i] = 0u;
    __syncthreads();
    if (gathered) {
      for (uint32_t j0 = 0; j0 < nc; j0 += TOPK_NT) {
        const uint32_t j = j0 + (uint32_t)tid;
        const uint32_t key = j < nc ? cand[j] : 0u;
        hist_add(hist, j < nc && (key & pmask) == prefix, (key >> shift) & dmask);
      }
    } else {
#pragma unroll
      for (int k = 0; k < RSLOTS; ++k)
        if (k < nslots) hist_add(hist, (kv[k] & pmask) == prefix, (kv[k] >> shift) & dmask);
#pragma unroll 2
      for (int k = RSLOTS; k < nslots; ++k) {
        const uint32_t key = lkey(k);
        hist_add(hist, (key & pmask) == prefix, (key >> shift) & dmask);
      }
    }
    __syncthreads();
    pick(remaining);
    prefix |= sel_digit << shift;
    pmask |= dmask << shift;
    remaining -= (int)sel_below;
  }
  const uint32_t T = prefix;
  const int need = remaining;

  // compaction, step 1: per round and wave, the keys below and equal to T
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  auto count = [&](int k, uint32_t key) {
    const bool valid = k * TOPK_NT + tid < n;
    const uint64_t blt = __ballot(valid && key < T), beq = __ballot(valid && key == T);
    if (lane == 0) {
      cnt[0][k * NWV + w] = (uint32_t)__popcll(blt);
      cnt[1][k * NWV + w] = (uint32_t)__popcll(beq);
    }
  };
#pragma unroll
  for (int k = 0; k < RSLOTS; ++k)
    if (k < nslots) count(k, kv[k]);
  for (int k = RSLOTS; k < nslots; ++k) count(k, lkey(k));
  __syncthreads();
  // step 2: exclusive scans of both count arrays in position order (wave 0
  // scans the lt counts, wave 1 the eq counts; each lane owns a contiguous run)
  if (w < 2) {
    uint32_t* c = cnt[w];
    const int total = nslots * NWV;
    const int per = (total + 63) / 64;
    const int b0 = lane * per, b1 = min(total, b0 + per);
    uint32_t local = 0;
    for (int j = b0; j < b1; ++j) local += c[j];
    uint32_t incl = local;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    uint32_t run = incl - local;
    for (int j = b0; j < b1; ++j) {
      const uint32_t v = c[j];
      c[j] = run;
      run += v;
    }
  }
  __syncthreads();
  // step 3: place every chosen id: rank = #(keys < T before it) +
  // min(#(keys == T before it), need)
  auto place = [&](int k, uint32_t key) {
    const int i = k * TOPK_NT + tid;
    const bool valid = i < n;
    const bool lt = valid && key < T;
    const bool eq = valid && key == T;
    const uint64_t blt = __ballot(lt), beq = __ballot(eq);
    const uint32_t lt_before = cnt[0][k * NWV + w] + (uint32_t)__popcll(blt & lt_mask);
    const uint32_t eq_before = cnt[1][k * NWV + w] + (uint32_t)__popcll(beq & lt_mask);
    if (lt || (eq && eq_before < (uint32_t)need)) {
      const uint32_t rank = lt_before + (eq_before < (uint32_t)need ? eq_before : (uint32_t)need);
      if (rank < (uint32_t)K) out[rank] = i;   // rank < K by construction; kept as a bound
    }
  };
#pragma unroll
  for (int k = 0; k < RSLOTS; ++k)
    if (k < nslots) place(k, kv[k]);
  for (int k = RSLOTS; k < nslots; ++k) place(k, lkey(k));
}

constexpr int TOPK_REG_SLOTS = 80;    // rows of up to 81920 values
constexpr int TOPK_REG_RSLOTS = 50;   // ... the first 50 slots in registers, the rest in LDS

hipError_t run_topk(const float* scores, int32_t* idx, int64_t rows, int n, int K,
                    hipStream_t s) {
  const int64_t max_grid = 1 << 30;
  const bool in_regs = n <= TOPK_NT * TOPK_REG_SLOTS;
  for (int64_t r0 = 0; r0 < rows; r0 += max_grid) {
    const int64_t nr = rows - r0 < max_grid ? rows - r0 : max_grid;
    if (in_regs)
      hipLaunchKernelGGL((topk_reg_kernel<TOPK_REG_SLOTS, TOPK_REG_RSLOTS>), dim3((unsigned)nr), dim3(TOPK_NT), 0, s,
                         scores + r0 * (int64_t)n, idx + r0 * (int64_t)K, n, K);
    else
      hipLaunchKernelGGL(topk_kernel, dim3((unsigned)nr), dim3(TOPK_NT), 0, s,
                         scores + r0 * (int64_t)n, idx + r0 * (int64_t)K, n, K);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace mcs
