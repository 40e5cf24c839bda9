// Workgroup-level selection of the r smallest 32-bit keys of a sequence, ties
// broken by position (earlier first), and the order-preserving compaction
// that follows.  Used by the top-K of the exact selector (keys = inverted
// score bits, so the largest scores are the smallest keys) and by the
// median split of PDDP (keys = order-preserving projection bits).
#pragma once

#include "mcs_common.h"

namespace mcs {

// Order-preserving map of a float to uint32 (ascending floats -> ascending keys).
__device__ __forceinline__ uint32_t float_order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int NT>
struct RadixLds {
  uint32_t hist[NT / 64][256];
  uint32_t wcnt[2][NT / 64][2];
  uint32_t digit, below, eqcnt;
};

// Finds T, the r-th smallest key (1 <= r <= n), and need = r - #(keys < T),
// the number of keys equal to T that belong to the r smallest (the first
// `need` of them in position order).  key(i) must be pure (re-evaluated).
template <int NT, class KeyFn>
__device__ void radix_select_smallest(KeyFn key, int n, int r, RadixLds<NT>& L, uint32_t& T,
                                      int& need) {
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  uint32_t prefix = 0, pmask = 0;
  int remaining = r;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < (NT / 64) * 256; i += NT) (&L.hist[0][0])[i] = 0u;
    __syncthreads();
    for (int i = tid; i < n; i += NT) {
      const uint32_t k = key(i);
      if ((k & pmask) == prefix) atomicAdd(&L.hist[w][(k >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 256) {
      uint32_t s = 0;
#pragma unroll
      for (int ww = 0; ww < NT / 64; ++ww) s += L.hist[ww][tid];
      L.hist[0][tid] = s;
    }
    __syncthreads();
    if (w == 0) {
      uint32_t c[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) c[k] = L.hist[0][4 * lane + k];
      const uint32_t local = c[0] + c[1] + c[2] + c[3];
      uint32_t incl = local;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
      }
      const uint32_t excl = incl - local;
      if (excl < (uint32_t)remaining && (uint32_t)remaining <= incl) {
        uint32_t acc = excl;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          if (acc + c[k] >= (uint32_t)remaining) {
            L.digit = 4 * lane + k;
            L.below = acc;
            L.eqcnt = c[k];
            break;
          }
          acc += c[k];
        }
      }
    }
    __syncthreads();
    prefix |= L.digit << shift;
    pmask |= 255u << shift;
    remaining -= (int)L.below;
  }
  T = prefix;
  need = remaining;
}

// Walks positions 0..n-1 in order.  Position i is selected when key(i) < T, or
// key(i) == T and fewer than `need` earlier positions had key == T.  Calls
// emit(i, selected, rank) for every i < n, with rank = number of selected
// positions before i if selected, else the number of unselected ones before i.
template <int NT, class KeyFn, class EmitFn>
__device__ void ordered_compact(KeyFn key, int n, uint32_t T, int need, RadixLds<NT>& L,
                                EmitFn emit) {
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  uint32_t base_lt = 0, base_eq = 0;
  int round = 0;
  for (int i0 = 0; i0 < n; i0 += NT, ++round) {
    const int i = i0 + tid;
    const bool valid = i < n;
    const uint32_t k = valid ? key(i) : 0xffffffffu;
    const bool lt = valid && k < T;
    const bool eq = valid && k == T;
    const uint64_t blt = __ballot(lt), beq = __ballot(eq);
    const uint32_t lt_before_w = __popcll(blt & lt_mask), eq_before_w = __popcll(beq & lt_mask);
    const int rb = round & 1;
    if (lane == 0) {
      L.wcnt[rb][w][0] = __popcll(blt);
      L.wcnt[rb][w][1] = __popcll(beq);
    }
    __syncthreads();
    uint32_t wl = 0, we = 0, tl = 0, te = 0;
#pragma unroll
    for (int ww = 0; ww < NT / 64; ++ww) {
      const uint32_t a = L.wcnt[rb][ww][0], b = L.wcnt[rb][ww][1];
      if (ww < w) {
        wl += a;
        we += b;
      }
      tl += a;
      te += b;
    }
    if (valid) {
      const uint32_t lt_before = base_lt + wl + lt_before_w;
      const uint32_t eq_before = base_eq + we + eq_before_w;
      const uint32_t sel_before = lt_before + (eq_before < (uint32_t)need ? eq_before : (uint32_t)need);
      const bool sel = lt || (eq && eq_before < (uint32_t)need);
      emit(i, sel, sel ? (int)sel_before : (int)((uint32_t)i - sel_before));
    }
    base_lt += tl;
    base_eq += te;
  }
}

}  // namespace mcs
