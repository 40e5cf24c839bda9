// Device-side building blocks shared by the gfx950 kernels of libmcs.
//
// Wave64 everywhere.  Matrix products use the CDNA4 bf16 MFMA
// v_mfma_f32_32x32x16_bf16: per lane an A fragment (8 bf16 of one row m = lane%32),
// a B fragment (8 bf16 of one column n = lane%32) and 16 fp32 accumulators.
// The kernels only rely on two facts about its lane layout:
//   * A and B use the same k-slot assignment (lane half lane/32, element e), so
//     whatever k each (half, e) slot stands for, loading A and B with the same
//     slot -> index mapping computes the intended contraction;
//   * accumulator element 4*j + i of lane L holds D[8*j + 4*(L/32) + i][L%32].
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace mcs {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16_t mfma32x32x16(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16_t zero16() {
  f32x16_t z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

__device__ __forceinline__ u32x4_t ldg16(const void* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t x) {
  return __builtin_bit_cast(bf16x8_t, x);
}

__device__ __forceinline__ u32x4_t zero_u32x4() {
  u32x4_t z = {0u, 0u, 0u, 0u};
  return z;
}

// 2^x on the transcendental unit (v_exp_f32).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
// log2(x) on the transcendental unit (v_log_f32).
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Two floats -> packed bf16 pair (lo in bits 0..15), round to nearest even
// (one v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// acc + lo(w) + hi(w) for a packed bf16 pair (v_dot2c_f32_bf16 against 1.0, 1.0).
__device__ __forceinline__ float add_bf16_pair(uint32_t w, float acc) {
  const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), ones, acc, false);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Values of lanes L and L^32 combined; every lane receives the pair
// (own, partner) in some order, so max and sum below are symmetric.
__device__ __forceinline__ float halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  // IEEE addition is commutative, so both lanes of a pair get the same sum.
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Values of lanes L and L^16 combined, as halves_sum: v_permlane16_swap
// exchanges the odd 16-lane rows of one operand with the even rows of the
// other, so with both operands x every lane receives (own, partner).
__device__ __forceinline__ float rows_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum over the 64 lanes of a wave, all on the VALU.  Every step pairs each
// lane with a partner under a permutation that is its own inverse (xor 1,
// xor 2, mirror within 8 and within 16 lanes, xor 16, xor 32), so both lanes
// of a pair add the same two values and every lane ends with bitwise the
// same total.
__device__ __forceinline__ float wave_sum(float x) {
  auto dpp = [](float v, auto ctrl_c) {
    constexpr int CTRL = decltype(ctrl_c)::value;
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
  };
  x += dpp(x, std::integral_constant<int, 0xB1>{});    // quad_perm [1,0,3,2]
  x += dpp(x, std::integral_constant<int, 0x4E>{});    // quad_perm [2,3,0,1]
  x += dpp(x, std::integral_constant<int, 0x141>{});   // row_half_mirror
  x += dpp(x, std::integral_constant<int, 0x140>{});   // row_mirror
  return halves_sum(rows_sum(x));
}

// Eight sums over the 64 lanes of a wave at once, by recursive halving: at
// each exchange a lane keeps half of its values, each added to its partner's
// copy.  v_permlane32_swap(x, y) swaps lanes 32..63 of x with lanes 0..31 of
// y, so a lower lane receives (own x, partner x) and an upper lane
// (partner y, own y); v_permlane16_swap does the same between the odd and
// even 16-lane rows; a DPP mirror pairs the two 8-lane halves of a row.
// Value k ends up fully summed in lanes 8k..8k+7 and is read from lane 8k,
// so every wave that runs this on the same inputs gets bitwise the same
// sums.  The sums are returned in h (wave-uniform).
__device__ __forceinline__ void wave_sum8(float (&h)[8]) {
  const int lane = __lane_id();
  float a[4], b[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {      // lanes l, l^32: lower keeps 0..3, upper 4..7
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(h[i]), __float_as_uint(h[i + 4]), false,
                                              false);
    a[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {      // lanes l, l^16: even rows keep a0, a1, odd rows a2, a3
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a[i]), __float_as_uint(a[i + 2]), false,
                                              false);
    b[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  auto dpp = [](float v, auto ctrl_c) {
    constexpr int CTRL = decltype(ctrl_c)::value;
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
  };
  const bool upper8 = (lane & 8) != 0;   // lanes l, 15-l of a row: low half keeps b0, high b1
  const float send = upper8 ? b[0] : b[1];
  float c = (upper8 ? b[1] : b[0]) + dpp(send, std::integral_constant<int, 0x140>{});   // row_mirror
  c += dpp(c, std::integral_constant<int, 0x141>{});   // row_half_mirror
  c += dpp(c, std::integral_constant<int, 0x4E>{});    // quad_perm [2,3,0,1]
  c += dpp(c, std::integral_constant<int, 0xB1>{});    // quad_perm [1,0,3,2]
#pragma unroll
  for (int k = 0; k < 8; ++k) h[k] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(c), 8 * k));
}

// A value that is the same in every lane, moved to a scalar register.
__device__ __forceinline__ float uniform_f(float x) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}

__device__ __forceinline__ int clamp_id(int v, int n) { return v < 0 ? 0 : (v >= n ? n - 1 : v); }

// Workgroup -> (head, group) order.  Workgroups are dispatched round-robin over
// the 8 XCDs; this remap hands every XCD one contiguous range of the logical
// (head, group) sequence, so the workgroups resident on one XCD work on
// neighbouring groups of the same head and share its L2.
__device__ __forceinline__ int xcd_remap(int block, int total) {
  const int nx = 8;
  const int xcd = block % nx;
  const int slot = block / nx;
  const int base = total / nx, extra = total % nx;
  return xcd * base + (xcd < extra ? xcd : extra) + slot;
}

typedef __attribute__((address_space(3))) void* lds_void_t;

// 16-byte chunk swizzle of a K or V row in LDS.  The gfx950 LDS has 64 banks of
// 4 bytes, i.e. 16 bank groups of 16 bytes; a ds_read_b128 serves 16 lanes per
// cycle and a ds_read_b64_tr_b16 32 lanes.  D = 128 (256-byte rows, bank
// group = physical chunk): f maps any 16 consecutive rows to a permutation of
// 0..15 (K fragment reads: 16 rows, one logical chunk) and the 4 rows of a
// transpose read (rows 4a..4a+3) to 0, 4, 8, 12 (+ a constant), so their 4
// consecutive chunks land in 16 distinct groups.  D = 64 (128-byte rows, two
// rows per bank row): the same two properties with the row's half taken into
// account.
template <int D>
__device__ __forceinline__ int swz(int row) {
  if (D == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
  return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

// Buffer resource of one head's K or V rows: loads at byte offsets at or past
// `bytes` return zeros (rows past the end of a tile, ids outside [0, N)).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// head_rsrc from a base and size made wave-uniform explicitly, for kernels in
// which the compiler would otherwise keep the descriptor in vector registers
// (the DMA instructions need it in scalar ones).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc_uniform(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return head_rsrc(reinterpret_cast<const void*>((uintptr_t)(((uint64_t)hi << 32) | lo)),
                   __builtin_amdgcn_readfirstlane(bytes));
}

// One 16-byte buffer load per lane written straight to LDS: the wave writes
// 1 KiB at lds (wave-uniform) + 16 * lane.
//
// Issued as inline assembly on purpose: the compiler cannot tell the LDS
// range a DMA writes from the ranges the tile loop reads, and for the builtin
// it places a full vmcnt wait before the next LDS read, which would make every
// tile step wait for the loads it has just issued.  The kernels order DMA and
// LDS reads themselves: an explicit vmcnt wait and a barrier before a buffer
// is read, and the DMA and the reads of one step touch disjoint buffers.
// VMEM operations the compiler does not see can only make its own (in-order)
// vmcnt waits stricter, never looser.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, void* lds) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(lds_void_t)lds;
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(r), "{m0}"(m0) : "memory");
}

// dma16 with a wave-uniform byte offset soff added to voff (the buffer's
// range check covers the sum: a load at or past the descriptor's end reads
// zeros; the LDS placement does not depend on soff).
__device__ __forceinline__ void dma16s(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, void* lds) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(lds_void_t)lds;
  asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(r), "s"(soff), "{m0}"(m0) : "memory");
}

// One 4-byte buffer load per lane written straight to LDS: the wave writes
// 256 bytes at lds (wave-uniform) + 4 * lane (same ordering rules as dma16).
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, uint32_t voff, void* lds) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(lds_void_t)lds;
  asm volatile("buffer_load_dword %0, %1, 0 offen lds" ::"v"(voff), "s"(r), "{m0}"(m0) : "memory");
}

__device__ __forceinline__ void wait_vmem_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

}  // namespace mcs
