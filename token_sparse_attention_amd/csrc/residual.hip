// Anchor-step residual R = O_dense - O_sparse (wispaper.ai, "Residual correction
// recovers the discarded tail": the anchor records the dense-minus-sparse output
// difference that reuse steps add back).  Elementwise, HBM-bound: 16-byte loads
// and stores (8 bf16 per thread and step), fp32 subtraction, bf16 store.
#include "mcs_common.h"
#include "mcs_internal.h"

namespace mcs {

// r may alias od or osp: every element is read and then written by the same
// thread, and no thread touches another's elements.
__global__ __launch_bounds__(256) void residual_kernel(const uint16_t* od, const uint16_t* osp,
                                                       uint16_t* r, int64_t n) {
  const int64_t nvec = n / 8;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nvec; i += stride) {
    const u32x4_t a = ldg16(od + i * 8);
    const u32x4_t b = ldg16(osp + i * 8);
    u32x4_t y;
#pragma unroll
    for (int wd = 0; wd < 4; ++wd)
      y[wd] = pack_bf16x2(bf16_lo(a[wd]) - bf16_lo(b[wd]), bf16_hi(a[wd]) - bf16_hi(b[wd]));
    *reinterpret_cast<u32x4_t*>(r + i * 8) = y;
  }
  // tail (n not a multiple of 8)
  const int64_t t = nvec * 8 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t < n) {
    const float x = __uint_as_float((uint32_t)od[t] << 16) - __uint_as_float((uint32_t)osp[t] << 16);
    r[t] = (uint16_t)(pack_bf16x2(x, 0.f) & 0xffffu);
  }
}

hipError_t run_residual(const uint16_t* od, const uint16_t* osp, uint16_t* r, int64_t n,
                        hipStream_t s) {
  const int64_t nvec = n / 8;
  // One 16-byte vector per thread.  The same loop over a grid capped at 32
  // workgroups per CU measured 4.2-4.7 TB/s at the large shape, the full grid
  // 6 TB/s; the grid-stride loop only serves grids past the launch limit.
  int64_t blocks = (nvec + 255) / 256;
  if (blocks > (int64_t)1 << 30) blocks = (int64_t)1 << 30;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(residual_kernel, dim3((unsigned)blocks), dim3(256), 0, s, od, osp, r, n);
  return hipGetLastError();
}

}  // namespace mcs
