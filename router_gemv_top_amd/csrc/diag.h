// diag.h - measurement kernels: a pure streaming read (the floor a kernel
// that must read the same bytes cannot beat) and a plain copy (a kernel of
// known traffic for calibrating hardware byte counters).
#pragma once

#include "device.h"

namespace rgt {

// Every workgroup reads its share of `bytes` with 16-byte loads and folds
// the words into one value, stored per workgroup so the loads stay live.
__global__ void __launch_bounds__(256) diag_read_kernel(const uint4* src, size_t n16, u32* sink) {
  u32 acc = 0;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
    const uint4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  acc = (u32)wave_max_u32(acc);
  if (threadIdx.x == 0) sink[blockIdx.x] = acc;
}

__global__ void __launch_bounds__(256) diag_copy_kernel(const uint4* src, uint4* dst, size_t n16) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

}  // namespace rgt
