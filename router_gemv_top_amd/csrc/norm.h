// norm.h - the RMSNorm producer in front of the router.
//
// The Gemma RMSNorm (+ residual) producer of the MiniMax-M3.1-Flash MoE/GEMM
// kernels page (Summary: fp8 producers), which publishes each token's rstd
// (the "route on the norm's scale" commit of the MiniMax-M3.1 FFN monokernel
// page):
//   h    = bf16(fp32(x) + fp32(residual))   (or x without a residual)
//   rstd = 1 / sqrt(mean_i h_i^2 + eps)      (fp32; the sum's order is this kernel's)
//   xn_i = bf16(fp32(fp32(h_i * rstd) * fp32(1 + gamma_i)))
// One workgroup per row; thread t holds the 8-element chunks t, t + 256, ...
// of the row in registers between the sum of squares and the scaling, so the
// row is read once.
#pragma once

#include "device.h"

namespace rgt {

// fp32 -> bf16 bits, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ u32 bf16_rne(float f) {
  const u32 u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

template <int CH>
__global__ void __launch_bounds__(256) rmsnorm_kernel(const uint16_t* x, int64_t ldx, const uint16_t* res,
                                                      int64_t ldr, const uint16_t* gamma, float eps, int k,
                                                      uint16_t* xn, int64_t ldxn, uint16_t* res_out, int64_t ldro,
                                                      float* rstd_out) {
  __shared__ float s_part[4];
  const int row = blockIdx.x, t = threadIdx.x, wave = t >> 6;
  const int nch = k >> 3;
  uint4 hv[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int idx = min(t + 256 * c, nch - 1);
    hv[c] = *reinterpret_cast<const uint4*>(x + (int64_t)row * ldx + 8 * idx);
  }
  if (res) {
    uint4 rv[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int idx = min(t + 256 * c, nch - 1);
      rv[c] = *reinterpret_cast<const uint4*>(res + (int64_t)row * ldr + 8 * idx);
    }
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      u32* hw = reinterpret_cast<u32*>(&hv[c]);
      const u32* rw = reinterpret_cast<const u32*>(&rv[c]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32 lo = bf16_rne(__fadd_rn(bf16_lo(hw[i]), bf16_lo(rw[i])));
        const u32 hi = bf16_rne(__fadd_rn(bf16_hi(hw[i]), bf16_hi(rw[i])));
        hw[i] = lo | (hi << 16);
      }
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    if (t + 256 * c < nch) {
      const u32* hw = reinterpret_cast<const u32*>(&hv[c]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a = bf16_lo(hw[i]), b = bf16_hi(hw[i]);
        ss += a * a;
        ss += b * b;
      }
    }
  }
  ss = wave_sum(ss);
  if ((t & 63) == 0) s_part[wave] = ss;
  __syncthreads();
  const float total = ((s_part[0] + s_part[1]) + s_part[2]) + s_part[3];
  const float rstd = __fdiv_rn(1.0f, __fsqrt_rn(__fadd_rn(__fdiv_rn(total, (float)k), eps)));
  if (t == 0 && rstd_out) rstd_out[row] = rstd;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int idx = t + 256 * c;
    if (idx >= nch) continue;
    const uint4 gv = *reinterpret_cast<const uint4*>(gamma + 8 * idx);
    const u32* hw = reinterpret_cast<const u32*>(&hv[c]);
    const u32* gw = reinterpret_cast<const u32*>(&gv);
    uint4 out;
    u32* ow = reinterpret_cast<u32*>(&out);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lo = __fmul_rn(__fmul_rn(bf16_lo(hw[i]), rstd), __fadd_rn(1.0f, bf16_lo(gw[i])));
      const float hi = __fmul_rn(__fmul_rn(bf16_hi(hw[i]), rstd), __fadd_rn(1.0f, bf16_hi(gw[i])));
      ow[i] = bf16_rne(lo) | (bf16_rne(hi) << 16);
    }
    *reinterpret_cast<uint4*>(xn + (int64_t)row * ldxn + 8 * idx) = out;
    if (res && res_out) *reinterpret_cast<uint4*>(res_out + (int64_t)row * ldro + 8 * idx) = hv[c];
  }
}

}  // namespace rgt
