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

// Two fp32 values to a packed bf16 pair (lo in bits 0-15), round to nearest
// even: gfx950's packed conversion, one instruction for the pair (equal to
// bf16_rne on finite values).
__device__ __forceinline__ u32 bf16x2_rne(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_cvt_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(u32, __builtin_convertvector(v, bf16x2_cvt_t));
}

// h = bf16(x + r) on a pair of bf16 values (one fp32 add, nearest even).
__device__ __forceinline__ u32 add_bf16x2(u32 x, u32 r) {
  return bf16x2_rne(__fadd_rn(bf16_lo(x), bf16_lo(r)), __fadd_rn(bf16_hi(x), bf16_hi(r)));
}

// xn = bf16((h * rstd) * (1 + gamma)) on a pair of bf16 values.
__device__ __forceinline__ u32 norm_bf16x2(u32 h, u32 g, float rstd) {
  return bf16x2_rne(__fmul_rn(__fmul_rn(bf16_lo(h), rstd), __fadd_rn(1.0f, bf16_lo(g))),
                    __fmul_rn(__fmul_rn(bf16_hi(h), rstd), __fadd_rn(1.0f, bf16_hi(g))));
}

__device__ __forceinline__ uint4 add_bf16x8(uint4 x, uint4 r) {
  return make_uint4(add_bf16x2(x.x, r.x), add_bf16x2(x.y, r.y), add_bf16x2(x.z, r.z), add_bf16x2(x.w, r.w));
}

__device__ __forceinline__ uint4 norm_bf16x8(uint4 h, uint4 g, float rstd) {
  return make_uint4(norm_bf16x2(h.x, g.x, rstd), norm_bf16x2(h.y, g.y, rstd), norm_bf16x2(h.z, g.z, rstd),
                    norm_bf16x2(h.w, g.w, rstd));
}

// The row's rstd from its h values, held as 8-element chunks: chunk c of
// thread t is row chunk t + 256c (chunks past the row add nothing). Each
// thread sums its squares in chunk order with fused multiply-adds, each wave
// sums its lanes (wave_sum's fixed butterfly), and the four wave sums are
// added in wave order, so every workgroup that runs this on a row gets the
// same bits. The whole workgroup calls it (one barrier).
template <int CH>
__device__ __forceinline__ float row_rstd(const uint4 (&hv)[CH], int nch, int k, float eps) {
  __shared__ float s_part[4];
  const int t = threadIdx.x;
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    if (t + 256 * c < nch) {
      const u32* hw = reinterpret_cast<const u32*>(&hv[c]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a = bf16_lo(hw[i]), b = bf16_hi(hw[i]);
        ss = __builtin_fmaf(a, a, ss);
        ss = __builtin_fmaf(b, b, ss);
      }
    }
  }
  ss = wave_sum(ss);
  if ((t & 63) == 0) s_part[t >> 6] = ss;
  __syncthreads();
  const float total = ((s_part[0] + s_part[1]) + s_part[2]) + s_part[3];
  return __fdiv_rn(1.0f, __fsqrt_rn(__fadd_rn(__fdiv_rn(total, (float)k), eps)));
}

template <int CH>
__global__ void __launch_bounds__(256) rmsnorm_kernel(const uint16_t* x, int64_t ldx, const uint16_t* res,
                                                      int64_t ldr, const uint16_t* gamma, float eps, int k,
                                                      uint16_t* xn, int64_t ldxn, uint16_t* res_out, int64_t ldro,
                                                      float* rstd_out) {
  const int row = blockIdx.x, t = threadIdx.x;
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
    for (int c = 0; c < CH; ++c) hv[c] = add_bf16x8(hv[c], rv[c]);
  }
  const float rstd = row_rstd<CH>(hv, nch, k, eps);
  if (t == 0 && rstd_out) rstd_out[row] = rstd;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int idx = t + 256 * c;
    if (idx >= nch) continue;
    const uint4 gv = *reinterpret_cast<const uint4*>(gamma + 8 * idx);
    *reinterpret_cast<uint4*>(xn + (int64_t)row * ldxn + 8 * idx) = norm_bf16x8(hv[c], gv, rstd);
    if (res && res_out) *reinterpret_cast<uint4*>(res_out + (int64_t)row * ldro + 8 * idx) = hv[c];
  }
}

}  // namespace rgt
