// device.h - device-side building blocks of the routing front-end (gfx950).
//
// Wave64 reductions, cross-workgroup arrival counters and bounded waits,
// the bf16 -> e4m3fn encoder for MXFP8, and the fp64 exponential used by the
// top-k gate. Everything here is written for CDNA4: 64-lane wavefronts,
// agent-scope atomics that are coherent across the eight XCD L2 caches.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rgt {

typedef uint32_t u32;
typedef uint64_t u64;

constexpr int kWave = 64;

// Error bits kept in the workspace error word.
constexpr u32 kErrTimeout = 1u;

// ---------------------------------------------------------------------------
// bf16 helpers: a 32-bit word holds two bf16 values, element 0 in the low half.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(u32 v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(u32 v) { return __uint_as_float(v & 0xffff0000u); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

// acc + a.lo*b.lo + a.hi*b.hi with one v_dot2 instruction (two bf16 products,
// fp32 accumulate).
__device__ __forceinline__ float dot2_bf16(u32 a, u32 b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), acc, false);
}

// Dot product of two 16-byte bf16 vectors (8 products), added to acc.
__device__ __forceinline__ float dot8_bf16(uint4 a, uint4 b, float acc) {
  acc = dot2_bf16(a.x, b.x, acc);
  acc = dot2_bf16(a.y, b.y, acc);
  acc = dot2_bf16(a.z, b.z, acc);
  acc = dot2_bf16(a.w, b.w, acc);
  return acc;
}

// ---------------------------------------------------------------------------
// Wave64 reductions. The xor butterfly leaves the same bits in every lane
// (each step adds the same two operands on both sides), so the result is
// deterministic and uniform.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ u32 wave_max_u32(u32 v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    u32 t = (u32)__shfl_xor((int)v, o, kWave);
    v = t > v ? t : v;
  }
  return v;
}

__device__ __forceinline__ u64 ballot64(bool p) { return __ballot(p); }

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Mask of lanes below the calling lane.
__device__ __forceinline__ u64 lanemask_lt() {
  int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// ---------------------------------------------------------------------------
// Agent-scope arrival counters and bounded waits. Counters live in the
// caller's workspace; they start at zero and every launch leaves them at zero.
// ---------------------------------------------------------------------------
__device__ __forceinline__ u32 atomic_add_agent(u32* p, u32 v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ u32 atomic_load_agent(const u32* p) {
  return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void atomic_store_agent(u32* p, u32 v) {
  __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void atomic_or_agent(u32* p, u32 v) {
  __hip_atomic_fetch_or(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Real-time clock at a constant 100 MHz.
__device__ __forceinline__ u64 rt_clock() { return wall_clock64(); }

// Spin (one thread) until *ctr >= target or the deadline passes. On expiry
// the error word gets kErrTimeout and false is returned.
__device__ __forceinline__ bool wait_geq(const u32* ctr, u32 target, u64 budget_ticks, u32* err) {
  u64 t0 = rt_clock();
  while (atomic_load_agent(ctr) < target) {
    __builtin_amdgcn_s_sleep(1);
    if (rt_clock() - t0 > budget_ticks) {
      atomic_or_agent(err, kErrTimeout);
      return false;
    }
  }
  return true;
}

// ---------------------------------------------------------------------------
// MXFP8 element encoder: e4m3fn code of v / 2^se, where v is a bf16 given by
// its bits. Integer-only: v = sig * 2^e0 exactly, so v / 2^se = sig * 2^(e0-se)
// and rounding to the e4m3 grid is a shift with round-to-nearest-even.
// Saturates at 448 (code 0x7e), keeps the sign (so -0 -> 0x80).
// ---------------------------------------------------------------------------
__device__ __forceinline__ u32 e4m3_of_bf16(u32 h, int se) {
  const u32 sign = (h >> 8) & 0x80u;
  const u32 ef = (h >> 7) & 0xffu;
  const u32 mf = h & 0x7fu;
  if ((h & 0x7fffu) == 0) return sign;
  const int sig = ef ? (int)(mf | 0x80u) : (int)mf;
  const int ey = (ef ? (int)ef - 134 : -133) - se;  // value = sig * 2^ey
  const int msb = 31 - __clz(sig);
  const int binade = msb + ey;                       // floor(log2 value)
  if (binade > 8) return sign | 0x7eu;               // >= 512: saturate
  const int b = binade < -6 ? -6 : binade;           // subnormal grid below 2^-6
  const int sh = (b - 3) - ey;                       // grid spacing is 2^(b-3)
  u32 units;
  if (sh <= 0) {
    units = (u32)sig << (-sh);
  } else if (sh >= 9) {
    units = 0;                                       // sig < 2^8: below half a step
  } else {
    const u32 q = (u32)sig >> sh;
    const u32 rem = (u32)sig & ((1u << sh) - 1u);
    const u32 half = 1u << (sh - 1);
    units = q + ((rem > half || (rem == half && (q & 1u))) ? 1u : 0u);
  }
  if (units == 0) return sign;
  u32 code;
  if (b == -6 && units < 8) {
    code = units;                                    // subnormal
  } else {
    int bb = b;
    if (units >= 16) { units >>= 1; ++bb; }          // rounded up into the next binade
    code = ((u32)(bb + 7) << 3) | (units - 8);
  }
  if (code > 0x7eu) code = 0x7eu;                    // above 448 saturates
  return sign | code;
}

// Shared exponent of a 32-element block from the largest magnitude's bits
// (bits & 0x7fff, all finite): clamp(floor(log2 amax) - 8, -127, 127), and
// -127 for an all-zero block.
__device__ __forceinline__ int mx_shared_exp(u32 amax_bits) {
  const u32 ef = amax_bits >> 7;
  const u32 mf = amax_bits & 0x7fu;
  int e;
  if (ef) e = (int)ef - 127;
  else if (mf) e = (31 - __clz((int)mf)) - 133;
  else return -127;
  int se = e - 8;
  return se < -127 ? -127 : (se > 127 ? 127 : se);
}

// ---------------------------------------------------------------------------
// exp(d) for d <= 0 in fp64 by a fixed operation sequence (Cody & Waite range
// reduction, degree-13 Taylor polynomial by Horner, exact scaling). Contraction
// into fused multiply-adds is switched off so that the sequence of IEEE
// operations is exactly the written one:
//   n = rint(d * log2(e)); r = (d - n*LN2_HI) - n*LN2_LO;
//   p = sum_{j<=13} r^j/j! (Horner, multiply then add); result p * 2^n;
//   d < -200 gives 0.
// LN2_HI is ln 2 cut to 24 significant bits, so n*LN2_HI is exact.
// ---------------------------------------------------------------------------
__device__ __noinline__ double exp64_recipe(double d) {
#pragma clang fp contract(off)
  if (d < -200.0) return 0.0;
  const double kLog2e = 0x1.71547652b82fep+0;
  const double kLn2Hi = 0x1.62e42e0000000p-1;
  const double kLn2Lo = 0x1.efa39ef35793cp-25;
  const double n = __builtin_rint(d * kLog2e);
  const double r = (d - n * kLn2Hi) - n * kLn2Lo;
  double p = 0x1.6124613a86d09p-33;  // 1/13!
  p = p * r; p = p + 0x1.1eed8eff8d898p-29;  // 1/12!
  p = p * r; p = p + 0x1.ae64567f544e4p-26;  // 1/11!
  p = p * r; p = p + 0x1.27e4fb7789f5cp-22;  // 1/10!
  p = p * r; p = p + 0x1.71de3a556c734p-19;  // 1/9!
  p = p * r; p = p + 0x1.a01a01a01a01ap-16;  // 1/8!
  p = p * r; p = p + 0x1.a01a01a01a01ap-13;  // 1/7!
  p = p * r; p = p + 0x1.6c16c16c16c17p-10;  // 1/6!
  p = p * r; p = p + 0x1.1111111111111p-7;   // 1/5!
  p = p * r; p = p + 0x1.5555555555555p-5;   // 1/4!
  p = p * r; p = p + 0x1.5555555555555p-3;   // 1/3!
  p = p * r; p = p + 0x1.0p-1;               // 1/2!
  p = p * r; p = p + 0x1.0p+0;               // 1/1!
  p = p * r; p = p + 0x1.0p+0;               // 1/0!
  return __builtin_ldexp(p, (int)n);
}

// Order-preserving map of a finite fp32 score to u32 (larger score -> larger
// key); -0 is first turned into +0 so the two compare equal. Key 0 is never
// produced for a finite score and marks "taken / absent".
__device__ __forceinline__ u32 score_key(float s) {
  u32 b = __float_as_uint(s);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key_score(u32 k) {
  u32 b = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(b);
}

}  // namespace rgt
