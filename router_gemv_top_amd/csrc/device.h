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

// Every counter sits in its own 128-byte line, so atomics and polls on one
// counter do not queue behind traffic on another.
constexpr int kCtrStride = 32;  // u32 words between neighbouring counters

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
// Wave64 reductions with DPP. Inside each row of 16 lanes four DPP steps
// (quad_perm xor 1, quad_perm xor 2, row_half_mirror, row_mirror) combine
// every lane with a partner, so every lane ends with the row result; the four
// row results are then read as scalars and combined in a fixed order. Every
// step combines the same two operands on both sides, so the result is
// deterministic and the same in every lane.
// ---------------------------------------------------------------------------
constexpr int kDppQuadXor1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // row_half_mirror
constexpr int kDppMirror = 0x140;     // row_mirror

// row_shl:n (lane i of a 16-lane row takes lane i+n; lanes past the row end
// take 0).
template <int N>
__device__ __forceinline__ u32 dpp_row_shl(u32 v) {
  return (u32)__builtin_amdgcn_update_dpp(0, (int)v, 0x100 + N, 0xF, 0xF, true);
}

// Workgroups are dispatched to the 8 XCDs round-robin (block b runs on XCD
// b % 8). Map block b to tile t so that each XCD gets one contiguous run of
// tiles: tiles that share an x slice (consecutive t) then share an L2, and x
// is fetched from memory once per slice instead of once per XCD.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_tile(int b, int tiles) {
  const int x = b % kXcds, local = b / kXcds;
  const int per = tiles / kXcds, rem = tiles % kXcds;
  return x * per + min(x, rem) + local;
}

template <int CTRL>
__device__ __forceinline__ u32 dpp_u32(u32 v) {
  return (u32)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ u32 umax(u32 a, u32 b) { return a > b ? a : b; }
__device__ __forceinline__ u32 readlane_u32(u32 v, int l) { return (u32)__builtin_amdgcn_readlane((int)v, l); }
__device__ __forceinline__ float readlane_f32(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ double readlane_f64(double v, int l) {
  const u64 b = __double_as_longlong(v);
  const u32 lo = readlane_u32((u32)b, l), hi = readlane_u32((u32)(b >> 32), l);
  return __longlong_as_double((long long)(((u64)hi << 32) | lo));
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f32<kDppQuadXor1>(v);
  v += dpp_f32<kDppQuadXor2>(v);
  v += dpp_f32<kDppHalfMirror>(v);
  v += dpp_f32<kDppMirror>(v);
  return (readlane_f32(v, 0) + readlane_f32(v, 16)) + (readlane_f32(v, 32) + readlane_f32(v, 48));
}

__device__ __forceinline__ int wave_sum_i32(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, kDppQuadXor1, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, kDppQuadXor2, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, kDppHalfMirror, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, kDppMirror, 0xF, 0xF, false);
  return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) + __builtin_amdgcn_readlane(v, 32) +
         __builtin_amdgcn_readlane(v, 48);
}

// Inclusive prefix sum over the 64 lanes: DPP row_shr steps inside each row
// of 16 lanes (shifted-in lanes read 0), then the row totals are read as
// scalars and added to the later rows.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);  // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31),
            r2 = __builtin_amdgcn_readlane(v, 47);
  const int row = __lane_id() >> 4;
  return v + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}

// u / d for u * d < 2^32, with magic = ceil(2^32 / d) (d >= 2) from the
// host: the high word of u * magic (one multiply instead of a division).
__device__ __forceinline__ int div_magic(int u, u32 magic) { return (int)__umulhi((u32)u, magic); }

// Wave maximum: the row maximum by DPP, then row_bcast:15 carries rows 0 and
// 2 into rows 1 and 3 and row_bcast:31 carries row 1 into rows 2 and 3, so
// lane 63 ends with the maximum of all 64 lanes.
__device__ __forceinline__ u32 wave_max_u32(u32 v) {
  v = umax(v, dpp_u32<kDppQuadXor1>(v));
  v = umax(v, dpp_u32<kDppQuadXor2>(v));
  v = umax(v, dpp_u32<kDppHalfMirror>(v));
  v = umax(v, dpp_u32<kDppMirror>(v));
  v = umax(v, (u32)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x142, 0xa, 0xf, false));  // row_bcast:15
  v = umax(v, (u32)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x143, 0xc, 0xf, false));  // row_bcast:31
  return readlane_u32(v, 63);
}

__device__ __forceinline__ u64 ballot64(bool p) { return __ballot(p); }

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Mask of lanes below the calling lane.
__device__ __forceinline__ u64 lanemask_lt() {
  int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// ---------------------------------------------------------------------------
// Arrival counters and bounded waits. Counters live in the caller's
// workspace; they start at zero and every launch leaves them at zero.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void or_agent(u32* p, u32 v) {
  __hip_atomic_fetch_or(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Cross-workgroup data. Values one workgroup hands to another in the same
// launch (split-K partials, logits, top-k results) are moved with agent-scope
// relaxed atomic loads and stores: on gfx950 these are device-coherent memory
// operations (they bypass the non-coherent cache levels), so no L2 write-back
// or invalidate of the whole cache is needed to hand them over.
__device__ __forceinline__ void st_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(int32_t* p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t ld_agent(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ u32 ld_agent(const u32* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ u32 add_agent(u32* p, u32 v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(u32* p, u32 v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(u64* p, u64 v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ u64 ld_agent(const u64* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A kernel argument read from the kernarg segment where it is used. For
// values only the end of a kernel needs, in kernels whose arguments exceed
// the scalar register budget: loaded at the start, they are spilled to
// vector lanes and restored as a whole 16-register group before each use
// (16 v_readlane a store). The empty asm makes the segment pointer opaque,
// so the load stays where it is written (a scalar load, normally a hit in
// the scalar cache). off: the byte offset of the value in the segment.
template <class T>
__device__ __forceinline__ T kernarg_at(unsigned off) {
  typedef const __attribute__((address_space(4))) char* seg_ptr;
  seg_ptr p = (seg_ptr)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(p));
  return *(const __attribute__((address_space(4))) T*)(p + off);
}

// Tagged words: a 32-bit payload and the 32-bit tag of the call that wrote
// it, stored and loaded as one 8-byte atomic. A reader polls the word itself
// until the tag is its own call's, so data and "ready" arrive together and no
// counter, drain or separate load is needed for that hand-off.
__device__ __forceinline__ u64 tag_word(u32 payload, u32 tag) { return ((u64)tag << 32) | payload; }
__device__ __forceinline__ bool tag_ok(u64 w, u32 tag) { return (u32)(w >> 32) == tag; }

// 16-byte device-coherent load (buffer_load_dwordx4 with the sc1 cache
// policy) from a buffer of `bytes` bytes; out-of-range reads return zeros.
typedef u32 u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_rsrc(const void* base, u32 bytes) {
  // 0x00020000: raw 32-bit data format in the descriptor's last word.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4_t ld_agent16(__amdgpu_buffer_rsrc_t r, u32 byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 16 /* sc1 */);
}

// Wait until every vector memory operation this wave issued has completed
// (stores acknowledged at their scope), and keep the compiler from moving
// memory operations across this point. Publishing a hand-off is: each wave
// drains, the workgroup meets at a barrier, then one thread bumps the
// counter with an agent-scope atomic.
__device__ __forceinline__ void vm_drain() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Publish this workgroup's agent-scope stores and arrive on a counter.
// Returns the counter value before the add (in thread 0 only; 0 elsewhere).
__device__ __forceinline__ u32 publish_arrive(u32* ctr) {
  vm_drain();
  __syncthreads();
  u32 old = 0;
  if (threadIdx.x == 0) old = add_agent(ctr, 1u);
  return old;
}

// Real-time clock at a constant 100 MHz.
__device__ __forceinline__ u64 rt_clock() { return wall_clock64(); }

// Phase stamps of the trace build (compile with -DRGT_TRACE): thread 0 of each
// workgroup writes the real-time clock into trace[blockIdx.x * 16 + slot].
// Slots of the one-launch kernel: 0 start; 1 wave 0's tile done; 4 the
// workgroup's tile done; 3 tail entry; 11 first poll issued (norm path: rstd
// published); 15 poll loop done; 5 logits gathered; 12 scores + bias; 13 top-k
// selected; 14 selection ordered; 6 ids / weights written; 10 ids polled;
// 8 positions ready; 7 layout written; 9 quant stores issued; 2 stores
// acknowledged.
#ifdef RGT_TRACE
#define RGT_STAMP(trace, slot)                                                         \
  do {                                                                                 \
    if (threadIdx.x == 0 && (trace)) (trace)[blockIdx.x * 16 + (slot)] = rgt::rt_clock(); \
  } while (0)
#else
#define RGT_STAMP(trace, slot) \
  do {                         \
  } while (0)
#endif

// Spin (one thread) until *ctr - base >= target (unsigned, so a counter that
// only grows may wrap) or the deadline passes. On expiry the error word gets
// kErrTimeout and false is returned.
__device__ __forceinline__ bool wait_reach(const u32* ctr, u32 base, u32 target, u64 budget_ticks, u32* err) {
  u64 t0 = rt_clock();
  while (ld_agent(ctr) - base < target) {
    __builtin_amdgcn_s_sleep(2);
    if (rt_clock() - t0 > budget_ticks) {
      or_agent(err, kErrTimeout);
      return false;
    }
  }
  return true;
}

// ---------------------------------------------------------------------------
// e4m3fn codes of four bf16 values divided by 2^se. The division is a
// power-of-two scaling in fp32, exact whenever the result is a normal fp32
// (anything smaller is far below 2^-10 and rounds to zero in e4m3 anyway);
// clamping to +-448 makes every value that would round above 448 saturate to
// 448 (code 0x7e) and keeps the conversion clear of overflow; v_cvt_pk_fp8_f32
// then rounds to nearest, ties to even, onto the e4m3fn grid, normals and
// subnormals alike, and keeps the sign of zero (-0 -> 0x80).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float scaled_bf16(u32 bits_hi16, int se) {
  return __builtin_amdgcn_fmed3f(__builtin_amdgcn_ldexpf(__uint_as_float(bits_hi16), -se), -448.f, 448.f);
}
__device__ __forceinline__ u32 e4m3x4_of_bf16(u32 w0, u32 w1, int se) {
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(scaled_bf16(w0 << 16, se), scaled_bf16(w0 & 0xffff0000u, se), 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(scaled_bf16(w1 << 16, se), scaled_bf16(w1 & 0xffff0000u, se), r, true);
  return (u32)r;
}

// ---------------------------------------------------------------------------
// e2m1 (MXFP4 element) code of one bf16 value (in the high 16 bits) divided
// by 2^se. y = |v| / 2^se is exact in fp32 (or far below 0.25, where every
// rounding gives 0), and below 8 for every element of a block whose shared
// exponent follows the floor rule. The e2m1 grid (0, 0.5, 1, 1.5, 2, 3, 4, 6)
// has spacing 0.5 below 2, 1 below 4 and 2 above, so rounding to it is one
// round-to-nearest-even (v_rndne_f32) of y in units of its spacing, plus the
// code of the binade's first grid point; a result past 7 (y rounding to 8) is
// the saturation to 6. Sign in bit 3, so -0 gives 0x8.
// ---------------------------------------------------------------------------
__device__ __forceinline__ u32 e2m1_of_bf16(u32 bits_hi16, int se) {
  const float y = __builtin_amdgcn_ldexpf(__uint_as_float(bits_hi16 & 0x7fff0000u), -se);
  const bool lo = y < 2.f, mid = y < 4.f;
  const float units = lo ? 2.f : (mid ? 1.f : 0.5f);   // grid points per unit of y
  const float first = lo ? 0.f : (mid ? 2.f : 4.f);    // code of the binade's first point, minus its units
  const float c = __builtin_fminf(__builtin_rintf(y * units) + first, 7.f);
  return (u32)c | ((bits_hi16 >> 28) & 8u);
}
// Eight e2m1 codes of four bf16 pairs (the pair's low half is the earlier
// element), element 0 in bits 0-3, element 7 in bits 28-31.
__device__ __forceinline__ u32 e2m1x8_of_bf16(u32 w0, u32 w1, u32 w2, u32 w3, int se) {
  const u32 w[4] = {w0, w1, w2, w3};
  u32 r = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    r |= (e2m1_of_bf16(w[i] << 16, se) << (8 * i)) | (e2m1_of_bf16(w[i] & 0xffff0000u, se) << (8 * i + 4));
  return r;
}

// Shared exponent of a 32-element block from the largest magnitude's bits
// (bits & 0x7fff, all finite): clamp(floor(log2 amax) - 8, -127, 127), and
// -127 for an all-zero block.
// EMAX is the element format's largest binade: 8 for e4m3, 2 for e2m1.
template <int EMAX>
__device__ __forceinline__ int mx_shared_exp_e(u32 amax_bits) {
  const u32 ef = amax_bits >> 7;
  const u32 mf = amax_bits & 0x7fu;
  int e;
  if (ef) e = (int)ef - 127;
  else if (mf) e = (31 - __clz((int)mf)) - 133;
  else return -127;
  int se = e - EMAX;
  return se < -127 ? -127 : (se > 127 ? 127 : se);
}
__device__ __forceinline__ int mx_shared_exp(u32 amax_bits) { return mx_shared_exp_e<8>(amax_bits); }

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
__device__ __forceinline__ double exp64_recipe(double d) {
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
