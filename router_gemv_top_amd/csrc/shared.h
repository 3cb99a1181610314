// shared.h - the router's split-K partials and the shared expert's gate/up
// SwiGLU on MXFP8 weights, in one launch.
//
// MiniMax-M3.1-Flash MoE/GEMM kernels page, Summary: Router: the split-K
// router exposes its partials (the gate sums them in order) and shares one
// launch with the shared expert's fp8 SwiGLU; Summary: GEMM: that shared
// expert's gate_up is 1536 x 6144. Its weights are MXFP8 (monokernel page,
// MXFP8 shared-expert commit): e4m3fn codes [2I][K], the I gate rows first,
// then the I up rows, and one e8m0 scale per 32 codes along K.
//
//   h[m][j] = bf16( silu(g) * u ),  g = x[m] . Wg[j],  u = x[m] . Wu[j]
//   silu(g) = g / (1 + exp(-g)), all in fp32.
//
// The grid is the router's VALU or MFMA tiles (their partials go straight to
// the caller's part[S][M][N]; no fixup) followed by the shared expert's
// workgroups: the VALU form described here up to 8 rows of x, the MFMA form
// further down for 9 to 16. A VALU-form workgroup (4 waves) takes 4 / KW
// columns j, KW waves a column, each wave 1/KW of K (KW = 2 for M <= 2, else 4). Lane l of a
// wave takes the 16-code chunks c = c0 + l + 64 i of the gate row and of the
// up row (16-byte loads: one wave load covers 1 KiB of a row), all
// issued before any arithmetic. A code widens exactly to bf16 (an e4m3 value
// has at most 4 significant bits and an exponent inside bf16's range), so
// v_dot2_f32_bf16 forms each chunk's dot product with the x row, and the
// chunk's power-of-two scale multiplies that sum into the fp32 accumulator
// (exact while the scaled sum stays above 2^-126). A wave butterfly reduces
// each part; the parts meet in LDS (added in part order), and lane m of the
// first part's wave finishes row m.
#pragma once

#include "gemv.h"
#include "norm.h"

namespace rgt {

struct SharedArgs {
  const u16* x;
  int64_t ldx;
  const uint8_t* wq;  // [2I][K] e4m3fn codes, rows K bytes apart
  const uint8_t* ws;  // [2I][K/32] e8m0 scale bytes, rows K/32 bytes apart
  u16* h;             // [M][ldh] bf16
  int64_t ldh;
  int m, k, inter;
};

constexpr int kSharedMaxM = 16;
constexpr int kSharedMaxK = 8192;  // at most 8 / KW 16-code chunks per lane

// e8m0 scale byte -> fp32 2^(b - 127): 0 is the subnormal 2^-127, 255 NaN.
__device__ __forceinline__ float e8m0_f32(u32 b) {
  u32 bits = b << 23;                        // integer selects, no branches
  bits = b == 0u ? 0x00400000u : bits;
  bits = b == 255u ? 0x7fc00000u : bits;
  return __uint_as_float(bits);
}

// Two e4m3fn codes (16-bit word HIW of d) -> one bf16 pair, the lower byte in the
// low half. The fp32 conversion is exact and its low 16 bits are zero.
template <bool HIW>
__device__ __forceinline__ u32 e4m3x2_bf16(u32 d) {
  const auto f = __builtin_amdgcn_cvt_pk_f32_fp8((int)d, HIW);
  return (__float_as_uint(f[1]) & 0xffff0000u) | (__float_as_uint(f[0]) >> 16);
}

// Sixteen codes (memory order) -> codes 0..7 and 8..15 as bf16 vectors.
__device__ __forceinline__ void e4m3x16_bf16(uint4 c, uint4& lo, uint4& hi) {
  lo = make_uint4(e4m3x2_bf16<false>(c.x), e4m3x2_bf16<true>(c.x), e4m3x2_bf16<false>(c.y), e4m3x2_bf16<true>(c.y));
  hi = make_uint4(e4m3x2_bf16<false>(c.z), e4m3x2_bf16<true>(c.z), e4m3x2_bf16<false>(c.w), e4m3x2_bf16<true>(c.w));
}

// Waves per column (each takes 1/KW of K): two for M <= 2, four from M = 4
// (measured at N = 128, K = 6144, I = 768: equal at M = 4, 11.3 -> 10.7 us at
// M = 8). The host sizes the grid with the same function.
constexpr int shared_kw(int mt) { return mt >= 4 ? 4 : 2; }

// lds: at least 4 * 2 * MT floats.
template <int MT>
__device__ __forceinline__ void shared_swiglu(const SharedArgs& b, int job, float* lds) {
  constexpr int KW = shared_kw(MT), COLS = 4 / KW;
  constexpr int NCH = kSharedMaxK / 1024 / KW;  // chunks per lane, at most
  // x loads of every chunk up front for up to 4 rows; 8 rows load x per chunk
  // (up front they take the 8-row instance to 176 VGPRs and 2 waves a SIMD:
  // measured 10.8 -> 11.3 us at M = 8, while M = 1 gains 5.5 -> 5.25 us)
  constexpr bool XPRE = MT <= 4;
  constexpr int XN = XPRE ? NCH : 1;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int slot = wave / KW, part = wave % KW;
  const int j = COLS * job + slot;
  const bool col_ok = j < b.inter;
  const int jc = col_ok ? j : b.inter - 1;  // an idle column loads a valid row and stores nothing
  const int ch = (b.k >> 4) / KW;           // chunks per wave
  const int kq = b.k >> 5;                  // scale bytes per row
  const uint8_t* rg = b.wq + (int64_t)jc * b.k;
  const uint8_t* ru = b.wq + (int64_t)(b.inter + jc) * b.k;
  const uint8_t* sg = b.ws + (int64_t)jc * kq;
  const uint8_t* su = b.ws + (int64_t)(b.inter + jc) * kq;
  // every weight load of the lane first (and, XPRE, every x load: one memory
  // round trip); rows past M read row M-1 (their sums are never stored)
  uint4 cg[NCH], cu[NCH], xa[XN][MT], xb[XN][MT];
  auto load_x = [&](int c, uint4(&ya)[MT], uint4(&yb)[MT]) {
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const u16* xr = b.x + (int64_t)min(m, b.m - 1) * b.ldx + 16 * c;
      ya[m] = ld16(xr);
      yb[m] = ld16(xr + 8);
    }
  };
  u32 eg[NCH], eu[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    if (64 * i < ch) {  // uniform; guards, not a break, keep the indexes constant
      const int q = lane + 64 * i;               // chunk index inside the wave's part
      const int c = part * ch + min(q, ch - 1);  // lanes past the part reload its last chunk (not used)
      cg[i] = *reinterpret_cast<const uint4*>(rg + 16 * c);
      cu[i] = *reinterpret_cast<const uint4*>(ru + 16 * c);
      eg[i] = sg[c >> 1];
      eu[i] = su[c >> 1];
      if constexpr (XPRE) load_x(c, xa[i], xb[i]);
    }
  }
  float accg[MT], accu[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) accg[m] = accu[m] = 0.f;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int q = lane + 64 * i;
    if (64 * i < ch && q < ch) {
      const int xi = XPRE ? i : 0;  // a constant once unrolled
      if constexpr (!XPRE) load_x(part * ch + q, xa[0], xb[0]);
      uint4 glo, ghi, ulo, uhi;
      e4m3x16_bf16(cg[i], glo, ghi);
      e4m3x16_bf16(cu[i], ulo, uhi);
      const float fg = e8m0_f32(eg[i]), fu = e8m0_f32(eu[i]);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const float pg = dot8_bf16(xb[xi][m], ghi, dot8_bf16(xa[xi][m], glo, 0.f));
        const float pu = dot8_bf16(xb[xi][m], uhi, dot8_bf16(xa[xi][m], ulo, 0.f));
        accg[m] = __fmaf_rn(fg, pg, accg[m]);
        accu[m] = __fmaf_rn(fu, pu, accu[m]);
      }
    }
  }
  // wave totals (uniform), then lane m keeps row m's
  float gm = 0.f, um = 0.f;
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const float tg = wave_sum(accg[m]), tu = wave_sum(accu[m]);
    if (lane == m) gm = tg, um = tu;
  }
  // parts 1..KW-1 hand their totals to part 0, which adds them in part order
  float* ex = lds + slot * (KW - 1) * 2 * MT;
  if (part > 0 && lane < MT) {
    ex[(part - 1) * 2 * MT + lane] = gm;
    ex[(part - 1) * 2 * MT + MT + lane] = um;
  }
  __syncthreads();
  if (part == 0 && lane < MT && lane < b.m && col_ok) {
    float g = gm, u = um;
#pragma unroll
    for (int q = 0; q < KW - 1; ++q) {
      g += ex[q * 2 * MT + lane];
      u += ex[q * 2 * MT + MT + lane];
    }
    const float sg_ = g / (1.f + expf(-g));
    b.h[(int64_t)lane * b.ldh + j] = (u16)bf16_rne(sg_ * u);
  }
}

// Sixteen codes times their power-of-two scale -> two bf16x8 MFMA operands
// (codes 0..7 and 8..15). Exact while each scaled value is zero or at least
// 2^-126 in magnitude (4 significant bits then fit bf16).
template <bool HIW>
__device__ __forceinline__ u32 e4m3x2_bf16_scaled(u32 d, float sc) {
  const auto f = __builtin_amdgcn_cvt_pk_f32_fp8((int)d, HIW);
  return (__float_as_uint(f[1] * sc) & 0xffff0000u) | (__float_as_uint(f[0] * sc) >> 16);
}
__device__ __forceinline__ void e4m3x16_bf16_scaled(uint4 c, float sc, uint4& lo, uint4& hi) {
  lo = make_uint4(e4m3x2_bf16_scaled<false>(c.x, sc), e4m3x2_bf16_scaled<true>(c.x, sc),
                  e4m3x2_bf16_scaled<false>(c.y, sc), e4m3x2_bf16_scaled<true>(c.y, sc));
  hi = make_uint4(e4m3x2_bf16_scaled<false>(c.z, sc), e4m3x2_bf16_scaled<true>(c.z, sc),
                  e4m3x2_bf16_scaled<false>(c.w, sc), e4m3x2_bf16_scaled<true>(c.w, sc));
}

// MFMA form for up to 16 rows of x: a workgroup takes MC columns as one
// 16-row weight tile (their gate and up rows) and x as the A operand (rows past M read row M-1 and are never
// stored), so one x load feeds 16 weight rows. Wave w takes the w-th quarter
// of K in 64-element steps; in a step, lane group g = lane/16 loads 16 codes
// at k + 16 g of weight row lane%16 (its scale is one byte: the run lies in
// one 32-group) and the same 16 elements of x row lane%16, which feed two
// v_mfma_f32_16x16x32_bf16. The four waves' 16 x 16 tiles meet in LDS, added
// in wave order, and thread t < 16 MC finishes row t/MC, column j0 + t%MC.
// lds: at least 4 * 256 floats.
constexpr int kSharedMfmaSteps = kSharedMaxK / 256;

// MC columns a tile (2, 4 or 8): B columns q < MC are their gate rows,
// MC <= q < 2 MC their up rows, and the rest repeat those (same addresses,
// so no extra memory traffic): narrower tiles give more workgroups.
template <int MC>
__device__ __forceinline__ void shared_swiglu_mfma(const SharedArgs& b, int job, float* lds) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r16 = lane & 15, grp = lane >> 4;
  const int q = r16 % (2 * MC);
  const int j0 = job * MC;
  const int jc = min(j0 + q % MC, b.inter - 1);  // idle columns load a valid row and store nothing
  const int wrow = q < MC ? jc : b.inter + jc;
  const int kq = b.k >> 5;
  const uint8_t* wr = b.wq + (int64_t)wrow * b.k;
  const uint8_t* sr = b.ws + (int64_t)wrow * kq;
  const u16* xr = b.x + (int64_t)min(r16, b.m - 1) * b.ldx;
  const int kw = b.k >> 2;    // elements per wave (a multiple of 128)
  const int nit = kw >> 6;     // 64-element steps (2 .. kSharedMfmaSteps)
  const int kb0 = wave * kw + 16 * grp;
  // all of the wave's weight loads first (one memory round trip)
  uint4 c[kSharedMfmaSteps];
  u32 e[kSharedMfmaSteps];
#pragma unroll
  for (int i = 0; i < kSharedMfmaSteps; ++i) {
    if (i < nit) {  // uniform; guards, not a break, keep the indexes constant
      const int kk = kb0 + 64 * i;
      c[i] = *reinterpret_cast<const uint4*>(wr + kk);
      e[i] = sr[kk >> 5];
    }
  }
  floatx4_t acc = floatx4_t{0.f, 0.f, 0.f, 0.f};
  // x in groups of four steps, double-buffered: group g+1's loads go out
  // before group g is multiplied (a step past the last reloads the last)
  uint4 xa[2][4], xb[2][4];
  auto load_x = [&](int g, uint4(&ya)[4], uint4(&yb)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kk = kb0 + 64 * min(4 * g + i, nit - 1);
      ya[i] = ld16(xr + kk);
      yb[i] = ld16(xr + kk + 8);
    }
  };
  load_x(0, xa[0], xb[0]);
#pragma unroll
  for (int g = 0; g < kSharedMfmaSteps / 4; ++g) {
    if (4 * g < nit) {  // uniform
      if (4 * g + 4 < nit) load_x(g + 1, xa[(g + 1) & 1], xb[(g + 1) & 1]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (4 * g + i < nit) {
          uint4 lo, hi;
          e4m3x16_bf16_scaled(c[4 * g + i], e8m0_f32(e[4 * g + i]), lo, hi);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, xa[g & 1][i]),
                                                        __builtin_bit_cast(bf16x8_t, lo), acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, xb[g & 1][i]),
                                                        __builtin_bit_cast(bf16x8_t, hi), acc, 0, 0, 0);
        }
      }
    }
  }
  // D lane l: rows 4*(l/16) + r (x rows), column l%16 (weight row of the tile)
#pragma unroll
  for (int r = 0; r < 4; ++r) lds[wave * 256 + (4 * grp + r) * 16 + r16] = acc[r];
  __syncthreads();
  const int t = threadIdx.x, m = t / MC, cc = t % MC, j = j0 + cc;
  if (t < 16 * MC && m < b.m && j < b.inter) {
    float g = lds[m * 16 + cc], u = lds[m * 16 + MC + cc];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      g += lds[w * 256 + m * 16 + cc];
      u += lds[w * 256 + m * 16 + MC + cc];
    }
    const float sg_ = g / (1.f + expf(-g));
    b.h[(int64_t)m * b.ldh + j] = (u16)bf16_rne(sg_ * u);
  }
}

// Shared part's form: MFMA for 9..16 rows (measured at M = 16, N = 128,
// K = 6144, I = 768: 13.9 us against 15.8 for the VALU form; at M = 8 the
// VALU form's 768 workgroups win, 10.5 against 13.4 us, the MFMA form's 96
// eight-column tiles streaming the weights through too few CUs). The host
// sizes the grid with the same functions.
constexpr bool shared_use_mfma(int mt) { return mt >= 16; }
constexpr int shared_mfma_cols(int mt) { return 8; }
constexpr int shared_cols_per_wg(int mt) { return shared_use_mfma(mt) ? shared_mfma_cols(mt) : 4 / shared_kw(mt); }

// Router tiles first (blocks [0, router_wgs)), then ceil(I / cols) shared
// workgroups (cols = shared_cols_per_wg of the shared part's rows). KS == 0:
// VALU router tile <MT, 1, L>; else the 16-row MFMA tile with KS k-steps
// (from 5 rows at up to 128 experts, else 9..16). The shared part takes SMR
// rows if given (8: the VALU form behind an MFMA router tile at 5..8 rows),
// else MT (16 with MFMA).
// The shared part's operands lead the arguments as scalars (router_wgs, wq,
// ws, x, ldx, k, inter, m: b's), preloaded into scalar registers at dispatch
// (the unit is built with eight preloaded arguments), so its workgroups'
// first loads do not wait ~0.2 us for the argument block.
template <int MT, int L, int KS, int SMR = 0>
__global__ void __launch_bounds__(256) router_shared_kernel(int router_wgs, const uint8_t* wq, const uint8_t* ws,
                                                            const u16* x, int ldx, int k, int inter, int m,
                                                            GemvArgs a, SharedArgs bk) {
  constexpr int SM = SMR ? SMR : (KS ? 16 : MT);
  SharedArgs b = bk;
  b.wq = wq;
  b.ws = ws;
  b.x = x;
  b.ldx = ldx;
  b.k = k;
  b.inter = inter;
  b.m = m;
  __shared__ float lds[(KS || shared_use_mfma(SM)) ? 4 * 256 : 4 * 2 * SM];
  if ((int)blockIdx.x < router_wgs) {
    const int t = xcd_tile(blockIdx.x, router_wgs);
    const int nb = t % a.nb_count, s = t / a.nb_count;
    if constexpr (KS == 0)
      valu_tile<MT, 1, L>(a, nb, s, PartialSink{a.part, a.m, a.n});
    else
      mfma_tile<1, KS>(a, 0, nb, s, lds, PartialSink{a.part, a.m, a.n});
    return;
  }
  if constexpr (shared_use_mfma(SM))
    shared_swiglu_mfma<shared_mfma_cols(SM)>(b, (int)blockIdx.x - router_wgs, lds);
  else
    shared_swiglu<SM>(b, (int)blockIdx.x - router_wgs, lds);
}

}  // namespace rgt
