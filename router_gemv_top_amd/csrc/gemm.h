// gemm.h - router logits for large batches as an LDS-tiled MFMA GEMM.
//
// logits[M][N] fp32 = x[M][K] bf16 . W[N][K]^T bf16, the same contraction as
// the split-K GEMV ("MiniMax-M3: Triton split-K router GEMV with in-kernel
// split-K fixup", opening summary) for batches of more than 64 tokens.
// Prefill (thousands of tokens) has tiles enough for every workgroup to take
// the whole k range: no split, the dense-GEMM regime the configurations name
// for prefill routing. Wide batches (128-512 tokens) have a handful of tiles,
// so the k range is split into S slices of ksl elements and workgroup
// (slice s, tile) writes its fp32 partial to out + s*M*N; the gate of the
// next launch sums the slices in order (the gate taking the partials, as the
// MiniMax-M3.1-Flash MoE/GEMM kernels page's router does). A 128 x 128 tile
// reads each x row once per 128 experts.
//
// Workgroup tile 128 rows of x by 128 experts, k-step 64. The next k-step's
// tiles are loaded into registers while the current one is multiplied from
// LDS (one LDS buffer, two barriers per step). 4 waves in 2 x 2, each owning
// 64 x 64 outputs as 4 x 4 v_mfma_f32_16x16x32_bf16 tiles. LDS rows are 64
// bf16 plus 8 of padding (144 bytes), which spreads the 16 rows one
// ds_read_b128 touches over disjoint banks.
#pragma once

#include "device.h"

namespace rgt {

constexpr int kGemmBM = 128, kGemmBN = 128, kGemmBK = 64;
constexpr int kGemmLds = kGemmBK + 8;  // bf16 per LDS row

// Tiles (row block, expert block) are numbered row-block major, and the
// XCD-aware map gives each XCD a contiguous run of them, so the x rows a run
// shares stay in one L2.
// ksl: k elements per slice (a multiple of kGemmBK dividing K); the grid is
// (K / ksl) x tiles workgroups. PRE > 1: the slice is exactly PRE k-steps and
// all of them are loaded at once (one memory round trip for the slice instead
// of one per step: with a few k-steps per workgroup, each step's compute is
// far shorter than the latency its prefetch would have to hide).
template <int PRE>
__global__ void __launch_bounds__(256) router_gemm_kernel(const uint16_t* x, int64_t ldx, const uint16_t* w,
                                                          int64_t ldw, float* out, int M, int N, int ksl) {
  __shared__ __align__(16) uint16_t sA[kGemmBM * kGemmLds];
  __shared__ __align__(16) uint16_t sB[kGemmBN * kGemmLds];
  const int nbn = (N + kGemmBN - 1) / kGemmBN;
  const int tiles = ((M + kGemmBM - 1) / kGemmBM) * nbn;
  const int job = xcd_tile(blockIdx.x, gridDim.x);
  const int slice = job / tiles, tile = job - slice * tiles;
  const int kb = slice * ksl;
  float* logits = out + (int64_t)slice * M * N;
  const int m0 = (tile / nbn) * kGemmBM, n0 = (tile % nbn) * kGemmBN;
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int r16 = lane & 15, grp = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  // global -> register mapping: thread t moves the 16-byte column chunk t % 8
  // of rows t / 8 + 32*i (i < 4), for A and for B; rows past M or N read the
  // last row (never stored). Named registers, not arrays: the values cross
  // the loop's back edge, and an array there ends up in scratch memory.
  const int lc = t & 7, lr = t >> 3;
  const uint16_t* ga0 = x + (int64_t)min(m0 + lr, M - 1) * ldx + kb + 8 * lc;
  const uint16_t* ga1 = x + (int64_t)min(m0 + lr + 32, M - 1) * ldx + kb + 8 * lc;
  const uint16_t* ga2 = x + (int64_t)min(m0 + lr + 64, M - 1) * ldx + kb + 8 * lc;
  const uint16_t* ga3 = x + (int64_t)min(m0 + lr + 96, M - 1) * ldx + kb + 8 * lc;
  const uint16_t* gb0 = w + (int64_t)min(n0 + lr, N - 1) * ldw + kb + 8 * lc;
  const uint16_t* gb1 = w + (int64_t)min(n0 + lr + 32, N - 1) * ldw + kb + 8 * lc;
  const uint16_t* gb2 = w + (int64_t)min(n0 + lr + 64, N - 1) * ldw + kb + 8 * lc;
  const uint16_t* gb3 = w + (int64_t)min(n0 + lr + 96, N - 1) * ldw + kb + 8 * lc;
  auto ld = [](const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); };
  // one-step prefetch: the first step's loads go out before anything else
  uint4 ra0, ra1, ra2, ra3, rb0, rb1, rb2, rb3;
  if constexpr (PRE == 1) {
    ra0 = ld(ga0), ra1 = ld(ga1), ra2 = ld(ga2), ra3 = ld(ga3);
    rb0 = ld(gb0), rb1 = ld(gb1), rb2 = ld(gb2), rb3 = ld(gb3);
  }
  floatx4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  uint16_t* la = sA + lr * kGemmLds + 8 * lc;
  uint16_t* lb = sB + lr * kGemmLds + 8 * lc;
  auto stage = [&](const uint4& a0, const uint4& a1, const uint4& a2, const uint4& a3, const uint4& b0,
                   const uint4& b1, const uint4& b2, const uint4& b3) {
    *reinterpret_cast<uint4*>(la) = a0;
    *reinterpret_cast<uint4*>(la + 32 * kGemmLds) = a1;
    *reinterpret_cast<uint4*>(la + 64 * kGemmLds) = a2;
    *reinterpret_cast<uint4*>(la + 96 * kGemmLds) = a3;
    *reinterpret_cast<uint4*>(lb) = b0;
    *reinterpret_cast<uint4*>(lb + 32 * kGemmLds) = b1;
    *reinterpret_cast<uint4*>(lb + 64 * kGemmLds) = b2;
    *reinterpret_cast<uint4*>(lb + 96 * kGemmLds) = b3;
  };
  auto step = [&]() {
#pragma unroll
    for (int kk = 0; kk < kGemmBK; kk += 32) {
      uint4 fa[4], fb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        fa[i] = *reinterpret_cast<const uint4*>(sA + (wm * 64 + 16 * i + r16) * kGemmLds + kk + 8 * grp);
        fb[i] = *reinterpret_cast<const uint4*>(sB + (wn * 64 + 16 * i + r16) * kGemmLds + kk + 8 * grp);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, fa[i]),
                                                             __builtin_bit_cast(bf16x8_t, fb[j]), acc[i][j], 0, 0, 0);
    }
  };
  if constexpr (PRE > 1) {
    uint4 ra[PRE][4], rb[PRE][4];
#pragma unroll
    for (int j = 0; j < PRE; ++j) {
      ra[j][0] = ld(ga0 + kGemmBK * j);
      ra[j][1] = ld(ga1 + kGemmBK * j);
      ra[j][2] = ld(ga2 + kGemmBK * j);
      ra[j][3] = ld(ga3 + kGemmBK * j);
      rb[j][0] = ld(gb0 + kGemmBK * j);
      rb[j][1] = ld(gb1 + kGemmBK * j);
      rb[j][2] = ld(gb2 + kGemmBK * j);
      rb[j][3] = ld(gb3 + kGemmBK * j);
    }
#pragma unroll
    for (int j = 0; j < PRE; ++j) {
      if (j) __syncthreads();  // the previous step's LDS reads are done
      stage(ra[j][0], ra[j][1], ra[j][2], ra[j][3], rb[j][0], rb[j][1], rb[j][2], rb[j][3]);
      __syncthreads();
      step();
    }
  } else {
    for (int k0 = 0; k0 < ksl; k0 += kGemmBK) {
      __syncthreads();  // the previous step's LDS reads are done
      stage(ra0, ra1, ra2, ra3, rb0, rb1, rb2, rb3);
      __syncthreads();
      // prefetch the next step (the last step reloads itself: no branch)
      const int kn = min(k0 + kGemmBK, ksl - kGemmBK);
      ra0 = ld(ga0 + kn);
      ra1 = ld(ga1 + kn);
      ra2 = ld(ga2 + kn);
      ra3 = ld(ga3 + kn);
      rb0 = ld(gb0 + kn);
      rb1 = ld(gb1 + kn);
      rb2 = ld(gb2 + kn);
      rb3 = ld(gb3 + kn);
      step();
    }
  }
  // D lane l: rows 4*(l/16) + r of the 16 x 16 tile, column l % 16
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + wn * 64 + 16 * j + r16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + wm * 64 + 16 * i + 4 * grp + r;
        if (row < M && col < N) logits[(int64_t)row * N + col] = acc[i][j][r];
      }
    }
}

// ---------------------------------------------------------------------------
// Prefill GEMM (every workgroup the whole k range): workgroup tile 128 rows of
// x by 32*NJ experts (NJ = 7: 224, so N = 896 is four tiles and M = 8192
// gives 256 workgroups, one per CU), k-step 64. Eight waves, two a SIMD (so
// one wave's products run while the other waits on LDS or memory), as 4 x 2,
// each 32 rows by 16*NJ experts as 2 x NJ v_mfma_f32_16x16x32_bf16 tiles.
// Two LDS buffers and one barrier a step: the loads of steps s+1 and s+2 are
// in flight in two named register sets while step s is multiplied, and step
// s+1 goes into the other buffer (last read in step s-1, before the barrier
// that ended it). LDS rows as above (72 bf16). Tiles are numbered row-block
// major and spread over the XCDs in contiguous runs, so the n-blocks of one
// row block share x in one L2. Measured at M = 8192, N = 896, K = 3584: four
// waves of 64 x 112 took 74 us, these eight 66 us (the same bits).
// ---------------------------------------------------------------------------
template <int NJ>
constexpr int gemm_big_lds_bytes() {
  return 2 * (kGemmBM + 32 * NJ) * kGemmLds * 2;
}

template <int NJ>
__global__ void __launch_bounds__(512) router_gemm_big_kernel(const uint16_t* x, int64_t ldx, const uint16_t* w,
                                                              int64_t ldw, float* out, int M, int N, int K) {
  constexpr int BN = 32 * NJ;
  constexpr int B_LD = (BN * 8 + 511) / 512;        // 16-byte chunks of W a thread moves per step
  constexpr int BUF = (kGemmBM + BN) * kGemmLds;    // bf16 per buffer
  static_assert(kGemmBM * 8 == 2 * 512 && B_LD >= 2 && B_LD <= 4, "two x chunks, two to four W chunks a thread");
  extern __shared__ __align__(16) uint16_t smem_g[];
  const int nbn = (N + BN - 1) / BN;
  const int tiles = ((M + kGemmBM - 1) / kGemmBM) * nbn;
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  if (tile >= tiles) return;
  const int m0 = (tile / nbn) * kGemmBM, n0 = (tile % nbn) * BN;
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int r16 = lane & 15, grp = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  // global -> register -> LDS: chunk c of a step is row c / 8, 16-byte column
  // c % 8; thread t moves chunks t + 512*i. Rows past M or N read the last
  // row (never stored); W chunks past the tile (224 rows: 3.5 a thread) read
  // its last row and are not stored. Named registers, recomputed addresses:
  // arrays of them that cross the loop's back edge end up in scratch memory.
  const int lc = t & 7, lr = t >> 3;
  const int steps = K / kGemmBK;  // a multiple of 8
  auto lda = [&](int i, int k0) {
    return *reinterpret_cast<const uint4*>(x + (int64_t)min(m0 + lr + 64 * i, M - 1) * ldx + k0 + 8 * lc);
  };
  auto ldb = [&](int i, int k0) {
    return *reinterpret_cast<const uint4*>(w + (int64_t)min(n0 + min(lr + 64 * i, BN - 1), N - 1) * ldw + k0 +
                                           8 * lc);
  };
  auto sta = [&](int b, int i, const uint4& v) {
    *reinterpret_cast<uint4*>(smem_g + b * BUF + (lr + 64 * i) * kGemmLds + 8 * lc) = v;
  };
  auto stb = [&](int b, int i, const uint4& v) {
    if (lr + 64 * i < BN) *reinterpret_cast<uint4*>(smem_g + b * BUF + (kGemmBM + lr + 64 * i) * kGemmLds + 8 * lc) = v;
  };
  floatx4_t acc[2][NJ];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int b) {
    const uint16_t* sa = smem_g + b * BUF;
    const uint16_t* sb = sa + kGemmBM * kGemmLds;
#pragma unroll
    for (int kk = 0; kk < kGemmBK; kk += 32) {
      uint4 fa[2], fb[NJ];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        fa[i] = *reinterpret_cast<const uint4*>(sa + (wm * 32 + 16 * i + r16) * kGemmLds + kk + 8 * grp);
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        fb[j] = *reinterpret_cast<const uint4*>(sb + (wn * 16 * NJ + 16 * j + r16) * kGemmLds + kk + 8 * grp);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, fa[i]),
                                                             __builtin_bit_cast(bf16x8_t, fb[j]), acc[i][j], 0, 0, 0);
    }
  };
  // past the last step the loads repeat it and the stage fills a buffer
  // nobody reads (no branch, so the compiler counts the loads in flight)
#define RGT_GEMM_REGS(P) uint4 P##a0, P##a1, P##b0, P##b1, P##b2, P##b3;
#define RGT_GEMM_LOAD(P, st)                                                                        \
  {                                                                                                 \
    const int k0 = min(st, steps - 1) * kGemmBK;                                                   \
    P##a0 = lda(0, k0), P##a1 = lda(1, k0), P##b0 = ldb(0, k0), P##b1 = ldb(1, k0);                \
    if constexpr (B_LD > 2) P##b2 = ldb(2, k0);                                                     \
    if constexpr (B_LD > 3) P##b3 = ldb(3, k0);                                                     \
  }
#define RGT_GEMM_STAGE(P, b)                                                                        \
  sta(b, 0, P##a0), sta(b, 1, P##a1), stb(b, 0, P##b0), stb(b, 1, P##b1);                           \
  if constexpr (B_LD > 2) stb(b, 2, P##b2);                                                         \
  if constexpr (B_LD > 3) stb(b, 3, P##b3);
  RGT_GEMM_REGS(p_)
  RGT_GEMM_REGS(q_)
  RGT_GEMM_LOAD(p_, 0)
  RGT_GEMM_LOAD(q_, 1)
  RGT_GEMM_STAGE(p_, 0)
  __syncthreads();
  for (int s = 0; s < steps; s += 2) {
    RGT_GEMM_LOAD(p_, s + 2)
    compute(0);
    RGT_GEMM_STAGE(q_, 1)
    __syncthreads();
    RGT_GEMM_LOAD(q_, s + 3)
    compute(1);
    RGT_GEMM_STAGE(p_, 0)
    __syncthreads();
  }
#undef RGT_GEMM_REGS
#undef RGT_GEMM_LOAD
#undef RGT_GEMM_STAGE
  // D lane l: rows 4*(l/16) + r of the 16 x 16 tile, column l % 16
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int col = n0 + wn * 16 * NJ + 16 * j + r16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + wm * 32 + 16 * i + 4 * grp + r;
        if (row < M && col < N) out[(int64_t)row * N + col] = acc[i][j][r];
      }
    }
}

// logits = the k-slice partials part[S][count] summed in slice order, one
// fp32 add per slice (the order of the gate that takes the partials, so the
// two give the same bits). Four consecutive values per thread (count is a
// multiple of 4; part is 16-byte aligned, out only 4-byte aligned), slices
// loaded eight at a time so their latencies overlap.
__global__ void __launch_bounds__(256) sum_partials_kernel(const float* part, int S, int64_t count, float* out) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= count) return;
  float4 acc = *reinterpret_cast<const float4*>(part + i);
  for (int s0 = 1; s0 < S; s0 += 8) {
    float4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = *reinterpret_cast<const float4*>(part + (int64_t)min(s0 + j, S - 1) * count + i);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (s0 + j < S) {
        acc.x = __fadd_rn(acc.x, v[j].x);
        acc.y = __fadd_rn(acc.y, v[j].y);
        acc.z = __fadd_rn(acc.z, v[j].z);
        acc.w = __fadd_rn(acc.w, v[j].w);
      }
  }
  out[i] = acc.x;
  out[i + 1] = acc.y;
  out[i + 2] = acc.z;
  out[i + 3] = acc.w;
}

}  // namespace rgt
