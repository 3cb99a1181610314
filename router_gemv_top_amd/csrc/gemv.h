// gemv.h - split-K router GEMV tiles for gfx950 and the in-launch fixup.
//
// logits[M][N] fp32 = x[M][K] bf16 . W[N][K]^T bf16 ("MiniMax-M3: Triton
// split-K router GEMV with in-kernel split-K fixup", opening summary). The
// grid is split over (row tile, n-block, k-slice). Each workgroup writes an
// fp32 partial for its tile and k-slice to the workspace and arrives on the
// tile's counter; the last workgroup to arrive sums the partials in k-slice
// order (deterministic), writes the logits and puts the counter back to zero,
// so no memset launch and no separate reduce launch is needed.
//
// Two tile kinds, chosen per M bucket (the page's per-M-bucket configs):
//   * VALU tile (M <= 8): each wave streams RPW rows of W with 16-byte loads
//     (a wave load covers 512 consecutive k of one row, fully coalesced) and
//     forms dot products with v_dot2_f32_bf16; a wave64 butterfly reduces.
//   * MFMA tile (8 < M): v_mfma_f32_16x16x32_bf16 with x as the A operand
//     (16 rows) and W as the B operand (16 experts); the four waves of a
//     workgroup split the k-slice and their 16x16 accumulators are summed in
//     wave order through LDS.
#pragma once

#include <type_traits>

#include "device.h"

namespace rgt {

typedef uint16_t u16;

struct GemvArgs {
  const u16* x;
  int64_t ldx;
  const u16* w;
  int64_t ldw;
  float* logits;   // [M][N]
  float* part;     // [S][M][N] fp32 partials (workspace)
  u32* ctr;        // [MB*NB] arrival counters, kCtrStride words apart (zero between calls)
  int m, n, k;
  int s_count;     // S: number of k-slices
  int nb_count;    // NB: number of n-blocks
};

__device__ __forceinline__ uint4 ld16(const u16* p) { return *reinterpret_cast<const uint4*>(p); }

// Receiver of a tile's partial sums: sink(s, m, c, v) gets the fp32 partial of
// row m, expert c, k-slice s. This one stores it with an agent-scope store to
// part[s][m][c] for the fixup by the last arriver.
struct PartialSink {
  float* part;
  int m, n;
  __device__ __forceinline__ void operator()(int s, int row, int col, float v) const {
    st_agent(part + ((int64_t)s * m + row) * n + col, v);
  }
};

// ---------------------------------------------------------------------------
// VALU tile. Workgroup = 4 waves; wave w owns rows n0 + w*RPW .. +RPW of the
// n-block, over the workgroup's k-slice of 512*L elements. Lane l covers the
// 8 elements at k = kslice + j*512 + 8*l for j < L.
// ---------------------------------------------------------------------------
// pre() runs once the tile's loads are issued (other loads to overlap).
struct NoPrefetch {
  __device__ __forceinline__ void operator()() const {}
};

// The tile's x as it is in memory. A transform with kOn = true instead has
// the tile load the residual and gamma chunks beside each x chunk and, after
// pre(), add the residual (residual(x, r) = h), run its row work, take its
// rows' scales (rstd_rows) and replace the chunk by apply(h, gamma, scale):
// the router behind the RMSNorm producer normalises its own columns.
struct NoNorm {
  static constexpr bool kOn = false;
  __device__ __forceinline__ uint4 res(int, int) const { return make_uint4(0, 0, 0, 0); }
  __device__ __forceinline__ uint4 gamma(int) const { return make_uint4(0, 0, 0, 0); }
  __device__ __forceinline__ void row_work() {}
  template <int R>
  __device__ __forceinline__ void rstd_rows(const int (&)[R], float (&out)[R]) {
    for (int i = 0; i < R; ++i) out[i] = 0.f;
  }
  __device__ __forceinline__ uint4 residual(uint4 x, uint4) const { return x; }
  __device__ __forceinline__ uint4 apply(uint4 x, uint4, float) const { return x; }
};

template <int MT, int RPW, int L, class Sink, class Pre = NoPrefetch, class XF = NoNorm>
__device__ __forceinline__ void valu_tile(const GemvArgs& a, int nb, int s, const Sink& sink, Pre&& pre = Pre(),
                                          XF&& xf = XF()) {
  constexpr bool kNorm = std::remove_reference_t<XF>::kOn;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nrow0 = nb * (4 * RPW) + wave * RPW;
  const int kb = s * (512 * L) + lane * 8;
  uint4 wv[RPW][L];
  auto load_w = [&]() {
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
      for (int j = 0; j < L; ++j) wv[r][j] = ld16(a.w + (int64_t)(nrow0 + r) * a.ldw + kb + j * 512);
  };
  // W first, except behind the norm: there the activation chunks go first,
  // so that (loads return in order) they can be normalised while W is still
  // on its way.
  if constexpr (!kNorm) load_w();
  // x rows past M read row M-1 (no branch between the loads, so they are all
  // in flight together); their sums are never stored.
  uint4 xv[MT][L];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int j = 0; j < L; ++j) xv[m][j] = ld16(a.x + (int64_t)min(m, a.m - 1) * a.ldx + kb + j * 512);
  [[maybe_unused]] uint4 rv[kNorm ? MT : 1][L], gv[L];
  if constexpr (kNorm) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int j = 0; j < L; ++j) rv[m][j] = xf.res(min(m, a.m - 1), kb + j * 512);
#pragma unroll
    for (int j = 0; j < L; ++j) gv[j] = xf.gamma(kb + j * 512);
    load_w();
  }
  pre();
  if constexpr (kNorm) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int j = 0; j < L; ++j) xv[m][j] = xf.residual(xv[m][j], rv[m][j]);
    xf.row_work();
    int rows[MT];
    float rs[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) rows[m] = min(m, a.m - 1);
    xf.rstd_rows(rows, rs);
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int j = 0; j < L; ++j) xv[m][j] = xf.apply(xv[m][j], gv[j], rs[m]);
  }
  float acc[RPW][MT];
#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[r][m] = 0.f;
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int j = 0; j < L; ++j)
#pragma unroll
      for (int r = 0; r < RPW; ++r) acc[r][m] = dot8_bf16(wv[r][j], xv[m][j], acc[r][m]);
#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[r][m] = wave_sum(acc[r][m]);
#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m)
      if (lane == r * MT + m && m < a.m) sink(s, m, nrow0 + r, acc[r][m]);
}

// ---------------------------------------------------------------------------
// MFMA tile. Workgroup = 4 waves over a k-slice of 4*32*KS elements and a
// tile of 16*MT rows of x by 16 experts. Wave w takes the w-th quarter of the
// slice; inside it, lane group g = lane/16 takes a contiguous run of 8*KS
// elements, and k-step j feeds elements [8j, 8j+8) of that run to the MFMA.
// (The dot product does not depend on how k is assigned to MFMA slots, as
// long as A and B use the same assignment.)
// A lane l: x[row0 + l%16][k-run of group l/16]; B lane l: W[n0 + l%16][same k].
// D lane l: rows 4*(l/16)+i (i < 4) of the 16x16 tile, column l%16.
// ---------------------------------------------------------------------------
template <int MT, int KS, class Sink, class Pre = NoPrefetch, class XF = NoNorm>
__device__ __forceinline__ void mfma_tile(const GemvArgs& a, int mb, int nb, int s, float* lds, const Sink& sink,
                                          Pre&& pre = Pre(), XF&& xf = XF()) {
  constexpr bool kNorm = std::remove_reference_t<XF>::kOn;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r16 = lane & 15, grp = lane >> 4;
  const int kslice = 4 * 32 * KS;
  const int krun = s * kslice + wave * (32 * KS) + grp * (8 * KS);
  const int n = nb * 16 + r16;
  uint4 bw[KS];
  auto load_w = [&]() {
#pragma unroll
    for (int j = 0; j < KS; ++j) bw[j] = ld16(a.w + (int64_t)n * a.ldw + krun + 8 * j);
  };
  // W first, except behind the norm (as in the VALU tile)
  if constexpr (!kNorm) load_w();
  floatx4_t acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  const int row_base = mb * (16 * MT);
  // x rows past M are loaded from row M-1 (no branch between the loads, so
  // they are all in flight together) and replaced by zeros.
  uint4 xv[MT][KS];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int m = min(row_base + t * 16 + r16, a.m - 1);
#pragma unroll
    for (int j = 0; j < KS; ++j) xv[t][j] = ld16(a.x + (int64_t)m * a.ldx + krun + 8 * j);
  }
  [[maybe_unused]] uint4 rv[kNorm ? MT : 1][KS], gv[KS];
  if constexpr (kNorm) {
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int m = min(row_base + t * 16 + r16, a.m - 1);
#pragma unroll
      for (int j = 0; j < KS; ++j) rv[t][j] = xf.res(m, krun + 8 * j);
    }
#pragma unroll
    for (int j = 0; j < KS; ++j) gv[j] = xf.gamma(krun + 8 * j);
    load_w();
  }
  pre();
  if constexpr (kNorm) {
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int j = 0; j < KS; ++j) xv[t][j] = xf.residual(xv[t][j], rv[t][j]);
    xf.row_work();
    int rows[MT];
    float rs[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) rows[t] = min(row_base + t * 16 + r16, a.m - 1);
    xf.rstd_rows(rows, rs);
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int j = 0; j < KS; ++j) xv[t][j] = xf.apply(xv[t][j], gv[j], rs[t]);
  }
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const bool ok = row_base + t * 16 + r16 < a.m;
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      const uint4 v = ok ? xv[t][j] : make_uint4(0, 0, 0, 0);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, v),
                                                      __builtin_bit_cast(bf16x8_t, bw[j]), acc[t], 0, 0, 0);
    }
  }
  // Sum the four waves' accumulators in wave order through LDS.
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) lds[((wave * MT + t) * 16 + grp * 4 + i) * 16 + r16] = acc[t][i];
  __syncthreads();
  for (int idx = threadIdx.x; idx < MT * 256; idx += 256) {
    const int t = idx >> 8, rc = idx & 255, rr = rc >> 4, cc = rc & 15;
    const int m = row_base + t * 16 + rr;
    float v = lds[((0 * MT + t) * 16 + rr) * 16 + cc];
    v += lds[((1 * MT + t) * 16 + rr) * 16 + cc];
    v += lds[((2 * MT + t) * 16 + rr) * 16 + cc];
    v += lds[((3 * MT + t) * 16 + rr) * 16 + cc];
    if (m < a.m) sink(s, m, nb * 16 + cc, v);
  }
}

// ---------------------------------------------------------------------------
// Split-K fixup. The partials were stored with agent-scope stores; the
// workgroup drains them, then one thread arrives on the tile counter. Returns
// true in the last workgroup to arrive: by then every other workgroup's
// partials are complete, and agent-scope loads read them coherently.
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool arrive_last(u32* ctr, u32 arrivals) {
  __shared__ u32 s_last;
  const u32 old = publish_arrive(ctr);
  if (threadIdx.x == 0) s_last = (old == arrivals - 1u) ? 1u : 0u;
  __syncthreads();
  return s_last != 0u;
}

// Sum the S partials of rows [r0, r1) x columns [c0, c0+bn) in k-slice order
// (s = 0, 1, ..., S-1 for every output, so every path that reduces the same
// partials gets the same bits). Each thread takes 4 neighbouring columns of one
// row and loads their partials with 16-byte coherent loads, 12 k-slices in
// flight at a time; out(m, c, sums) receives the 4 sums of columns c..c+3.
constexpr int kReduceBatch = 12;

template <class Out>
__device__ __forceinline__ void reduce_partials(const GemvArgs& a, int r0, int r1, int c0, int bn, Out out) {
  const int rows = r1 - r0, quads = bn >> 2, lq = __ffs(quads) - 1;  // quads is 1, 2 or 4
  const u32 slice = (u32)a.m * (u32)a.n * 4u;
  const auto rsrc = coherent_rsrc(a.part, slice * (u32)a.s_count);
  for (int idx = threadIdx.x; idx < rows * quads; idx += 256) {  // 256-thread workgroups
    const int m = r0 + (idx >> lq), c = c0 + 4 * (idx & (quads - 1));
    const u32 off = ((u32)m * (u32)a.n + (u32)c) * 4u;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s0 = 0; s0 < a.s_count; s0 += kReduceBatch) {
      u32x4_t v[kReduceBatch];
      // Slices past S read beyond the buffer and come back as zeros; they are
      // not added.
#pragma unroll
      for (int j = 0; j < kReduceBatch; ++j) v[j] = ld_agent16(rsrc, off + (u32)(s0 + j) * slice);
#pragma unroll
      for (int j = 0; j < kReduceBatch; ++j) {
        if (s0 + j < a.s_count) {
          acc.x += __uint_as_float(v[j].x);
          acc.y += __uint_as_float(v[j].y);
          acc.z += __uint_as_float(v[j].z);
          acc.w += __uint_as_float(v[j].w);
        }
      }
    }
    out(m, c, acc);
  }
}

// Writer of plain fp32 logits (read by later launches).
struct LogitsOut {
  float* logits;
  int n;
  __device__ __forceinline__ void operator()(int m, int c, float4 v) const {
    *reinterpret_cast<float4*>(logits + (int64_t)m * n + c) = v;
  }
};

// Standalone router kernels: tile, then fixup by the last arriver.
template <int MT, int RPW, int L>
__global__ void __launch_bounds__(256) router_valu_kernel(GemvArgs a) {
  const int t = xcd_tile(blockIdx.x, gridDim.x);
  const int nb = t % a.nb_count, s = t / a.nb_count;
  valu_tile<MT, RPW, L>(a, nb, s, PartialSink{a.part, a.m, a.n});
  u32* ctr = a.ctr + nb * kCtrStride;
  if (arrive_last(ctr, (u32)a.s_count)) {
    reduce_partials(a, 0, a.m, nb * 4 * RPW, 4 * RPW, LogitsOut{a.logits, a.n});
    if (threadIdx.x == 0) st_agent(ctr, 0u);
  }
}

template <int MT, int KS>
__global__ void __launch_bounds__(256) router_mfma_kernel(GemvArgs a) {
  __shared__ float lds[4 * MT * 256];
  const int t = xcd_tile(blockIdx.x, gridDim.x);
  // row block fastest: the row blocks of one W tile run side by side on one
  // XCD, so W streams from HBM once and the second block reads it from L2
  const int mbc = (int)gridDim.x / (a.nb_count * a.s_count);
  const int mb = t % mbc, r = t / mbc;
  const int nb = r % a.nb_count;
  const int s = r / a.nb_count;
  mfma_tile<MT, KS>(a, mb, nb, s, lds, PartialSink{a.part, a.m, a.n});
  u32* ctr = a.ctr + (mb * a.nb_count + nb) * kCtrStride;
  if (arrive_last(ctr, (u32)a.s_count)) {
    const int r0 = mb * 16 * MT;
    const int r1 = min(a.m, r0 + 16 * MT);
    reduce_partials(a, r0, r1, nb * 16, 16, LogitsOut{a.logits, a.n});
    if (threadIdx.x == 0) st_agent(ctr, 0u);
  }
}

}  // namespace rgt
