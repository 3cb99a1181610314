// fused.h - the whole decode front-end in one launch (M <= 64).
//
// Phases of one co-resident grid (every wait is bounded by a deadline):
//   0. each thread loads the bf16 chunk of x it will quantise (issued with the
//      W stream so the quant costs no extra round trip later);
//   1. split-K GEMV tile -> fp32 partial; arrive on the n-block counter; the
//      last workgroup to arrive sums the partials in k-slice order, writes the
//      logits, zeroes that counter and arrives on the logits counter
//      ("MiniMax-M3: Triton split-K router GEMV with in-kernel split-K fixup",
//      opening summary);
//   2. row-owner workgroups (4 rows each, one wave per row) wait for all
//      n-blocks, run the top-k gate and arrive on the gate counter;
//   3. every workgroup waits for the gate, sorts the M*k pairs in its own LDS
//      (the sort is tiny at decode sizes, so redundant sorting is cheaper than
//      another grid-wide hand-off) and stores its quantised chunks to the
//      padded positions; workgroup 0 also writes sorted_ids, expert_ids and
//      offsets;
//   4. the last workgroup to leave zeroes the phase counters.
// The pages fuse router, gate and sort into one decode launch (MiniMax-M3.1-
// Flash MoE/GEMM kernels, Summary: Router; Kimi-K3 fused routing, sort, quant,
// Motivation); this is that chain laid out for a gfx950 grid.
#pragma once

#include "device.h"
#include "gate.h"
#include "gemv.h"
#include "sortq.h"

namespace rgt {

// Control words at the head of the workspace.
enum : int { kCtlErr = 0, kCtlLogits = 1, kCtlGate = 2, kCtlExit = 3 };

struct FusedArgs {
  GemvArgs g;
  const float* bias;
  int topk, block;
  int32_t* topk_ids;
  float* topk_w;
  int32_t* sorted_ids;
  int32_t* expert_ids;
  int32_t* offsets;
  uint8_t* a_q;
  uint8_t* a_scale;
  u32* ctl;
  u64 budget;        // deadline of each wait, in 100 MHz ticks
  int fault_skip;    // host-forced fault: 1 = gate owners never arrive
};

// Bounded wait by thread 0, result shared with the workgroup; on success every
// thread performs an acquire so data published before the counter is visible.
__device__ __forceinline__ bool wg_wait_geq(u32* ctr, u32 target, const FusedArgs& a) {
  __shared__ u32 s_ok;
  if (threadIdx.x == 0) s_ok = wait_geq(ctr, target, a.budget, a.ctl + kCtlErr) ? 1u : 0u;
  __syncthreads();
  const bool ok = s_ok != 0u;
  if (ok) __threadfence();
  return ok;
}

template <int NV>
__device__ __forceinline__ void fused_tail(const FusedArgs& a, int* smem, bool have_unit, int unit,
                                           const uint4& codes_in, u32 sb_in) {
  const GemvArgs& g = a.g;
  const int m = g.m, n = g.n, k = a.topk;
  const int row_groups = (m + 3) >> 2;
  // Phase 2: top-k by the row owners.
  if ((int)blockIdx.x < row_groups) {
    if (!wg_wait_geq(a.ctl + kCtlLogits, (u32)g.nb_count, a)) return;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row < m)
      wave_topk_row<NV>(g.logits + (int64_t)row * n, a.bias, n, k, a.topk_ids + (int64_t)row * k,
                        a.topk_w + (int64_t)row * k);
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0 && !a.fault_skip) atomic_add_agent(a.ctl + kCtlGate, 1u);
  }
  // Phase 3: sort in LDS, then store the quantised chunks.
  if (!wg_wait_geq(a.ctl + kCtlGate, (u32)row_groups, a)) return;
  const int P = m * k;
  int* s_e = smem;
  int* s_pos = s_e + P;
  int* s_hist = s_pos + P;
  int* s_cnt = s_hist + 4 * n;
  int* s_off = s_cnt + n;
  int* s_scr = s_off + n + 1;
  wg_sort(a.topk_ids, P, n, a.block, s_e, s_hist, s_cnt, s_off, s_scr, s_pos);
  if (blockIdx.x == 0) {
    for (int p = threadIdx.x; p < P; p += blockDim.x)
      if (s_pos[p] >= 0) a.sorted_ids[s_pos[p]] = p;
    write_sort_layout(s_cnt, s_off, n, a.block, P, a.sorted_ids, a.expert_ids, a.offsets);
  }
  if (have_unit) {
    const int K = g.k, cpr = K >> 4;
    const int t = unit / cpr, c = unit - t * cpr;
    const int64_t kscale = K >> 5;
    for (int j = 0; j < k; ++j) {
      const int64_t d = s_pos[t * k + j];
      if (d < 0) continue;
      *reinterpret_cast<uint4*>(a.a_q + d * K + 16 * c) = codes_in;
      if ((c & 1) == 0) a.a_scale[d * kscale + (c >> 1)] = (uint8_t)sb_in;
    }
  }
  // Phase 4: the last workgroup out zeroes the phase counters.
  __syncthreads();
  if (threadIdx.x == 0) {
    if (atomic_add_agent(a.ctl + kCtlExit, 1u) == gridDim.x - 1u) {
      atomic_store_agent(a.ctl + kCtlLogits, 0u);
      atomic_store_agent(a.ctl + kCtlGate, 0u);
      atomic_store_agent(a.ctl + kCtlExit, 0u);
    }
  }
}

// Quant unit of this thread: unit = global thread id (the host guarantees
// M*K/16 <= grid*256). Codes are computed after the GEMV tile.
template <int NV, int MT, int RPW, int L>
__global__ void __launch_bounds__(256) fused_valu_kernel(FusedArgs a) {
  extern __shared__ int smem[];
  const GemvArgs& g = a.g;
  const int units = g.m * (g.k >> 4);
  const int unit = blockIdx.x * 256 + threadIdx.x;
  const bool have_unit = unit < units;
  const int nb = blockIdx.x % g.nb_count, s = blockIdx.x / g.nb_count;
  valu_tile<MT, RPW, L>(g, nb, s);
  if (arrive_last(g.ctr + nb, (u32)g.s_count)) {
    reduce_partials(g, 0, g.m, nb * 4 * RPW, 4 * RPW, g.logits);
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
      atomic_store_agent(g.ctr + nb, 0u);
      atomic_add_agent(a.ctl + kCtlLogits, 1u);
    }
  }
  u32 sb = 0;
  uint4 codes = make_uint4(0, 0, 0, 0);
  if (have_unit) {
    const int cpr = g.k >> 4, t = unit / cpr, c = unit - t * cpr;
    codes = mx_quant16(g.x + (int64_t)t * g.ldx + 16 * c, sb);
  }
  fused_tail<NV>(a, smem, have_unit, unit, codes, sb);
}

template <int NV, int MT, int KS>
__global__ void __launch_bounds__(256) fused_mfma_kernel(FusedArgs a) {
  extern __shared__ int smem[];
  const GemvArgs& g = a.g;
  const int units = g.m * (g.k >> 4);
  const int unit = blockIdx.x * 256 + threadIdx.x;
  const bool have_unit = unit < units;
  const int nb = blockIdx.x % g.nb_count, s = blockIdx.x / g.nb_count;
  mfma_tile<MT, KS>(g, 0, nb, s, reinterpret_cast<float*>(smem));
  if (arrive_last(g.ctr + nb, (u32)g.s_count)) {
    reduce_partials(g, 0, g.m, nb * 16, 16, g.logits);
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
      atomic_store_agent(g.ctr + nb, 0u);
      atomic_add_agent(a.ctl + kCtlLogits, 1u);
    }
  }
  u32 sb = 0;
  uint4 codes = make_uint4(0, 0, 0, 0);
  if (have_unit) {
    const int cpr = g.k >> 4, t = unit / cpr, c = unit - t * cpr;
    codes = mx_quant16(g.x + (int64_t)t * g.ldx + 16 * c, sb);
  }
  __syncthreads();  // the MFMA tile's LDS is reused by the sort
  fused_tail<NV>(a, smem, have_unit, unit, codes, sb);
}

}  // namespace rgt
