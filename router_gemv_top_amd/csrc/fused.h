// fused.h - the whole decode front-end in one launch (M <= 64).
//
// The pages run the router, the gate and the sort of a decode step as one
// launch (MiniMax-M3.1-Flash MoE/GEMM kernels, Summary: Router; Kimi-K3 fused
// routing, sort, quant, Motivation). On gfx950 each hand-off between
// workgroups costs a device-coherent memory round trip (about a microsecond),
// so the chain below is laid out to have as few of them as possible:
//
//   1. every workgroup computes one split-K GEMV tile and stores its fp32
//      partial; the last workgroup to arrive at the n-block's counter sums
//      the partials in k-slice order and zeroes the counter ("MiniMax-M3:
//      Triton split-K router GEMV with in-kernel split-K fixup", opening
//      summary), then publishes the n-block's logits as tagged words;
//   2. row-owner workgroups (one wave per token row) poll their row's tagged
//      logits, run the softmax top-k gate and publish the row's expert ids as
//      tagged words;
//   3. workgroup 0 and every workgroup that owns a quant chunk poll the tagged
//      ids, sort the M*k pairs in LDS with one wave (tiny at decode sizes, so
//      redundant sorting beats another hand-off) and store their MXFP8 chunk
//      (quantised in registers while waiting) to the padded rows of the
//      token's pairs; workgroup 0 also writes sorted_ids, expert_ids and
//      offsets and advances the call epoch.
//
// A tagged word is a 32-bit payload plus the tag (epoch + 1) of the call that
// wrote it, stored as one 8-byte atomic; readers poll the words themselves, so
// these hand-offs need no counter. The epoch is read by every workgroup at
// start and advanced by workgroup 0 only after every id is in, which implies
// every workgroup has arrived in step 1, hence has read it. Every wait is
// bounded by a deadline that sets the workspace error word.
#pragma once

#include "device.h"
#include "gate.h"
#include "gemv.h"
#include "sortq.h"

namespace rgt {

// Control words at the head of the workspace, 128 bytes apart.
enum : int { kCtlErr = 0, kCtlEpoch = kCtrStride };

struct FusedArgs {
  GemvArgs g;          // g.logits unused here
  const float* bias;   // [N] or null
  int topk, block;
  float* logits_out;   // [M][N] or null
  int32_t* topk_ids;
  float* topk_w;
  int32_t* sorted_ids;
  int32_t* expert_ids;
  int32_t* offsets;
  uint8_t* a_q;
  uint8_t* a_scale;
  u32* ctl;
  u64* tlogits;        // [M][N] tagged logits (workspace)
  u64* tids;           // [M*topk] tagged expert ids (workspace)
  u64 budget;          // deadline of each wait, in 100 MHz ticks
  int fault_skip;      // host-forced fault: 1 = row owners never publish ids
  u64* trace;          // phase stamps (trace build only), 16 per workgroup
};

// Writer of the finisher's sums: optional plain logits, and tagged logits.
struct TaggedLogitsOut {
  float* logits_out;
  u64* tlogits;
  int n;
  u32 tag;
  __device__ __forceinline__ void operator()(int m, int c, float4 v) const {
    if (logits_out) *reinterpret_cast<float4*>(logits_out + (int64_t)m * n + c) = v;
    u64* t = tlogits + (int64_t)m * n + c;
    st_agent(t + 0, tag_word(__float_as_uint(v.x), tag));
    st_agent(t + 1, tag_word(__float_as_uint(v.y), tag));
    st_agent(t + 2, tag_word(__float_as_uint(v.z), tag));
    st_agent(t + 3, tag_word(__float_as_uint(v.w), tag));
  }
};

__device__ __forceinline__ void set_timeout(const FusedArgs& a) { or_agent(a.ctl + kCtlErr, kErrTimeout); }

// One wave polls its row of tagged logits until every word carries `tag`.
template <int NV>
__device__ __forceinline__ bool poll_row(const u64* trow, int n, u32 tag, const FusedArgs& a, float (&sv)[NV]) {
  const int lane = lane_id();
  const u64 t0 = rt_clock();
  for (;;) {
    u64 w[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) w[i] = ld_agent(trow + min(lane + 64 * i, n - 1));
    bool ok = true;
#pragma unroll
    for (int i = 0; i < NV; ++i) ok = ok && tag_ok(w[i], tag);
    if (__all(ok)) {
#pragma unroll
      for (int i = 0; i < NV; ++i) sv[i] = __uint_as_float((u32)w[i]);
      return true;
    }
    if (rt_clock() - t0 > a.budget) {
      if (lane == 0) set_timeout(a);
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// The workgroup polls all P tagged ids until every word carries `tag`, then
// leaves the experts in s_e.
__device__ __forceinline__ bool poll_ids(const u64* tids, int P, u32 tag, const FusedArgs& a, int* s_e) {
  __shared__ u32 s_late;
  constexpr int kPer = 8;  // words per thread per pass (P <= 2048)
  const u64 t0 = rt_clock();
  for (;;) {
    u64 w[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) w[j] = ld_agent(tids + min((int)threadIdx.x + 256 * j, P - 1));
    bool ok = true;
#pragma unroll
    for (int j = 0; j < kPer; ++j) ok = ok && tag_ok(w[j], tag);
    if (__syncthreads_and(ok)) {
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int p = threadIdx.x + 256 * j;
        if (p < P) s_e[p] = (int)(u32)w[j];
      }
      __syncthreads();
      return true;
    }
    if (threadIdx.x == 0) s_late = rt_clock() - t0 > a.budget ? 1u : 0u;
    __syncthreads();
    if (s_late) {
      if (threadIdx.x == 0) set_timeout(a);
      return false;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

template <int NV>
__device__ __forceinline__ void fused_tail(const FusedArgs& a, int* smem, u32 tag, bool have_unit, int unit,
                                           const uint4& codes_in, u32 sb_in) {
  const GemvArgs& g = a.g;
  const int m = g.m, n = g.n, k = a.topk;
  const int lane = threadIdx.x & 63;
  const int row_groups = (m + 3) >> 2;
  // Step 2: top-k by the row owners, one wave per token row.
  if ((int)blockIdx.x < row_groups) {
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row < m) {
      float sv[NV];
      if (poll_row<NV>(a.tlogits + (int64_t)row * n, n, tag, a, sv)) {
        RGT_STAMP(a.trace, 5);
        add_bias<NV>(sv, a.bias, n);
        int id;
        float w;
        wave_topk_regs<NV>(sv, n, k, id, w);
        if (lane < k) {
          a.topk_ids[(int64_t)row * k + lane] = id;
          a.topk_w[(int64_t)row * k + lane] = w;
          if (!a.fault_skip) st_agent(a.tids + (int64_t)row * k + lane, tag_word((u32)id, tag));
        }
        RGT_STAMP(a.trace, 6);
      }
    }
  }
  // Step 3: workgroup 0 and the quant owners wait for every id.
  const int units = m * (g.k >> 4);
  if (blockIdx.x != 0 && (int)blockIdx.x * 256 >= units) return;
  const int P = m * k;
  int* s_e = smem;
  int* s_rank = s_e + P;
  int* s_pos = s_rank + P;
  int* s_cnt = s_pos + P;
  int* s_off = s_cnt + n;
  if (!poll_ids(a.tids, P, tag, a, s_e)) return;
  RGT_STAMP(a.trace, 7);
  // Every workgroup has read the epoch (all ids are in, so every workgroup
  // arrived in step 1): advance it for the next call.
  if (blockIdx.x == 0 && threadIdx.x == 0) st_agent(a.ctl + kCtlEpoch, tag);
  if (threadIdx.x < 64) wave_sort((const int32_t*)nullptr, P, n, a.block, s_e, s_rank, s_cnt, s_off, s_pos);
  __syncthreads();
  RGT_STAMP(a.trace, 8);
  if (blockIdx.x == 0) {
    for (int p = threadIdx.x; p < P; p += blockDim.x)
      if (s_pos[p] >= 0) a.sorted_ids[s_pos[p]] = p;
    write_sort_layout(s_cnt, s_off, n, a.block, P, a.sorted_ids, a.expert_ids, a.offsets);
  }
  const u32 scales4 = pack_scales(sb_in);  // all lanes: DPP reads neighbouring lanes
  if (have_unit) store_unit(a.a_q, a.a_scale, g.k, k, unit, s_pos, codes_in, scales4);
  RGT_STAMP(a.trace, 9);
}

// Shared head of both kernels: read the epoch, run the tile, fix up, quantise.
// tile(nb, s) computes this workgroup's GEMV tile; bn is experts per n-block.
template <int NV, class Tile>
__device__ __forceinline__ void fused_body(const FusedArgs& a, int* smem, int bn, Tile tile) {
  __shared__ u32 s_tag;
  const GemvArgs& g = a.g;
  const int units = g.m * (g.k >> 4);
  const int unit = blockIdx.x * 256 + threadIdx.x;
  const bool have_unit = unit < units;
  const int tile_id = xcd_tile(blockIdx.x, gridDim.x);
  const int nb = tile_id % g.nb_count;
  RGT_STAMP(a.trace, 0);
  // The epoch load completes before this workgroup's arrival (the arrival
  // drains every outstanding memory operation first).
  if (threadIdx.x == 0) {
    const u32 t = ld_agent(a.ctl + kCtlEpoch) + 1u;
    s_tag = t ? t : 1u;  // tag 0 is never used, so zero-filled words never look ready
  }
  tile(nb, tile_id / g.nb_count);
  RGT_STAMP(a.trace, 1);
  u32* tile_ctr = g.ctr + nb * kCtrStride;
  const bool last = arrive_last(tile_ctr, (u32)g.s_count);  // has barriers: s_tag is visible after it
  const u32 tag = s_tag;
  if (last) {
    RGT_STAMP(a.trace, 2);
    reduce_partials(g, 0, g.m, nb * bn, bn, TaggedLogitsOut{a.logits_out, a.tlogits, g.n, tag});
    if (threadIdx.x == 0) st_agent(tile_ctr, 0u);
    RGT_STAMP(a.trace, 3);
  }
  u32 sb = 0;
  uint4 codes = make_uint4(0, 0, 0, 0);
  if (have_unit) {
    const int cpr = g.k >> 4, t = unit / cpr, c = unit - t * cpr;
    codes = mx_quant16(g.x + (int64_t)t * g.ldx + 16 * c, sb);
  }
  __syncthreads();  // the tile's LDS is reused below
  fused_tail<NV>(a, smem, tag, have_unit, unit, codes, sb);
}

// Quant unit of a thread: unit = global thread id (the host guarantees
// M*K/16 <= grid*256).
template <int NV, int MT, int RPW, int L>
__global__ void __launch_bounds__(256) fused_valu_kernel(FusedArgs a) {
  extern __shared__ int smem[];
  fused_body<NV>(a, smem, 4 * RPW, [&](int nb, int s) { valu_tile<MT, RPW, L>(a.g, nb, s); });
}

template <int NV, int MT, int KS>
__global__ void __launch_bounds__(256) fused_mfma_kernel(FusedArgs a) {
  extern __shared__ int smem[];
  fused_body<NV>(a, smem, 16,
                 [&](int nb, int s) { mfma_tile<MT, KS>(a.g, 0, nb, s, reinterpret_cast<float*>(smem)); });
}

}  // namespace rgt
