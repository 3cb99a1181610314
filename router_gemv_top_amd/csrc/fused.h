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
//   2. the softmax top-k gate. Small M (each wave's rows fit in registers):
//      workgroup 0 and every workgroup that owns a quant chunk poll the
//      tagged logits and run the gate for every row themselves, so no further
//      hand-off is needed. Larger M: row-owner workgroups (one wave per row)
//      run it and publish the ids as tagged words, which the others poll;
//   3. the same workgroups sort the M*k pairs in LDS with one wave (tiny at
//      decode sizes, so redundant sorting beats another hand-off) and store
//      their MXFP8 chunk (quantised in registers while waiting) to the padded
//      rows of the token's pairs; workgroup 0 also writes topk_ids, topk_w,
//      sorted_ids, expert_ids and offsets and advances the call epoch.
//
// A tagged word is a 32-bit payload plus the tag (epoch + 1) of the call that
// wrote it, stored as one 8-byte atomic; readers poll the words themselves, so
// these hand-offs need no counter. The epoch is read by every workgroup at
// start and advanced by workgroup 0 only after all logits are in, which
// implies every workgroup has arrived in step 1, hence has read it. Every wait is
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
  int fault_skip;      // host-forced fault: 1 = the fixup never publishes logits
  u64* trace;          // phase stamps (trace build only), 16 per workgroup
};

// Writer of the finisher's sums: optional plain logits, and tagged logits.
struct TaggedLogitsOut {
  float* logits_out;
  u64* tlogits;
  int n;
  u32 tag;
  int skip;  // host-forced fault: publish nothing, so every reader's wait expires
  __device__ __forceinline__ void operator()(int m, int c, float4 v) const {
    if (logits_out) *reinterpret_cast<float4*>(logits_out + (int64_t)m * n + c) = v;
    if (skip) return;
    u64* t = tlogits + (int64_t)m * n + c;
    st_agent(t + 0, tag_word(__float_as_uint(v.x), tag));
    st_agent(t + 1, tag_word(__float_as_uint(v.y), tag));
    st_agent(t + 2, tag_word(__float_as_uint(v.z), tag));
    st_agent(t + 3, tag_word(__float_as_uint(v.w), tag));
  }
};

__device__ __forceinline__ void set_timeout(const FusedArgs& a) { or_agent(a.ctl + kCtlErr, kErrTimeout); }

// Rows of tagged logits one wave holds at once (register budget: 8 score
// slots per lane).
template <int NV>
struct RowsHeld {
  static constexpr int value = NV >= 8 ? 1 : 8 / NV;
};

// Small mode: every participating workgroup runs the gate for every row
// itself (no ids hand-off), possible while each wave's rows fit in registers.
template <int NV>
__host__ __device__ constexpr bool small_mode(int m) {
  return (m + 3) / 4 <= RowsHeld<NV>::value;
}

// One wave polls `cnt` rows of tagged logits (rows r0, r0 + 4, ...) until
// every word carries `tag`. Two polls are kept in flight, so a hand-off is
// seen about one memory round trip after it lands.
template <int NV, int R>
__device__ __forceinline__ bool poll_rows(const u64* tlog, int n, int r0, int cnt, u32 tag, const FusedArgs& a,
                                          float (&sv)[R][NV]) {
  const int lane = lane_id();
  auto issue = [&](u64 (&w)[R][NV]) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int row = r < cnt ? r0 + 4 * r : r0;
        w[r][i] = ld_agent(tlog + (int64_t)row * n + min(lane + 64 * i, n - 1));
      }
  };
  auto ready = [&](const u64 (&w)[R][NV]) {
    bool ok = true;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int i = 0; i < NV; ++i) ok = ok && tag_ok(w[r][i], tag);
    return __all(ok);
  };
  auto take = [&](const u64 (&w)[R][NV]) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int i = 0; i < NV; ++i) sv[r][i] = __uint_as_float((u32)w[r][i]);
  };
  const u64 t0 = rt_clock();
  u64 wa[R][NV], wb[R][NV];
  issue(wa);
  issue(wb);
  for (;;) {
    if (ready(wa)) { take(wa); return true; }
    issue(wa);
    if (ready(wb)) { take(wb); return true; }
    issue(wb);
    if (rt_clock() - t0 > a.budget) {
      if (lane == 0) set_timeout(a);
      return false;
    }
  }
}

// The workgroup polls all P tagged ids until every word carries `tag`, then
// leaves the experts in s_e. Two polls in flight, as above.
__device__ __forceinline__ bool poll_ids(const u64* tids, int P, u32 tag, const FusedArgs& a, int* s_e) {
  __shared__ u32 s_late;
  constexpr int kPer = 8;  // words per thread per pass (P <= 2048)
  auto issue = [&](u64 (&w)[kPer]) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) w[j] = ld_agent(tids + min((int)threadIdx.x + 256 * j, P - 1));
  };
  auto ready = [&](const u64 (&w)[kPer]) {
    bool ok = true;
#pragma unroll
    for (int j = 0; j < kPer; ++j) ok = ok && tag_ok(w[j], tag);
    return __syncthreads_and(ok) != 0;
  };
  auto take = [&](const u64 (&w)[kPer]) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int p = threadIdx.x + 256 * j;
      if (p < P) s_e[p] = (int)(u32)w[j];
    }
    __syncthreads();
  };
  const u64 t0 = rt_clock();
  u64 wa[kPer], wb[kPer];
  issue(wa);
  issue(wb);
  for (;;) {
    if (ready(wa)) { take(wa); return true; }
    issue(wa);
    if (ready(wb)) { take(wb); return true; }
    issue(wb);
    if (threadIdx.x == 0) s_late = rt_clock() - t0 > a.budget ? 1u : 0u;
    __syncthreads();
    if (s_late) {
      if (threadIdx.x == 0) set_timeout(a);
      return false;
    }
  }
}

template <int NV>
__device__ __forceinline__ void fused_tail(const FusedArgs& a, int* smem, u32 tag, bool have_unit, int unit,
                                           const uint4& codes_in, u32 sb_in) {
  __shared__ u32 s_fail;
  const GemvArgs& g = a.g;
  const int m = g.m, n = g.n, k = a.topk;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int units = m * (g.k >> 4);
  const bool participant = blockIdx.x == 0 || (int)blockIdx.x * 256 < units;
  const int P = m * k;
  int* s_e = smem;
  int* s_rank = s_e + P;
  int* s_pos = s_rank + P;
  int* s_cnt = s_pos + P;
  int* s_off = s_cnt + n;
  if (small_mode<NV>(m)) {
    // Step 2 (small): each participant runs the gate for every row; wave w
    // takes rows w, w + 4, ... straight from the tagged logits.
    if (!participant) return;
    if (threadIdx.x == 0) s_fail = 0u;
    __syncthreads();
    constexpr int R = RowsHeld<NV>::value;
    const int cnt = wave < m ? (m - 1 - wave) / 4 + 1 : 0;
    if (cnt > 0) {
      float sv[R][NV];
      if (poll_rows<NV, R>(a.tlogits, n, wave, cnt, tag, a, sv)) {
        RGT_STAMP(a.trace, 5);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          if (r < cnt) {
            const int row = wave + 4 * r;
            add_bias<NV>(sv[r], a.bias, n);
            int id;
            float w;
            wave_topk_regs<NV>(sv[r], n, k, id, w);
            if (lane < k) {
              s_e[row * k + lane] = id;
              if (blockIdx.x == 0) {
                a.topk_ids[(int64_t)row * k + lane] = id;
                a.topk_w[(int64_t)row * k + lane] = w;
              }
            }
          }
        }
        RGT_STAMP(a.trace, 6);
      } else if (lane == 0) {
        s_fail = 1u;
      }
    }
    __syncthreads();
    if (s_fail) return;
  } else {
    // Step 2 (large): row owners, one wave per row, publish tagged ids.
    const int row_groups = (m + 3) >> 2;
    if ((int)blockIdx.x < row_groups) {
      const int row = blockIdx.x * 4 + wave;
      if (row < m) {
        float sv[1][NV];
        if (poll_rows<NV, 1>(a.tlogits, n, row, 1, tag, a, sv)) {
          RGT_STAMP(a.trace, 5);
          add_bias<NV>(sv[0], a.bias, n);
          int id;
          float w;
          wave_topk_regs<NV>(sv[0], n, k, id, w);
          if (lane < k) {
            a.topk_ids[(int64_t)row * k + lane] = id;
            a.topk_w[(int64_t)row * k + lane] = w;
            st_agent(a.tids + (int64_t)row * k + lane, tag_word((u32)id, tag));
          }
          RGT_STAMP(a.trace, 6);
        }
      }
    }
    if (!participant) return;
    if (!poll_ids(a.tids, P, tag, a, s_e)) return;
  }
  RGT_STAMP(a.trace, 7);
  // Every workgroup has read the epoch (all logits are in, so every
  // workgroup arrived in step 1): advance it for the next call.
  if (blockIdx.x == 0 && threadIdx.x == 0) st_agent(a.ctl + kCtlEpoch, tag);
  // Step 3: one wave sorts the pairs in LDS; the workgroup stores its
  // quantised chunk to the padded rows of the token's pairs.
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
    reduce_partials(g, 0, g.m, nb * bn, bn, TaggedLogitsOut{a.logits_out, a.tlogits, g.n, tag, a.fault_skip});
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
