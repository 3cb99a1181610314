// gate.h - softmax top-k gate, one wave64 per token row.
//
// The gate of the MiniMax-M3.1-Flash MoE/GEMM kernels page (sglang PR #46691,
// Summary: Router) and the routing step of "Kimi-K3: fused MoE routing, sort,
// quant and epilogue" (sglang PR #46652, Modifications): choose the k experts
// with the largest scores and renormalise their softmax weights.
//
//   s[n]  = fp32(logits[n] + bias[n])      (bias optional)
//   ids   = top k of s by (s descending, n ascending), -0 == +0
//   w_j   = exp(s_j - s_0) / sum_{i<k} exp(s_i - s_0)     (fp64, then fp32)
//
// Lane l holds the scores of experts l*NV .. l*NV + NV - 1 (lane-major) as
// order-preserving u32 keys and keeps its best key and the lowest slot
// holding it. Each of the k rounds takes the wave maximum; the lowest lane
// holding it, at its lowest such slot, is the lowest expert index with that
// score, so one ballot and one find-first-set name the winner. Only the
// winner's key is cleared; every lane rescans its slots (no branches).
#pragma once

#include "device.h"

namespace rgt {

// Scores of one row, lane-major: sv[i] is expert lane*NV + i (valid below n).
// The optional bias is added in fp32.
template <int NV>
__device__ __forceinline__ void add_bias(float (&sv)[NV], const float* bias, int n) {
  if (!bias) return;
  const int c0 = lane_id() * NV;
  float bv[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) bv[i] = bias[min(c0 + i, n - 1)];
#pragma unroll
  for (int i = 0; i < NV; ++i) sv[i] = __fadd_rn(sv[i], bv[i]);
}

// Sum of lanes 0..S-1 in lane order as one fixed chain of fp64 adds (lanes at
// or past k hold +0, which leaves the sum unchanged), with no branches.
template <int S>
__device__ __forceinline__ double slot_sum(double e) {
  double total = readlane_f64(e, 0);
#pragma unroll
  for (int j = 1; j < S; ++j) total = total + readlane_f64(e, j);
  return total;
}

// Top-k of one row of scores held in registers (lane-major, valid below n).
// Lane j < k ends with the j-th expert in my_id and its renormalised weight
// in my_w.
template <int NV>
__device__ __forceinline__ void wave_topk_regs(const float (&sv)[NV], int n, int k, int& my_id, float& my_w) {
  const int lane = lane_id();
  u32 key[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) key[i] = lane * NV + i < n ? score_key(sv[i]) : 0u;
  u32 best;
  int bslot;
  auto rescan = [&]() {
    best = key[0];
    bslot = 0;
#pragma unroll
    for (int i = 1; i < NV; ++i) {
      const bool gt = key[i] > best;  // strict: the lowest slot wins ties inside a lane
      best = gt ? key[i] : best;
      bslot = gt ? i : bslot;
    }
  };
  rescan();
  my_id = 0;
  u32 my_key = 0u;
  for (int j = 0; j < k; ++j) {
    const u32 top = wave_max_u32(best);
    const int wl = (int)__builtin_ctzll(ballot64(best == top));
    const int ws = __builtin_amdgcn_readlane(bslot, wl);
    const bool mine = lane == wl;
#pragma unroll
    for (int i = 0; i < NV; ++i) key[i] = (mine && i == ws) ? 0u : key[i];
    rescan();
    if (lane == j) {
      my_id = wl * NV + ws;
      my_key = top;
    }
  }
  // Renormalised softmax over the k selected scores, slot 0 the largest.
  const float my_s = key_score(my_key);
  const double s0 = (double)readlane_f32(my_s, 0);
  double e = 0.0;
  if (lane < k) e = exp64_recipe((double)my_s - s0);
  const double total = k <= 8 ? slot_sum<8>(e) : (k <= 16 ? slot_sum<16>(e) : slot_sum<32>(e));
  my_w = lane < k ? (float)(e / total) : 0.f;
}

// Load a row of logits lane-major (all loads issued before any is used:
// addresses are clamped into the row), add the bias and run the top-k; lanes
// j < k write slot j.
template <int NV>
__device__ __forceinline__ void wave_topk_row(const float* logits_row, const float* bias, int n, int k,
                                              int32_t* ids_out, float* w_out) {
  const int c0 = lane_id() * NV;
  float sv[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) sv[i] = logits_row[min(c0 + i, n - 1)];
  add_bias<NV>(sv, bias, n);
  int id;
  float w;
  wave_topk_regs<NV>(sv, n, k, id, w);
  if (lane_id() < k) {
    ids_out[lane_id()] = id;
    w_out[lane_id()] = w;
  }
}

template <int NV>
__global__ void __launch_bounds__(256) topk_gate_kernel(const float* logits, const float* bias, int m, int n, int k,
                                                        int32_t* ids, float* w) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= m) return;
  wave_topk_row<NV>(logits + (int64_t)row * n, bias, n, k, ids + (int64_t)row * k, w + (int64_t)row * k);
}

}  // namespace rgt
