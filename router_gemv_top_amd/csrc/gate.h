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
// Lane l holds the scores of experts l, l+64, l+128, ... as order-preserving
// u32 keys. Each of the k rounds takes the wave maximum of the keys and the
// lowest expert index holding it (ballots over the lane's slots in expert
// order), then clears that key.
#pragma once

#include "device.h"

namespace rgt {

// Add the optional bias to a row held in registers: sv[i] is the score of
// expert lane + 64*i.
template <int NV>
__device__ __forceinline__ void add_bias(float (&sv)[NV], const float* bias, int n) {
  if (!bias) return;
  const int lane = lane_id();
  float bv[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) bv[i] = bias[min(lane + 64 * i, n - 1)];
#pragma unroll
  for (int i = 0; i < NV; ++i) sv[i] = __fadd_rn(sv[i], bv[i]);
}

// Top-k of one row of scores held in registers (sv[i]: expert lane + 64*i,
// valid below n). Lane j < k ends with the j-th expert in my_id and its
// renormalised weight in my_w.
template <int NV>
__device__ __forceinline__ void wave_topk_regs(const float (&sv)[NV], int n, int k, int& my_id, float& my_w) {
  const int lane = lane_id();
  u32 key[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) key[i] = lane + 64 * i < n ? score_key(sv[i]) : 0u;
  // Each lane keeps its best key and the lowest slot holding it; a round
  // takes the wave maximum, finds the owning lane (the lowest expert index on
  // ties across lanes), and only that lane drops the key and rescans.
  u32 best;
  int bslot;
  auto rescan = [&]() {
    best = key[0];
    bslot = 0;
#pragma unroll
    for (int i = 1; i < NV; ++i)
      if (key[i] > best) {  // strict: the lowest slot wins ties inside a lane
        best = key[i];
        bslot = i;
      }
  };
  rescan();
  my_id = 0;
  float my_s = 0.f;
  for (int j = 0; j < k; ++j) {
    const u32 top = wave_max_u32(best);
    const u64 owners = ballot64(best == top);
    int win;
    if (__popcll(owners) == 1) {
      const int wl = (int)__builtin_ctzll(owners);
      win = 64 * __builtin_amdgcn_readlane(bslot, wl) + wl;
    } else {
      // equal maxima in several lanes: the lowest expert index among them
      const u32 cand = best == top ? (u32)(64 * bslot + lane) : 0xffffffffu;
      win = (int)~wave_max_u32(~cand);
    }
    if (lane == (win & 63)) {
#pragma unroll
      for (int i = 0; i < NV; ++i)
        if (i == (win >> 6)) key[i] = 0u;
      rescan();
    }
    if (lane == j) {
      my_id = win;
      my_s = key_score(top);
    }
  }
  // Renormalised softmax over the k selected scores, slot 0 the largest.
  const double s0 = (double)readlane_f32(my_s, 0);
  double e = 0.0;
  if (lane < k) e = exp64_recipe((double)my_s - s0);
  double total = readlane_f64(e, 0);
#pragma unroll
  for (int j = 1; j < 32; ++j)
    if (j < k) total = total + readlane_f64(e, j);
  my_w = lane < k ? (float)(e / total) : 0.f;
}

// Load a row of logits (all loads issued before any is used: addresses are
// clamped into the row and there are no branches between them), add the bias
// and run the top-k; lanes j < k write slot j.
template <int NV>
__device__ __forceinline__ void wave_topk_row(const float* logits_row, const float* bias, int n, int k,
                                              int32_t* ids_out, float* w_out) {
  const int lane = lane_id();
  float sv[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) sv[i] = logits_row[min(lane + 64 * i, n - 1)];
  add_bias<NV>(sv, bias, n);
  int id;
  float w;
  wave_topk_regs<NV>(sv, n, k, id, w);
  if (lane < k) {
    ids_out[lane] = id;
    w_out[lane] = w;
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
