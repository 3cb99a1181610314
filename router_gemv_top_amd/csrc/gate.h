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
// winner's key is cleared; every lane rescans its slots (no branches). That
// exact selection is the fallback of the faster ones below (a threshold
// bisection for up to four keys a lane, pruning to the keys that reach the
// k-th largest lane maximum above), which give the same ids in the same order.
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

// Exact selection: k rounds; in each, the wave maximum of the lanes' best
// keys, the lowest lane holding it (ballot, find-first-set) and its slot.
// The winner clears that key and every lane rescans. Lane j < k ends with the
// j-th key and expert.
template <int NV>
__device__ __forceinline__ void select_exact(u32 (&key)[NV], int k, u32& my_key, int& my_id) {
  const int lane = lane_id();
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
}

// Fast selection for two keys per lane. Each lane orders its pair once; a
// round is then only the wave maximum of the lanes' first keys and a shift in
// the lane(s) holding it, with the round's key kept in lane j. The experts
// are found afterwards: an element with key v is selected when v >= the k-th
// key, and its slot is the number of selected keys above v; it writes its
// expert to s_slot[slot] (this wave's LDS) for lane slot to read. This needs
// the k selected keys to be distinct and held by exactly k elements; when
// they are not (exact ties), true is returned and the caller runs the exact
// selection instead.
template <int R>
__device__ __forceinline__ void select_fast2(const u32 (&key)[R][2], int k, u32 (&my_key)[R], int (&my_id)[R],
                                             bool (&retry)[R], int* s_slot) {
  const int lane = lane_id();
  u32 b1[R], b2[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const bool sw = key[r][1] > key[r][0];
    b1[r] = sw ? key[r][1] : key[r][0];
    b2[r] = sw ? key[r][0] : key[r][1];
  }
  // R independent rows advance together, so their reductions interleave.
  for (int j = 0; j < k; ++j) {
    u32 top[R];
#pragma unroll
    for (int r = 0; r < R; ++r) top[r] = wave_max_u32(b1[r]);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const bool hit = b1[r] == top[r];
      b1[r] = hit ? b2[r] : b1[r];
      b2[r] = hit ? 0u : b2[r];
      my_key[r] = lane == j ? top[r] : my_key[r];
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const u32 kth = readlane_u32(my_key[r], k - 1);
    // distinct keys: the k kept keys strictly decrease
    const u32 prev = (u32)__builtin_amdgcn_ds_bpermute(4 * max(lane - 1, 0), (int)my_key[r]);
    const bool dup = lane >= 1 && lane < k && prev == my_key[r];
    const bool sel0 = key[r][0] >= kth, sel1 = key[r][1] >= kth;
    const int nsel = __popcll(ballot64(sel0)) + __popcll(ballot64(sel1));
    retry[r] = __popcll(ballot64(dup)) != 0 || nsel != k;
    if (retry[r]) continue;
    // slot = number of kept keys above the element's key: the kept keys go to
    // LDS (zeros past k) and every lane reads them back four at a time (one
    // LDS broadcast per four keys instead of a readlane per key)
    int* slot = s_slot + 64 * r;
    u32* s_k = reinterpret_cast<u32*>(slot + 32);
    if (lane < 32) s_k[lane] = lane < k ? my_key[r] : 0u;
    int r0 = 0, r1 = 0;
#pragma unroll
    for (int j0 = 0; j0 < 32; j0 += 4) {
      if (j0 < k) {
        const uint4 t = *reinterpret_cast<const uint4*>(s_k + j0);
        r0 += (t.x > key[r][0]) + (t.y > key[r][0]) + (t.z > key[r][0]) + (t.w > key[r][0]);
        r1 += (t.x > key[r][1]) + (t.y > key[r][1]) + (t.z > key[r][1]) + (t.w > key[r][1]);
      }
    }
    if (sel0) slot[r0] = 2 * lane;
    if (sel1) slot[r1] = 2 * lane + 1;
    my_id[r] = slot[min(lane, k - 1)];  // one wave: the LDS writes above land first
  }
}

// Descending sort of NV keys in registers: Batcher's odd-even merge sort
// (every loop bound is a compile-time constant, so it unrolls into a fixed
// network of max/min pairs).
template <int NV>
__device__ __forceinline__ void sort_desc(u32 (&b)[NV]) {
#pragma unroll
  for (int p = 1; p < NV; p <<= 1)
#pragma unroll
    for (int k = p; k >= 1; k >>= 1)
#pragma unroll
      for (int j = k % p; j + k < NV; j += 2 * k)
#pragma unroll
        for (int i = 0; i < k; ++i)
          if (i + j + k < NV && (i + j) / (2 * p) == (i + j + k) / (2 * p)) {
            const u32 hi = umax(b[i + j], b[i + j + k]), lo = b[i + j] + b[i + j + k] - hi;
            b[i + j] = hi;
            b[i + j + k] = lo;
          }
}

// Fast selection for NV > 2 keys per lane: each lane sorts its keys once; a
// round is the wave maximum of the lanes' first keys and a shift of the list
// in the lane(s) holding it, which also note their lane in s_slot[j]. Lane
// j then finds the expert by reading the winner lane's original keys
// (ds_bpermute) for the one equal to its key. As for two keys, ties make the
// caller run the exact selection: a round won by two lanes (more shifts than
// rounds), or equal kept keys.
template <int NV>
__device__ __forceinline__ bool select_fast_sorted(const u32 (&key)[NV], int k, u32& my_key, int& my_id,
                                                   int* s_slot) {
  const int lane = lane_id();
  u32 b[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) b[i] = key[i];
  sort_desc<NV>(b);
  int hits = 0;
  for (int j = 0; j < k; ++j) {
    const u32 top = wave_max_u32(b[0]);
    const bool hit = b[0] == top;
    // the shift as bit selects (v_bfi): a conditional select would be turned
    // into a computed register index
    const u32 msk = 0u - (u32)hit;
#pragma unroll
    for (int i = 0; i + 1 < NV; ++i) b[i] = (b[i + 1] & msk) | (b[i] & ~msk);
    b[NV - 1] &= ~msk;
    hits += hit ? 1 : 0;
    if (hit) s_slot[j] = lane;
    my_key = lane == j ? top : my_key;
  }
  const u32 prev = (u32)__builtin_amdgcn_ds_bpermute(4 * max(lane - 1, 0), (int)my_key);
  const bool dup = lane >= 1 && lane < k && prev == my_key;
  if (__popcll(ballot64(dup)) != 0 || wave_sum_i32(hits) != k) return true;
  const int wl = s_slot[min(lane, k - 1)];  // one wave: the LDS writes above land first
  int slot = 0;
#pragma unroll
  for (int i = NV - 1; i >= 0; --i) {  // the lowest matching slot wins
    const u32 v = (u32)__builtin_amdgcn_ds_bpermute(4 * wl, (int)key[i]);
    slot = v == my_key ? i : slot;
  }
  my_id = wl * NV + slot;
  return false;
}

// Top-k by threshold, for up to four keys per lane (lane-major: the key of
// expert lane*NV + i in key[i], 0 for an absent expert). The selected set is
// fixed by the largest T with #{key >= T} >= k, found bit by bit from the top
// bit: a candidate T | 2^b is kept when at least k keys reach it (one ballot
// count per key slot, uniform scalar work), and the search stops at the first
// T that exactly k keys reach. (Measured slower: two bits a step with three
// candidates counted at once, and skipping candidates above the largest key;
// the wave issues one instruction at a time, and the compiler turns either
// into a loop with more branches and selects than the steps they save.)
// Without such a T (equal keys straddle the k-th place) T ends as the k-th
// largest key: every key above it is selected, and of the keys equal to it
// the ones with the lowest expert index, as many as are missing. Lane-local
// result: sel[i].
#ifndef RGT_SELECT_EXIT_BITS
#define RGT_SELECT_EXIT_BITS 24
#endif
template <int NV>
__device__ __forceinline__ void wave_threshold_select(const u32 (&key)[NV], int k, bool (&sel)[NV]) {
  constexpr int kExitBits = RGT_SELECT_EXIT_BITS;
  static_assert(NV <= 4, "the threshold selection takes up to four keys per lane");
  u32 T = 0;
  bool exact = false;
#pragma unroll
  for (int b = 31; b >= 0; --b) {
    const u32 c = T | (1u << b);
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < NV; ++i) cnt += __popcll(ballot64(key[i] >= c));
    if (cnt >= k) {
      T = c;
      // No exit test in the sign and exponent rounds (saves its three
      // instructions where an exact count is rare). A count of exactly k
      // reached there stays exact: later candidates are kept only if k keys
      // still reach them, and if none is, the tie path below selects the
      // keys >= T, which are then exactly k.
      if (b < kExitBits && cnt == k) {
        exact = true;
        break;
      }
    }
  }
  if (exact) {
#pragma unroll
    for (int i = 0; i < NV; ++i) sel[i] = key[i] >= T;
  } else {
    int ngt = 0, below = 0;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      ngt += __popcll(ballot64(key[i] > T));
      below += __popcll(ballot64(key[i] == T) & lanemask_lt());
    }
    const int need = k - ngt;  // >= 1: at least k keys reach T, fewer exceed it
    int run = below;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const bool eq = key[i] == T;
      sel[i] = key[i] > T || (eq && run < need);
      run += eq ? 1 : 0;
    }
  }
}

// Position of each selected key in expert order among the selected ones
// (selected keys of lower lanes, then of lower slots of this lane): a
// one-to-one map of the selection onto 0 .. k-1, for callers to which the
// order of the k winners does not matter.
template <int NV>
__device__ __forceinline__ void wave_select_order(const bool (&sel)[NV], int (&pos)[NV]) {
  int cpos = 0;
#pragma unroll
  for (int i = 0; i < NV; ++i) cpos += __popcll(ballot64(sel[i]) & lanemask_lt());
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    pos[i] = cpos;
    cpos += sel[i] ? 1 : 0;
  }
}

// The winners' slots (the number of selected keys that rank above, by key,
// then expert index) from one compare against the k selected keys, compacted
// in expert order through s_c (KMAX u64 of LDS owned by the calling wave;
// k <= KMAX). Lane-local: for a selected key, slot[i].
template <int NV, int KMAX>
__device__ __forceinline__ void wave_select_slots(const u32 (&key)[NV], const bool (&sel)[NV], int (&slot)[NV],
                                                  u64* s_c) {
  const int lane = lane_id();
  int cpos[NV];
  wave_select_order<NV>(sel, cpos);
  u64 comp[NV];
  if (lane < KMAX) s_c[lane] = 0ull;  // entries past k never rank above anything
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    // key first; among equal keys the lower expert (lower position) ranks higher
    comp[i] = ((u64)key[i] << 32) | (u64)(~(u32)cpos[i]);
    if (sel[i]) s_c[cpos[i]] = comp[i];
  }
  // one wave: its LDS writes above land before these reads
  int cntv[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) cntv[i] = 0;
#pragma unroll
  for (int q = 0; q < KMAX; q += 2) {
    const ulonglong2 v = *reinterpret_cast<const ulonglong2*>(s_c + q);
#pragma unroll
    for (int i = 0; i < NV; ++i) cntv[i] += (v.x > comp[i] ? 1 : 0) + (v.y > comp[i] ? 1 : 0);
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) slot[i] = cntv[i];
}

// Selection and slots together (k <= KMAX).
template <int NV, int KMAX>
__device__ __forceinline__ void wave_topk_threshold(const u32 (&key)[NV], int k, bool (&sel)[NV], int (&slot)[NV],
                                                    u64* s_c) {
  wave_threshold_select<NV>(key, k, sel);
  wave_select_slots<NV, KMAX>(key, sel, slot, s_c);
}

#ifndef RGT_SELECT_PRUNED
#define RGT_SELECT_PRUNED 1
#endif
// Selection for many keys a lane (NV > 4) by pruning first. L, the k-th
// largest of the 64 lane maxima, is reached by at least k keys, so the k-th
// largest key, and with it every selected key, is at least L. The keys >= L
// are moved to LDS in expert order (lane l's after those of the lanes below
// it, each lane's in slot order) and, when at most 64 of them, selected one
// a lane with the threshold selection and its slots: the same set and order
// (descending key, equal keys by lower expert) as over all keys. Returns
// true (nothing selected) when more than 64 keys reach L or L is 0 (absent
// experts among the candidates); the caller then selects over all keys.
// s_w: 256 u32 of LDS owned by the calling wave (8-byte aligned).
template <int NV>
__device__ __forceinline__ bool select_pruned(const u32 (&key)[NV], int k, u32& my_key, int& my_id, u32* s_w) {
  const int lane = lane_id();
  u32 mx = key[0];
#pragma unroll
  for (int i = 1; i < NV; ++i) mx = umax(mx, key[i]);
  bool lsel[1];
  const u32 mk[1] = {mx};
  wave_threshold_select<1>(mk, k, lsel);
  const u32 L = ~wave_max_u32(lsel[0] ? ~mx : 0u);  // the smallest selected lane maximum
  int cnt = 0;
#pragma unroll
  for (int i = 0; i < NV; ++i) cnt += key[i] >= L ? 1 : 0;
  const int incl = wave_inclusive_scan(cnt);
  const int total = __builtin_amdgcn_readlane(incl, 63);
  if (L == 0u || total > 64) return true;  // uniform
  u32* const s_key = s_w;        // [64] candidate keys
  u32* const s_id = s_w + 64;    // [64] candidate experts
  u64* const s_c = reinterpret_cast<u64*>(s_w + 128);  // [32] slot ranks
  int p = incl - cnt;
#pragma unroll
  for (int i = 0; i < NV; ++i)
    if (key[i] >= L) {
      s_key[p] = key[i];
      s_id[p] = (u32)(lane * NV + i);
      ++p;
    }
  // one wave: the LDS writes above land before these reads
  const u32 ck[1] = {lane < total ? s_key[lane] : 0u};
  const u32 cid = s_id[lane];
  bool sel[1];
  int slot[1];
  if (k <= 8) wave_topk_threshold<1, 8>(ck, k, sel, slot, s_c);
  else if (k <= 16) wave_topk_threshold<1, 16>(ck, k, sel, slot, s_c);
  else wave_topk_threshold<1, 32>(ck, k, sel, slot, s_c);
  // slot j's key and expert to lane j (s_key / s_id are read above: reused)
  if (sel[0]) {
    s_key[slot[0]] = ck[0];
    s_id[slot[0]] = cid;
  }
  if (lane < k) {
    my_key = s_key[lane];
    my_id = (int)s_id[lane];
  }
  return false;
}

// Selection only for R rows at once (R = 1 or 2): lane j < k ends with the
// j-th expert of row r in my_id[r] and its score key in my_key[r]. s_slot:
// 64*R ints of LDS owned by the calling wave (16-byte aligned).
template <int NV, int R>
__device__ __forceinline__ void wave_select_rows(const float (&sv)[R][NV], int n, int k, int (&my_id)[R],
                                                 u32 (&my_key)[R], int* s_slot) {
  const int lane = lane_id();
  u32 key[R][NV];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int i = 0; i < NV; ++i) key[r][i] = lane * NV + i < n ? score_key(sv[r][i]) : 0u;
  bool retry[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    my_id[r] = 0;
    my_key[r] = 0u;
    retry[r] = true;
  }
  if constexpr (NV == 2) {
    select_fast2<R>(key, k, my_key, my_id, retry, s_slot);
  } else {
#if RGT_SELECT_PRUNED
    if constexpr (NV > 4) {
      __shared__ __align__(16) u32 s_prune[4][256];
#pragma unroll
      for (int r = 0; r < R; ++r) retry[r] = select_pruned<NV>(key[r], k, my_key[r], my_id[r], s_prune[threadIdx.x >> 6]);
    }
#endif
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (retry[r]) retry[r] = select_fast_sorted<NV>(key[r], k, my_key[r], my_id[r], s_slot + 64 * r);
  }
#pragma unroll
  for (int r = 0; r < R; ++r)
    if (retry[r]) select_exact<NV>(key[r], k, my_key[r], my_id[r]);
}

// Top-k of one row of scores held in registers (lane-major, valid below n).
// Lane j < k ends with the j-th expert in my_id and its renormalised weight
// in my_w.
// Selection only: lane j < k ends with the j-th expert in my_id and its
// score key in my_key. s_slot: 64 ints of LDS owned by the calling wave.
template <int NV>
__device__ __forceinline__ void wave_select(const float (&sv)[NV], int n, int k, int& my_id, u32& my_key,
                                            int* s_slot) {
  float sv1[1][NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) sv1[0][i] = sv[i];
  int id[1];
  u32 key[1];
  wave_select_rows<NV, 1>(sv1, n, k, id, key, s_slot);
  my_id = id[0];
  my_key = key[0];
}

// Renormalised softmax over the k selected scores (lane j holds the key of
// slot j; slot 0 the largest): the weight of lane j < k.
__device__ __forceinline__ float wave_weights(u32 my_key, int k) {
  const int lane = lane_id();
  const float my_s = key_score(my_key);
  const double s0 = (double)readlane_f32(my_s, 0);
  double e = 0.0;
  if (lane < k) e = exp64_recipe((double)my_s - s0);
  const double total = k <= 8 ? slot_sum<8>(e) : (k <= 16 ? slot_sum<16>(e) : slot_sum<32>(e));
  return lane < k ? (float)(e / total) : 0.f;
}

template <int NV>
__device__ __forceinline__ void wave_topk_regs(const float (&sv)[NV], int n, int k, int& my_id, float& my_w,
                                               int* s_slot) {
  u32 my_key;
  wave_select<NV>(sv, n, k, my_id, my_key, s_slot);
  my_w = wave_weights(my_key, k);
}

// Load a row of logits lane-major (all loads issued before any is used:
// addresses are clamped into the row), add the bias and run the top-k; lanes
// j < k write slot j.
template <int NV>
__device__ __forceinline__ void wave_topk_row(const float* logits_row, const float* bias, int n, int k,
                                              int32_t* ids_out, float* w_out, int* s_slot) {
  const int c0 = lane_id() * NV;
  float sv[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) sv[i] = logits_row[min(c0 + i, n - 1)];
  add_bias<NV>(sv, bias, n);
  int id;
  float w;
  wave_topk_regs<NV>(sv, n, k, id, w, s_slot);
  if (lane_id() < k) {
    ids_out[lane_id()] = id;
    w_out[lane_id()] = w;
  }
}

// Gate fed the split-K partials part[S][M][N] of the router: each lane sums
// its experts' partials in k-slice order (one fp32 add per slice; SB slices
// are loaded at a time, 32 for two experts a lane, so a wide batch's slices
// cost one memory round trip), optionally writes the
// logits, then selects as the plain gate. One wave per row.
template <int NV>
__global__ void __launch_bounds__(256) topk_gate_partials_kernel(const float* part, int S, float* logits_out,
                                                                 const float* bias, int m, int n, int k,
                                                                 int32_t* ids, float* w) {
  constexpr int SB = NV <= 2 ? 32 : (NV <= 4 ? 16 : (NV <= 8 ? 8 : 4));
  __shared__ __align__(16) int s_slot[4][64];
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= m) return;
  const int c0 = lane_id() * NV;
  const int64_t slice = (int64_t)m * n;
  const float* src = part + (int64_t)row * n;
  float sv[NV];
  for (int s0 = 0; s0 < S; s0 += SB) {
    float v[SB][NV];
#pragma unroll
    for (int j = 0; j < SB; ++j)
#pragma unroll
      for (int i = 0; i < NV; ++i) v[j][i] = src[(int64_t)min(s0 + j, S - 1) * slice + min(c0 + i, n - 1)];
#pragma unroll
    for (int j = 0; j < SB; ++j)
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        if (s0 + j == 0) sv[i] = v[j][i];
        else if (s0 + j < S) sv[i] = __fadd_rn(sv[i], v[j][i]);
      }
  }
  if (logits_out) {
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (c0 + i < n) logits_out[(int64_t)row * n + c0 + i] = sv[i];
  }
  add_bias<NV>(sv, bias, n);
  int id;
  float wt;
  wave_topk_regs<NV>(sv, n, k, id, wt, s_slot[threadIdx.x >> 6]);
  if (lane_id() < k) {
    ids[(int64_t)row * k + lane_id()] = id;
    w[(int64_t)row * k + lane_id()] = wt;
  }
}

template <int NV>
__global__ void __launch_bounds__(256) topk_gate_kernel(const float* logits, const float* bias, int m, int n, int k,
                                                        int32_t* ids, float* w) {
  __shared__ __align__(16) int s_slot[4][64];
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= m) return;
  wave_topk_row<NV>(logits + (int64_t)row * n, bias, n, k, ids + (int64_t)row * k, w + (int64_t)row * k,
                    s_slot[threadIdx.x >> 6]);
}

}  // namespace rgt
