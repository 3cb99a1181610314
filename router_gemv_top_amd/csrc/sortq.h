// sortq.h - token -> expert sort into block-padded segments, and the MXFP8
// gather-quant of the activations.
//
// Sort (sglang PR #46691, Summary: MoE sorting + quant; "Kimi-K3: fused MoE
// routing, sort, quant and epilogue", review snippet on the stable rank):
// pair p = m*k + j goes to expert e = ids[m][j]; segment e starts at
// offsets[e] = sum_{e'<e} roundup(cnt[e'], B) and lists its pairs in
// ascending p, then the sentinel P = M*k up to the block boundary.
//
// GPU method: histogram -> exclusive scan -> stable scatter. Stable ranks are
// built from wave batches of 64 pairs: lanes holding the same expert find one
// another with one ballot per bit of the expert id, so a lane's rank inside
// its batch is a popcount; a per-(wave, expert) running count in LDS carries
// the rank across batches. For decode sizes one workgroup does everything; for
// large P the histogram is split over workgroups and a scan launch joins them.
//
// Quant (OCP MX: e8m0 scale per 32 elements, e4m3fn elements; group-32 scales
// as in the MXFP8 shared-expert commit of sgl-amd-mono PR #56): each lane
// quantises 16 consecutive elements of a token row; two neighbouring lanes
// form a 32-element block and exchange their maxima. A token row is read once
// and its codes are stored to all k padded positions of its pairs.
#pragma once

#include "device.h"

namespace rgt {

// Lanes in the active mask whose expert id equals mine (bits of e < 2^bits).
__device__ __forceinline__ u64 match_peers(int e, bool valid, int bits) {
  u64 peers = ballot64(valid);
  for (int b = 0; b < bits; ++b) {
    const bool bit = (e >> b) & 1;
    const u64 m = ballot64(bit);
    peers &= bit ? m : ~m;
  }
  return peers;
}

// The same with a compile-time bound on the id bits (ids < 2^BITS): the
// ballots are unrolled, and bits above the ids' range are skipped at run time.
template <int BITS>
__device__ __forceinline__ u64 match_peers_n(int e, bool valid, int bits) {
  u64 peers = ballot64(valid);
#pragma unroll
  for (int b = 0; b < BITS; ++b) {
    if (b < bits) {
      const bool bit = (e >> b) & 1;
      const u64 m = ballot64(bit);
      peers &= bit ? m : ~m;
    }
  }
  return peers;
}

__device__ __forceinline__ int ceil_log2(int n) { return n <= 1 ? 0 : 32 - __clz(n - 1); }

// Block sizes are powers of two: round up / divide with masks and shifts (a
// GPU has no integer divide instruction; a runtime division costs ~40
// instructions).
__device__ __forceinline__ int pad_to(int c, int B) { return (c + B - 1) & -B; }
__device__ __forceinline__ int div_pow2(int a, int B) { return a >> (__ffs(B) - 1); }

// Exclusive scan of vals[0..n) in LDS (in place). Returns the total. Each
// thread sums a contiguous run of ceil(n / blockDim.x) values; wave 0 scans
// the thread sums (each lane a contiguous run of blockDim.x / 64 of them, then
// a DPP wave scan) and every thread writes its run's prefixes: two barriers
// whatever the workgroup size (a tree over the threads would need two per
// level). blockDim.x is a multiple of 64. Uses scratch[blockDim.x] of LDS.
__device__ __forceinline__ int block_exclusive_scan(int* vals, int n, int* scratch) {
  __shared__ int s_total;
  const int t = threadIdx.x, nt = blockDim.x;
  const int per = (n + nt - 1) / nt;
  const int b0 = min(n, t * per), b1 = min(n, b0 + per);
  int local = 0;
  for (int i = b0; i < b1; ++i) local += vals[i];
  scratch[t] = local;
  __syncthreads();
  if (t < 64) {
    const int q = nt >> 6;
    int sum = 0;
    for (int i = 0; i < q; ++i) sum += scratch[t * q + i];
    const int incl = wave_inclusive_scan(sum);
    int run = incl - sum;
    for (int i = 0; i < q; ++i) {
      const int v = scratch[t * q + i];
      scratch[t * q + i] = run;
      run += v;
    }
    if (t == 63) s_total = incl;
  }
  __syncthreads();
  int run = scratch[t];
  for (int i = b0; i < b1; ++i) {
    const int v = vals[i];
    vals[i] = run;
    run += v;
  }
  const int total = s_total;
  __syncthreads();
  return total;
}

// One-workgroup sort of P pairs. LDS (caller-provided):
//   s_e[P]      expert of each pair
//   s_hist[W*N] per-wave counts, turned into per-wave bases
//   s_cnt[N]    total count per expert
//   s_off[N+1]  padded segment starts
//   s_scr[blockDim.x]
// Results: s_off, s_cnt in LDS; pos[p] (LDS or global) = padded position of p.
// Returns the padded total.
// COH: the ids were written by other workgroups of the same launch.
template <bool COH, typename PosPtr>
__device__ int wg_sort(const int32_t* ids, int P, int N, int B, int* s_e, int* s_hist, int* s_cnt, int* s_off,
                       int* s_scr, PosPtr pos, int32_t* sorted_ids = nullptr) {
  const int t = threadIdx.x, nt = blockDim.x, nw = nt >> 6;
  const int wave = t >> 6, lane = t & 63;
  for (int p = t; p < P; p += nt) s_e[p] = COH ? ld_agent(ids + p) : ids[p];
  for (int i = t; i < nw * N; i += nt) s_hist[i] = 0;
  __syncthreads();
  // Pass 1: per-wave histograms over contiguous chunks of pairs.
  const int chunk = ((P + nw - 1) / nw + 63) & ~63;
  const int c0 = min(P, wave * chunk), c1 = min(P, c0 + chunk);
  for (int p = c0 + lane; p < c1; p += 64) {
    const int e = s_e[p];
    if ((unsigned)e < (unsigned)N) atomicAdd(&s_hist[wave * N + e], 1);
  }
  __syncthreads();
  // Per-expert totals; per-wave counts become exclusive per-wave bases.
  if (nw == 16) {
    // One 16-lane row per expert (lane = wave index w): a DPP scan inside the
    // row. N*16 is a multiple of 256, so whole waves take part.
    for (int idx = t; idx < N * 16; idx += nt) {
      const int e = idx >> 4, w = idx & 15;
      const int v = s_hist[w * N + e];
      int incl = v;
      incl += __builtin_amdgcn_update_dpp(0, incl, 0x111, 0xF, 0xF, true);  // row_shr:1
      incl += __builtin_amdgcn_update_dpp(0, incl, 0x112, 0xF, 0xF, true);  // row_shr:2
      incl += __builtin_amdgcn_update_dpp(0, incl, 0x114, 0xF, 0xF, true);  // row_shr:4
      incl += __builtin_amdgcn_update_dpp(0, incl, 0x118, 0xF, 0xF, true);  // row_shr:8
      s_hist[w * N + e] = incl - v;
      if (w == 15) {
        s_cnt[e] = incl;
        s_off[e] = pad_to(incl, B);
      }
    }
  } else {
    for (int e = t; e < N; e += nt) {
      int run = 0;
      for (int w = 0; w < nw; ++w) {
        const int c = s_hist[w * N + e];
        s_hist[w * N + e] = run;
        run += c;
      }
      s_cnt[e] = run;
      s_off[e] = pad_to(run, B);
    }
  }
  __syncthreads();
  const int total = block_exclusive_scan(s_off, N, s_scr);
  if (t == 0) s_off[N] = total;
  __syncthreads();
  // Pass 2: stable ranks inside each wave's chunk, batch by batch.
  const int bits = ceil_log2(N);
  for (int base = c0; base < c1; base += 64) {
    const int p = base + lane;
    const int e = p < c1 ? s_e[p] : 0;
    // Expert ids outside [0, N) are a caller error: such pairs are left out
    // of the sort (position -1) instead of indexing out of bounds.
    const bool valid = p < c1 && (unsigned)e < (unsigned)N;
    const u64 peers = match_peers(e, valid, bits);
    if (valid) {
      const int rank = __popcll(peers & lanemask_lt());
      const int q = s_off[e] + s_hist[wave * N + e] + rank;
      pos[p] = q;
      if (sorted_ids) sorted_ids[q] = p;
    } else if (p < c1) {
      pos[p] = -1;
    }
    // Order the reads above before the leader's update (same wave, LDS is in order).
    if (valid && (peers & lanemask_lt()) == 0ull) s_hist[wave * N + e] += __popcll(peers);
  }
  __syncthreads();
  return total;
}

// Padded counts -> exclusive segment offsets, by one wave. Lane l owns the C
// consecutive experts from l*C (C = ceil(N/64) <= CMAX). All CMAX counts are
// read from clamped addresses with no branch between the reads, so their LDS
// latencies overlap. Writes s_off[0..N]; returns the padded total.
template <int CMAX>
__device__ __forceinline__ int wave_scan_offsets(const int* s_cnt, int* s_off, int N, int B) {
  const int lane = lane_id();
  const int C = (N + 63) >> 6;
  const int e0 = lane * C;
  int pc[CMAX];
  int local = 0;
#pragma unroll
  for (int i = 0; i < CMAX; ++i) {
    const int v = s_cnt[min(e0 + i, N - 1)];
    pc[i] = (i < C && e0 + i < N) ? pad_to(v, B) : 0;
    local += pc[i];
  }
  const int incl = wave_inclusive_scan(local);
  const int total = (int)readlane_u32((u32)incl, 63);
  int run = incl - local;
#pragma unroll
  for (int i = 0; i < CMAX; ++i) {
    if (i < C && e0 + i < N) s_off[e0 + i] = run;
    run += pc[i];
  }
  if (lane == 0) s_off[N] = total;
  return total;
}

// One-wave sort of up to a few thousand pairs (called by one whole wave, no
// barriers: LDS accesses of one wave are performed in program order).
// Batches of 64 pairs are taken in pair order; a lane's stable rank is the
// running count of its expert before the batch plus its rank among the batch's
// lanes with the same expert, and the batch's first lane of each expert then
// advances that count. LDS: s_e[P], s_rank[P], s_cnt[N], s_off[N+1].
// Results: s_cnt, s_off (N+1 entries) and pos[p] (LDS or global), -1 for a
// pair whose expert id is outside [0, N). Returns the padded total.
// With ids == nullptr, s_e already holds the experts.
template <int CMAX, typename PosPtr>
__device__ int wave_sort(const int32_t* ids, int P, int N, int B, int* s_e, int* s_rank, int* s_cnt, int* s_off,
                         PosPtr pos) {
  const int lane = lane_id();
  for (int e = lane; e < N; e += 64) s_cnt[e] = 0;
  if (ids) {
    // Load the ids 8 per lane at a time with clamped addresses and no branches
    // between the loads, so each group costs one memory round trip.
    for (int p0 = 0; p0 < P; p0 += 8 * 64) {
      int v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = ids[min(p0 + j * 64 + lane, P - 1)];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (p0 + j * 64 + lane < P) s_e[p0 + j * 64 + lane] = v[j];
    }
  }
  const int bits = ceil_log2(N);
  for (int base = 0; base < P; base += 64) {
    const int p = base + lane;
    const int e = p < P ? s_e[p] : 0;
    const bool valid = p < P && (unsigned)e < (unsigned)N;
    const u64 peers = match_peers(e, valid, bits);
    if (valid) {
      const u64 below = peers & lanemask_lt();
      const int c = s_cnt[e];
      s_rank[p] = c + __popcll(below);
      if (below == 0ull) s_cnt[e] = c + __popcll(peers);
    }
  }
  const int total = wave_scan_offsets<CMAX>(s_cnt, s_off, N, B);
  for (int p = lane; p < P; p += 64) {
    const int e = s_e[p];
    pos[p] = (unsigned)e < (unsigned)N ? s_off[e] + s_rank[p] : -1;
  }
  return total;
}

// One-wave sort of at most 64 pairs (pair p in lane p), no loops: stable ranks
// from one batch of peer ballots, counts and padded offsets through LDS.
// s_e[P] holds the experts; results as for wave_sort.
constexpr int kWaveSortSmallP = 64;

template <int CMAX, typename PosPtr>
__device__ int wave_sort_small(int P, int N, int B, const int* s_e, int* s_cnt, int* s_off, PosPtr pos) {
  const int lane = lane_id();
  const int C = (N + 63) >> 6;
  const int e0 = lane * C;
#pragma unroll
  for (int i = 0; i < CMAX; ++i)
    if (i < C && e0 + i < N) s_cnt[e0 + i] = 0;
  const int e = s_e[min(lane, P - 1)];
  const bool valid = lane < P && (unsigned)e < (unsigned)N;
  const u64 peers = match_peers_n<6 + (CMAX > 1) + (CMAX > 2) + (CMAX > 4) + (CMAX > 8)>(e, valid, ceil_log2(N));
  const u64 below = peers & lanemask_lt();
  const int rank = __popcll(below);
  if (valid && below == 0ull) s_cnt[e] = __popcll(peers);  // after the zeroing (one wave: LDS in order)
  const int total = wave_scan_offsets<CMAX>(s_cnt, s_off, N, B);
  const int o = s_off[valid ? e : 0];
  if (lane < P) pos[lane] = valid ? o + rank : -1;
  return total;
}

// Write offsets, sentinel pads of sorted_ids and expert_ids from the LDS
// results of a sort. Pair entries of sorted_ids are written by the caller.
__device__ __forceinline__ void write_sort_layout(const int* s_cnt, const int* s_off, int N, int B, int P,
                                                  int32_t* sorted_ids, int32_t* expert_ids, int32_t* offsets) {
  for (int e = threadIdx.x; e <= N; e += blockDim.x) offsets[e] = s_off[e];
  for (int e = threadIdx.x; e < N; e += blockDim.x) {
    const int a = s_off[e], b = s_off[e + 1];
    for (int q = a + s_cnt[e]; q < b; ++q) sorted_ids[q] = P;
    for (int blk = div_pow2(a, B); blk < div_pow2(b, B); ++blk) expert_ids[blk] = e;
  }
}

// Four-wave sort of P <= kSortWg4MaxP pairs held in s_e (LDS), called by the
// whole 256-thread workgroup. Wave w takes the contiguous chunk of pairs
// [w*Q, (w+1)*Q) (Q a multiple of 64) in batches of 64: a pair's rank is the
// running count of its expert in the wave's chunk (s_hist[w][e]) plus its
// rank among the batch's lanes with the same expert. One wave then turns the
// per-wave counts into padded segment offsets and per-wave bases, and every
// pair's position is base + rank. LDS: s_rank[P], s_hist[4*N], s_cnt[N],
// s_off[N+1]. Results as for wave_sort.
constexpr int kSortWg4MaxP = 2048;

template <int CMAX, typename PosPtr>
__device__ int wg4_sort(int P, int N, int B, const int* s_e, int* s_rank, int* s_hist, int* s_cnt, int* s_off,
                        PosPtr pos) {
  constexpr int BITS = 6 + (CMAX > 1) + (CMAX > 2) + (CMAX > 4) + (CMAX > 8);
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  for (int i = t; i < 4 * N; i += 256) s_hist[i] = 0;
  __syncthreads();
  const int Q = (((P + 3) >> 2) + 63) & ~63;
  const int c0 = min(P, wave * Q), c1 = min(P, c0 + Q);
  const int bits = ceil_log2(N);
  int* run = s_hist + wave * N;
  for (int base = c0; base < c1; base += 64) {
    const int p = base + lane;
    const int e = s_e[min(p, P - 1)];
    const bool valid = p < c1 && (unsigned)e < (unsigned)N;
    const u64 peers = match_peers_n<BITS>(e, valid, bits);
    const u64 below = peers & lanemask_lt();
    if (valid) {
      const int c = run[e];
      s_rank[p] = c + __popcll(below);
      if (below == 0ull) run[e] = c + __popcll(peers);  // one wave: LDS in order
    }
  }
  __syncthreads();
  if (wave == 0) {
    // Lane l owns experts [l*C, l*C + C); the 4*C per-wave counts are read
    // from clamped addresses with no branch between the reads.
    const int C = (N + 63) >> 6;
    const int e0 = lane * C;
    int h[4][CMAX], pc[CMAX];
    int local = 0;
#pragma unroll
    for (int i = 0; i < CMAX; ++i)
#pragma unroll
      for (int w = 0; w < 4; ++w) h[w][i] = s_hist[w * N + min(e0 + i, N - 1)];
#pragma unroll
    for (int i = 0; i < CMAX; ++i) {
      const int tot = h[0][i] + h[1][i] + h[2][i] + h[3][i];
      pc[i] = (i < C && e0 + i < N) ? pad_to(tot, B) : 0;
      local += pc[i];
    }
    const int incl = wave_inclusive_scan(local);
    const int total = (int)readlane_u32((u32)incl, 63);
    int off = incl - local;
#pragma unroll
    for (int i = 0; i < CMAX; ++i) {
      if (i < C && e0 + i < N) {
        const int e = e0 + i;
        s_off[e] = off;
        s_cnt[e] = h[0][i] + h[1][i] + h[2][i] + h[3][i];
        s_hist[e] = off;
        s_hist[N + e] = off + h[0][i];
        s_hist[2 * N + e] = off + h[0][i] + h[1][i];
        s_hist[3 * N + e] = off + h[0][i] + h[1][i] + h[2][i];
      }
      off += pc[i];
    }
    if (lane == 0) s_off[N] = total;
  }
  __syncthreads();
  for (int p = c0 + lane; p < c1; p += 64) {
    const int e = s_e[p];
    pos[p] = (unsigned)e < (unsigned)N ? run[e] + s_rank[p] : -1;
  }
  __syncthreads();
  return s_off[N];
}

// Counting sort of the pairs by expert, from histograms alone (no full
// stable sort): with cnt[e] the number of pairs of expert e,
//   off[e] = sum over e' < e of roundup(cnt[e'], B),
//   pos(p) = off[e_p] + #{p' < p : e_p' = e_p}.
// A workgroup needs the positions of its own pairs [p0, p1) only; the pairs
// before p0 are counted by a second histogram pre[e] over p' < p0, and the
// earlier own pairs by peer ballots.
//
// hist_add: called once per pair as its expert becomes known (LDS atomics
// into s_cnt and s_pre, zeroed beforehand).
__device__ __forceinline__ void hist_add(int e, int p, int p0, int N, int* s_cnt, int* s_pre) {
  if ((unsigned)e < (unsigned)N) {
    atomicAdd(&s_cnt[e], 1);
    if (p < p0) atomicAdd(&s_pre[e], 1);
  }
}

// pair_positions: one wave, after the histograms are complete (a barrier
// after the last hist_add). Writes s_off[0..N] and s_pos[p - p0] for the own
// pairs (p1 - p0 <= 64; -1 for an expert id outside [0, N)).
template <int CMAX>
__device__ __forceinline__ void pair_positions(int P, int N, int B, int p0, int p1, const int* s_e, const int* s_cnt,
                                               const int* s_pre, int* s_off, int* s_pos) {
  constexpr int BITS = 6 + (CMAX > 1) + (CMAX > 2) + (CMAX > 4) + (CMAX > 8);
  const int lane = lane_id();
  const int p = p0 + lane;
  const int e = s_e[min(p, P - 1)];
  wave_scan_offsets<CMAX>(s_cnt, s_off, N, B);
  const bool valid = p < p1 && (unsigned)e < (unsigned)N;
  const u64 peers = match_peers_n<BITS>(e, valid, ceil_log2(N));
  const int rank = __popcll(peers & lanemask_lt());
  const int ee = valid ? e : 0;
  const int q = s_off[ee] + s_pre[ee] + rank;  // one wave: after the scan's writes
  if (p < p1) s_pos[lane] = valid ? q : -1;
}

// Offsets, expert_ids and the sentinel pads of sorted_ids of experts
// [e0, e1) from the histogram and offsets in LDS (the pairs' own entries are
// written by their owners; offsets[N] by the range that ends at N). Pads:
// one item (e, j) per slot j < B after expert e's pairs, eight items per
// thread with their LDS reads issued together. Called by all NT threads.
template <int NT>
__device__ __forceinline__ void write_layout(const int* s_cnt, const int* s_off, int N, int B, int P, int e0, int e1,
                                             int32_t* sorted_ids, int32_t* expert_ids, int32_t* offsets) {
  const int lb = __ffs(B) - 1;
  const int t = threadIdx.x;
  for (int e = e0 + t; e < e1 + (e1 == N ? 1 : 0); e += NT) offsets[e] = s_off[e];
  for (int e = e0 + t; e < e1; e += NT) {
    const int b0 = s_off[e] >> lb, b1 = s_off[e + 1] >> lb;
    for (int blk = b0; blk < b1; ++blk) expert_ids[blk] = e;
  }
  const int items = (e1 - e0) << lb;
  for (int it0 = 0; it0 < items; it0 += 8 * NT) {
    int a[8], b[8], c[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = e0 + min((it0 + t + u * NT) >> lb, e1 - e0 - 1);
      a[u] = s_off[e];
      b[u] = s_off[e + 1];
      c[u] = s_cnt[e];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int it = it0 + t + u * NT;
      const int q = a[u] + c[u] + (it & (B - 1));
      if (it < items && q < b[u]) sorted_ids[q] = P;
    }
  }
}

// Sort outputs of a decode-size sort held in LDS (s_e, pos, s_cnt, s_off):
// offsets; each pair's sorted_ids entry and the expert_ids entry of its block
// (every block of a segment holds at least one pair, so this covers every
// block; pairs of one block write the same value); and the sentinel pads,
// one item (e, j) per slot j < B after expert e's pairs, eight items per
// thread with their LDS reads issued together.
// Called by all NT threads of the workgroup.
template <int NT, typename PosPtr>
__device__ __forceinline__ void write_sort_outputs(const int* s_e, PosPtr pos, const int* s_cnt, const int* s_off,
                                                   int N, int B, int P, int32_t* sorted_ids, int32_t* expert_ids,
                                                   int32_t* offsets) {
  const int lb = __ffs(B) - 1;
  const int t = threadIdx.x;
  for (int e = t; e <= N; e += NT) offsets[e] = s_off[e];
  for (int p = t; p < P; p += NT) {
    const int q = pos[p];
    if (q >= 0) {
      sorted_ids[q] = p;
      expert_ids[q >> lb] = s_e[p];
    }
  }
  const int items = N << lb;
  for (int it0 = 0; it0 < items; it0 += 8 * NT) {
    int a[8], b[8], c[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = min((it0 + t + u * NT) >> lb, N - 1);
      a[u] = s_off[e];
      b[u] = s_off[e + 1];
      c[u] = s_cnt[e];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int it = it0 + t + u * NT;
      const int q = a[u] + c[u] + (it & (B - 1));
      if (it < items && q < b[u]) sorted_ids[q] = P;
    }
  }
}

// Pairs up to which one wave sorts alone (decode sizes: a few batches of 64);
// above, every wave of the workgroup takes a contiguous share.
constexpr int kWaveSortMaxP = 512;

// ---------------------------------------------------------------------------
// MX quantisation of 16 consecutive bf16 elements (two 16-byte loads). The
// partner lane (lane ^ 1) holds the other half of the 32-element block.
// MXFP8: the 16 e4m3 codes, packed little-endian in a uint4. MXFP4: the 16
// e2m1 codes two a byte (low nibble first) in .x and .y. Either way the
// block's scale byte goes to scale_byte. Must be called by both lanes of a
// pair.
// ---------------------------------------------------------------------------
__device__ __forceinline__ u32 block_amax16(const u32 (&w)[8]) {
  u32 amax = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const u32 lo = w[i] & 0x7fffu, hi = (w[i] >> 16) & 0x7fffu;
    amax = lo > amax ? lo : amax;
    amax = hi > amax ? hi : amax;
  }
  const u32 other = dpp_u32<kDppQuadXor1>(amax);  // partner lane (lane ^ 1)
  return other > amax ? other : amax;
}

__device__ __forceinline__ uint4 mx_quant16_regs(const uint4& a, const uint4& b, u32& scale_byte) {
  const u32 w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  const int se = mx_shared_exp(block_amax16(w));
  scale_byte = (u32)(se + 127);
  return make_uint4(e4m3x4_of_bf16(w[0], w[1], se), e4m3x4_of_bf16(w[2], w[3], se), e4m3x4_of_bf16(w[4], w[5], se),
                    e4m3x4_of_bf16(w[6], w[7], se));
}

__device__ __forceinline__ uint4 mx4_quant16_regs(const uint4& a, const uint4& b, u32& scale_byte) {
  const u32 w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  const int se = mx_shared_exp_e<2>(block_amax16(w));
  scale_byte = (u32)(se + 127);
  return make_uint4(e2m1x8_of_bf16(w[0], w[1], w[2], w[3], se), e2m1x8_of_bf16(w[4], w[5], w[6], w[7], se), 0u, 0u);
}

// fp4 is uniform across the wave (a launch argument).
__device__ __forceinline__ uint4 mx_quant16_fmt(const uint4& a, const uint4& b, u32& scale_byte, bool fp4) {
  return fp4 ? mx4_quant16_regs(a, b, scale_byte) : mx_quant16_regs(a, b, scale_byte);
}

__device__ __forceinline__ uint4 mx_quant16(const uint16_t* src, u32& scale_byte, bool fp4) {
  return mx_quant16_fmt(*reinterpret_cast<const uint4*>(src), *reinterpret_cast<const uint4*>(src + 8), scale_byte,
                        fp4);
}

// Units (16-element chunks) are numbered row-major, one per lane, so lanes
// 8q..8q+7 hold chunks 8c'..8c'+7 of one row (rows are multiples of 32
// chunks), i.e. the 4 scale bytes of blocks 4c'..4c'+3. The first lane of each
// group of 8 gathers them (DPP within the 16-lane row) into one 4-byte word.
// Called by every lane of the wave.
__device__ __forceinline__ u32 pack_scales(u32 sb) {
  const u32 s2 = dpp_row_shl<2>(sb), s4 = dpp_row_shl<4>(sb), s6 = dpp_row_shl<6>(sb);
  return (sb & 0xffu) | ((s2 & 0xffu) << 8) | ((s4 & 0xffu) << 16) | ((s6 & 0xffu) << 24);
}

// Store unit u's codes to the padded rows pos[t*k + j] of its token's pairs;
// lanes with u % 8 == 0 also store the packed scales of their 4 blocks. All
// KMAX >= k positions are read (clamped addresses, no branch between the
// reads) before the first store, so their latencies overlap. Row offsets are
// one 32 x 32 -> 64-bit product each. MXFP4 rows are K/2 bytes and a unit's
// codes 8 bytes.
template <int KMAX, bool FP4, typename PosPtr>
__device__ __forceinline__ void store_unit_kf(uint8_t* a_q, uint8_t* a_scale, int K, int k, int t, int c,
                                              PosPtr pos, const uint4& codes, u32 scales4) {
  const u32 row_bytes = FP4 ? (u32)K >> 1 : (u32)K;
  const u32 kscale = (u32)K >> 5;
  uint8_t* q_col = a_q + (FP4 ? 8 * c : 16 * c);
  uint8_t* s_col = a_scale + (c >> 1);
  const bool lead = (c & 7) == 0;
  int d[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) d[j] = pos[t * k + min(j, k - 1)];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (j < k && d[j] >= 0) {
      const u32 r = (u32)d[j];
      uint8_t* row = q_col + (uint64_t)r * row_bytes;
      if (FP4) *reinterpret_cast<uint2*>(row) = make_uint2(codes.x, codes.y);
      else *reinterpret_cast<uint4*>(row) = codes;
      if (lead) *reinterpret_cast<u32*>(s_col + (uint64_t)r * kscale) = scales4;
    }
  }
}

// cpr_magic: ceil(2^32 / (K/16)) for a multiply in place of the division of
// u by the chunks per row, or 0. fp4 is uniform across the wave.
template <typename PosPtr>
__device__ __forceinline__ void store_unit(uint8_t* a_q, uint8_t* a_scale, int K, int k, int u, PosPtr pos,
                                           const uint4& codes, u32 scales4, u32 cpr_magic, bool fp4) {
  const int cpr = K >> 4;  // 16-element chunks per row
  const int t = cpr_magic ? div_magic(u, cpr_magic) : u / cpr, c = u - t * cpr;
  if (fp4) {
    if (k <= 8) store_unit_kf<8, true>(a_q, a_scale, K, k, t, c, pos, codes, scales4);
    else if (k <= 16) store_unit_kf<16, true>(a_q, a_scale, K, k, t, c, pos, codes, scales4);
    else store_unit_kf<32, true>(a_q, a_scale, K, k, t, c, pos, codes, scales4);
  } else {
    if (k <= 8) store_unit_kf<8, false>(a_q, a_scale, K, k, t, c, pos, codes, scales4);
    else if (k <= 16) store_unit_kf<16, false>(a_q, a_scale, K, k, t, c, pos, codes, scales4);
    else store_unit_kf<32, false>(a_q, a_scale, K, k, t, c, pos, codes, scales4);
  }
}

}  // namespace rgt
