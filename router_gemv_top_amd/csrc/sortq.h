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

__device__ __forceinline__ int ceil_log2(int n) { return n <= 1 ? 0 : 32 - __clz(n - 1); }

// Block sizes are powers of two: round up / divide with masks and shifts (a
// GPU has no integer divide instruction; a runtime division costs ~40
// instructions).
__device__ __forceinline__ int pad_to(int c, int B) { return (c + B - 1) & -B; }
__device__ __forceinline__ int div_pow2(int a, int B) { return a >> (__ffs(B) - 1); }

// Exclusive scan of vals[0..n) in LDS (in place), n <= 4 * blockDim.x.
// Returns the total. Uses scratch[blockDim.x] of LDS.
__device__ __forceinline__ int block_exclusive_scan(int* vals, int n, int* scratch) {
  const int t = threadIdx.x, nt = blockDim.x;
  const int per = (n + nt - 1) / nt;
  const int b0 = min(n, t * per), b1 = min(n, b0 + per);
  int local = 0;
  for (int i = b0; i < b1; ++i) local += vals[i];
  scratch[t] = local;
  __syncthreads();
  // Hillis-Steele inclusive scan of the thread sums.
  for (int o = 1; o < nt; o <<= 1) {
    const int v = t >= o ? scratch[t - o] : 0;
    __syncthreads();
    scratch[t] += v;
    __syncthreads();
  }
  int run = scratch[t] - local;
  const int total = scratch[nt - 1];
  for (int i = b0; i < b1; ++i) {
    const int v = vals[i];
    vals[i] = run;
    run += v;
  }
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
                       int* s_scr, PosPtr pos) {
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
      pos[p] = s_off[e] + s_hist[wave * N + e] + rank;
    } else if (p < c1) {
      pos[p] = -1;
    }
    // Order the reads above before the leader's update (same wave, LDS is in order).
    if (valid && (peers & lanemask_lt()) == 0ull) s_hist[wave * N + e] += __popcll(peers);
  }
  __syncthreads();
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
template <typename PosPtr>
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
  // Padded counts -> exclusive segment offsets. Lane l owns C consecutive
  // experts (C <= 16); their counts are read once into registers.
  const int C = (N + 63) / 64;
  const int e0 = min(N, lane * C), e1 = min(N, e0 + C);
  int pc[16];
  int local = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    pc[i] = (i < C && e0 + i < e1) ? pad_to(s_cnt[e0 + i], B) : 0;
    local += pc[i];
  }
  const int incl = wave_inclusive_scan(local);
  const int total = (int)readlane_u32((u32)incl, 63);
  int run = incl - local;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if (i < C && e0 + i < e1) s_off[e0 + i] = run;
    run += pc[i];
  }
  if (lane == 0) s_off[N] = total;
  for (int p = lane; p < P; p += 64) {
    const int e = s_e[p];
    pos[p] = (unsigned)e < (unsigned)N ? s_off[e] + s_rank[p] : -1;
  }
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

// Decode-size sort: one workgroup (one wave sorts up to kWaveSortMaxP pairs,
// the whole workgroup above). pos goes to the workspace for the quant.
constexpr int kWaveSortMaxP = 2048;

__global__ void __launch_bounds__(256) sort_small_kernel(const int32_t* ids, int P, int N, int B,
                                                         int32_t* sorted_ids, int32_t* expert_ids,
                                                         int32_t* offsets, int32_t* pos_ws) {
  extern __shared__ int smem[];
  int* s_e = smem;
  int* s_hist = s_e + P;          // wave sort: per-pair ranks; workgroup sort: per-wave counts
  int* s_cnt = s_hist + (P > 4 * N ? P : 4 * N);
  int* s_off = s_cnt + N;
  int* s_scr = s_off + N + 1;
  if (P <= kWaveSortMaxP) {
    if (threadIdx.x < 64) wave_sort(ids, P, N, B, s_e, s_hist, s_cnt, s_off, pos_ws);
    vm_drain();
    __syncthreads();
  } else {
    wg_sort<false>(ids, P, N, B, s_e, s_hist, s_cnt, s_off, s_scr, pos_ws);
  }
  for (int p = threadIdx.x; p < P; p += blockDim.x) {
    const int q = pos_ws[p];
    if (q >= 0) sorted_ids[q] = p;
  }
  write_sort_layout(s_cnt, s_off, N, B, P, sorted_ids, expert_ids, offsets);
}

// ---------------------------------------------------------------------------
// Large-P sort: per-workgroup histograms -> one scan workgroup -> scatter.
// Workgroup g owns pairs [g*chunk, (g+1)*chunk).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) sort_hist_kernel(const int32_t* ids, int P, int N, int chunk, int32_t* ghist) {
  extern __shared__ int s_h[];
  for (int e = threadIdx.x; e < N; e += blockDim.x) s_h[e] = 0;
  __syncthreads();
  const int p0 = blockIdx.x * chunk, p1 = min(P, p0 + chunk);
  for (int p = p0 + threadIdx.x; p < p1; p += blockDim.x) {
    const int e = ids[p];
    if ((unsigned)e < (unsigned)N) atomicAdd(&s_h[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < N; e += blockDim.x) ghist[(int64_t)blockIdx.x * N + e] = s_h[e];
}

__global__ void __launch_bounds__(1024) sort_scan_kernel(int32_t* ghist, int G, int P, int N, int B,
                                                         int32_t* sorted_ids, int32_t* expert_ids,
                                                         int32_t* offsets, int32_t* off_ws) {
  extern __shared__ int smem[];
  int* s_cnt = smem;
  int* s_off = s_cnt + N;
  int* s_scr = s_off + N + 1;
  for (int e = threadIdx.x; e < N; e += blockDim.x) {
    int run = 0;
    for (int g = 0; g < G; ++g) {
      const int c = ghist[(int64_t)g * N + e];
      ghist[(int64_t)g * N + e] = run;
      run += c;
    }
    s_cnt[e] = run;
    s_off[e] = pad_to(run, B);
  }
  __syncthreads();
  const int total = block_exclusive_scan(s_off, N, s_scr);
  if (threadIdx.x == 0) s_off[N] = total;
  __syncthreads();
  for (int e = threadIdx.x; e <= N; e += blockDim.x) off_ws[e] = s_off[e];
  write_sort_layout(s_cnt, s_off, N, B, P, sorted_ids, expert_ids, offsets);
}

__global__ void __launch_bounds__(256) sort_scatter_kernel(const int32_t* ids, int P, int N, int chunk,
                                                           const int32_t* ghist, const int32_t* off_ws,
                                                           int32_t* sorted_ids, int32_t* pos_ws) {
  extern __shared__ int smem[];
  int* s_hist = smem;            // [4][N] per-wave counts -> bases
  int* s_base = s_hist + 4 * N;  // [N] offsets + this workgroup's global base
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int p0 = blockIdx.x * chunk, p1 = min(P, p0 + chunk);
  for (int i = t; i < 4 * N; i += blockDim.x) s_hist[i] = 0;
  for (int e = t; e < N; e += blockDim.x) s_base[e] = off_ws[e] + ghist[(int64_t)blockIdx.x * N + e];
  __syncthreads();
  const int sub = ((p1 - p0 + 3) / 4 + 63) & ~63;
  const int c0 = min(p1, p0 + wave * sub), c1 = min(p1, c0 + sub);
  for (int p = c0 + lane; p < c1; p += 64) {
    const int e = ids[p];
    if ((unsigned)e < (unsigned)N) atomicAdd(&s_hist[wave * N + e], 1);
  }
  __syncthreads();
  for (int e = t; e < N; e += blockDim.x) {
    int run = 0;
    for (int w = 0; w < 4; ++w) {
      const int c = s_hist[w * N + e];
      s_hist[w * N + e] = run;
      run += c;
    }
  }
  __syncthreads();
  const int bits = ceil_log2(N);
  for (int base = c0; base < c1; base += 64) {
    const int p = base + lane;
    const int e = p < c1 ? ids[p] : 0;
    const bool valid = p < c1 && (unsigned)e < (unsigned)N;
    const u64 peers = match_peers(e, valid, bits);
    if (valid) {
      const int q = s_base[e] + s_hist[wave * N + e] + __popcll(peers & lanemask_lt());
      pos_ws[p] = q;
      sorted_ids[q] = p;
    } else if (p < c1) {
      pos_ws[p] = -1;
    }
    if (valid && (peers & lanemask_lt()) == 0ull) s_hist[wave * N + e] += __popcll(peers);
  }
}

// ---------------------------------------------------------------------------
// MXFP8 of 16 consecutive bf16 elements (two 16-byte loads). The partner lane
// (lane ^ 1) holds the other half of the 32-element block. Returns the 16
// codes packed little-endian in a uint4 and the block's scale byte.
// Must be called by both lanes of a pair.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint4 mx_quant16(const uint16_t* src, u32& scale_byte) {
  const uint4 a = *reinterpret_cast<const uint4*>(src);
  const uint4 b = *reinterpret_cast<const uint4*>(src + 8);
  const u32 w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  u32 amax = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const u32 lo = w[i] & 0x7fffu, hi = (w[i] >> 16) & 0x7fffu;
    amax = lo > amax ? lo : amax;
    amax = hi > amax ? hi : amax;
  }
  const u32 other = dpp_u32<kDppQuadXor1>(amax);  // partner lane (lane ^ 1)
  amax = other > amax ? other : amax;
  const int se = mx_shared_exp(amax);
  scale_byte = (u32)(se + 127);
  u32 c[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const u32 w0 = w[2 * q], w1 = w[2 * q + 1];
    c[q] = e4m3_of_bf16(w0 & 0xffffu, se) | (e4m3_of_bf16(w0 >> 16, se) << 8) |
           (e4m3_of_bf16(w1 & 0xffffu, se) << 16) | (e4m3_of_bf16(w1 >> 16, se) << 24);
  }
  return make_uint4(c[0], c[1], c[2], c[3]);
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

// Store unit u's 16 codes to the padded rows pos[t*k + j] of its token's pairs;
// lanes with u % 8 == 0 also store the packed scales of their 4 blocks.
template <typename PosPtr>
__device__ __forceinline__ void store_unit(uint8_t* a_q, uint8_t* a_scale, int K, int k, int u, PosPtr pos,
                                           const uint4& codes, u32 scales4) {
  const int cpr = K >> 4;  // 16-element chunks per row
  const int t = u / cpr, c = u - t * cpr;
  const int64_t kscale = K >> 5;
  for (int j = 0; j < k; ++j) {
    const int64_t d = pos[t * k + j];
    if (d < 0) continue;
    *reinterpret_cast<uint4*>(a_q + d * K + 16 * c) = codes;
    if ((c & 7) == 0) *reinterpret_cast<u32*>(a_scale + d * kscale + (c >> 1)) = scales4;
  }
}

__global__ void __launch_bounds__(256) quant_kernel(const uint16_t* x, int64_t ldx, int M, int K, int k,
                                                    const int32_t* pos, uint8_t* a_q, uint8_t* a_scale) {
  const int units = M * (K >> 4);
  const int u = blockIdx.x * blockDim.x + threadIdx.x;
  const int cpr = K >> 4;
  // Units come in whole groups of 8 lanes (unit counts are multiples of 32),
  // so every lane of a pair or group is active together.
  u32 sb = 0;
  uint4 codes = make_uint4(0, 0, 0, 0);
  if (u < units) codes = mx_quant16(x + (int64_t)(u / cpr) * ldx + 16 * (u % cpr), sb);
  const u32 s4 = pack_scales(sb);
  if (u < units) store_unit(a_q, a_scale, K, k, u, pos, codes, s4);
}

}  // namespace rgt
