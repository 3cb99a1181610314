// sortq_kernels.h - the standalone sort and quant launches (the chain used
// by rgt_moe_sort_quant and by rgt_route_sort_quant outside the one-launch
// range). Included by the host translation unit only: the fused kernel's
// translation units share the device helpers of sortq.h, not these kernels.
#pragma once

#include "sortq.h"

namespace rgt {

// Sort of up to a few thousand pairs in one workgroup: one wave when launched
// with 256 threads (the host does so for small P, at most kWaveSortMaxP),
// every wave of the workgroup when launched with 1024 (each wave walks a
// sixteenth of the pairs in 64-pair batches); the pair positions go to pos_ws
// for the quant.
__global__ void __launch_bounds__(1024) sort_small_kernel(const int32_t* ids, int P, int N, int B,
                                                          int32_t* sorted_ids, int32_t* expert_ids,
                                                          int32_t* offsets, int32_t* pos_ws) {
  extern __shared__ int smem[];
  const int nw = blockDim.x >> 6;
  int* s_e = smem;
  int* s_hist = s_e + P;          // wave sort: per-pair ranks; workgroup sort: per-wave counts
  int* s_cnt = s_hist + (P > nw * N ? P : nw * N);
  int* s_off = s_cnt + N;
  int* s_scr = s_off + N + 1;
  if (blockDim.x == 256) {
    if (threadIdx.x < 64) wave_sort<16>(ids, P, N, B, s_e, s_hist, s_cnt, s_off, pos_ws);
    vm_drain();
    __syncthreads();
    for (int p = threadIdx.x; p < P; p += blockDim.x) {
      const int q = pos_ws[p];
      if (q >= 0) sorted_ids[q] = p;
    }
    write_sort_layout(s_cnt, s_off, N, B, P, sorted_ids, expert_ids, offsets);
  } else {
    // Every wave (launched with 1024 threads): the pairs' sorted_ids entries
    // go out as their positions are found, the pads and expert_ids one item
    // per (expert, slot) from consecutive lanes.
    wg_sort<false>(ids, P, N, B, s_e, s_hist, s_cnt, s_off, s_scr, pos_ws, sorted_ids);
    write_layout<1024>(s_cnt, s_off, N, B, P, 0, N, sorted_ids, expert_ids, offsets);
  }
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

// Per-group bases of the large sort: for every expert, an exclusive prefix
// of its counts over the G groups (in place in ghist) and its total (to
// cnt[e]). Workgroup b takes experts [64b, 64b + 64) (lane = expert) with
// sixteen waves; wave w takes a sixteenth of the groups, and the sixteen parts
// are joined through LDS. Loads go 8 at a time so their latencies overlap
// (at the prefill size each lane walks 16 groups: two batches a pass).
constexpr int kColscanWaves = 16;
__global__ void __launch_bounds__(1024) sort_colscan_kernel(int32_t* ghist, int G, int N, int32_t* cnt) {
  __shared__ int s_part[kColscanWaves][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int e = blockIdx.x * 64 + lane;
  const int ec = min(e, N - 1);
  const int gq = (G + kColscanWaves - 1) / kColscanWaves, g0 = min(G, wave * gq), g1 = min(G, g0 + gq);
  int sum = 0;
  for (int g = g0; g < g1; g += 8) {
    int v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = ghist[(int64_t)min(g + j, g1 - 1) * N + ec];
#pragma unroll
    for (int j = 0; j < 8; ++j) sum += g + j < g1 ? v[j] : 0;
  }
  s_part[wave][lane] = sum;
  __syncthreads();
  int run = 0;
  for (int w = 0; w < wave; ++w) run += s_part[w][lane];
  if (wave == 0 && e < N) {
    int total = 0;
    for (int w = 0; w < kColscanWaves; ++w) total += s_part[w][lane];
    cnt[e] = total;
  }
  if (e >= N) return;
  for (int g = g0; g < g1; g += 8) {
    int v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = ghist[(int64_t)min(g + j, g1 - 1) * N + e];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (g + j < g1) {
        ghist[(int64_t)(g + j) * N + e] = run;
        run += v[j];
      }
  }
}

// Padded offsets of the large sort from the per-expert totals in off_ws:
// off_ws[0..N] becomes the offsets and off_ws[N+1+e] keeps the count of
// expert e, for the scatter workgroups that write the layout.
__global__ void __launch_bounds__(1024) sort_scan_kernel(int N, int B, int32_t* off_ws) {
  extern __shared__ int smem[];
  int* s_off = smem;
  int* s_scr = s_off + N + 1;
  for (int e = threadIdx.x; e < N; e += blockDim.x) {
    const int c = off_ws[e];
    off_ws[N + 1 + e] = c;
    s_off[e] = pad_to(c, B);
  }
  __syncthreads();
  const int total = block_exclusive_scan(s_off, N, s_scr);
  if (threadIdx.x == 0) s_off[N] = total;
  __syncthreads();
  for (int e = threadIdx.x; e <= N; e += blockDim.x) off_ws[e] = s_off[e];
}

// Workgroup g scatters the pairs [g*chunk, (g+1)*chunk) to their padded
// positions, then writes the layout (offsets, expert_ids, pads) of its slice
// of ceil(N / gridDim.x) experts, so that work is spread over the grid with
// each expert's pads stored by consecutive lanes.
__global__ void __launch_bounds__(256) sort_scatter_kernel(const int32_t* ids, int P, int N, int B, int chunk,
                                                           const int32_t* ghist, const int32_t* off_ws,
                                                           int32_t* sorted_ids, int32_t* expert_ids,
                                                           int32_t* offsets, int32_t* pos_ws) {
  extern __shared__ int smem[];
  int* s_hist = smem;            // [4][N] per-wave counts -> bases
  int* s_base = s_hist + 4 * N;  // [N] offsets + this workgroup's global base
  int* s_off = s_base + N;       // [N+1] offsets of the layout slice
  int* s_cnt = s_off + N + 1;    // [N] counts of the layout slice
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int p0 = blockIdx.x * chunk, p1 = min(P, p0 + chunk);
  const int ls = (N + (int)gridDim.x - 1) / (int)gridDim.x;
  const int e0 = min(N, (int)blockIdx.x * ls), e1 = min(N, e0 + ls);
  for (int i = t; i < 4 * N; i += blockDim.x) s_hist[i] = 0;
  for (int e = t; e < N; e += blockDim.x) s_base[e] = off_ws[e] + ghist[(int64_t)blockIdx.x * N + e];
  for (int e = e0 + t; e <= e1; e += blockDim.x) {
    s_off[e] = off_ws[e];
    if (e < e1) s_cnt[e] = off_ws[N + 1 + e];
  }
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
  if (e0 < e1) write_layout<256>(s_cnt, s_off, N, B, P, e0, e1, sorted_ids, expert_ids, offsets);
}

// fp4: MXFP4 rows (K/2 bytes of packed e2m1 codes), else MXFP8.
__global__ void __launch_bounds__(256) quant_kernel(const uint16_t* x, int64_t ldx, int M, int K, int k,
                                                    const int32_t* pos, uint8_t* a_q, uint8_t* a_scale, int fp4) {
  const int units = M * (K >> 4);
  const int u = blockIdx.x * blockDim.x + threadIdx.x;
  const int cpr = K >> 4;
  // Units come in whole groups of 8 lanes (unit counts are multiples of 32),
  // so every lane of a pair or group is active together.
  u32 sb = 0;
  uint4 codes = make_uint4(0, 0, 0, 0);
  if (u < units) codes = mx_quant16(x + (int64_t)(u / cpr) * ldx + 16 * (u % cpr), sb, fp4 != 0);
  const u32 s4 = pack_scales(sb);
  if (u < units) store_unit(a_q, a_scale, K, k, u, pos, codes, s4, 0u, fp4 != 0);
}

}  // namespace rgt
