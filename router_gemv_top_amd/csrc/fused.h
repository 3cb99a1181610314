// fused.h - the whole decode front-end in one launch (M <= 64).
//
// The pages run the router, the gate and the sort of a decode step as one
// launch (MiniMax-M3.1-Flash MoE/GEMM kernels, Summary: Router; Kimi-K3 fused
// routing, sort, quant, Motivation). On gfx950 each hand-off between
// workgroups costs a device-coherent memory round trip (about a microsecond),
// so the chain below has as few of them as possible:
//
//   1. every workgroup computes one split-K GEMV tile and publishes its fp32
//      partials as tagged words. The split-K fixup ("MiniMax-M3: Triton
//      split-K router GEMV with in-kernel split-K fixup", opening summary) is
//      done by the consumers of the logits themselves: they poll the partials
//      of their rows and sum them in k-slice order, which gives the same bits
//      as the last-arriver fixup of the standalone router;
//   2. the softmax top-k gate. Small mode (all rows' partials fit one poll
//      per thread): every workgroup that owns a quant chunk, the layout
//      workgroup and the gate workgroup gather every row and run the gate
//      themselves, so no further hand-off is needed. Large mode: workgroup r
//      gathers row r, runs its gate and publishes the ids as tagged words,
//      which the others poll;
//   3. the same workgroups sort the M*k pairs in LDS with one wave (tiny at
//      decode sizes, so redundant sorting beats another hand-off) and store
//      their MXFP8 or MXFP4 chunk (quantised in registers while waiting) to
//      the padded rows of the token's pairs and their sorted_ids entries;
//      the layout workgroup writes offsets, expert_ids and the pads.
//
// topk_ids, topk_w and the logits come from the gate workgroup in small mode
// (the first one past the layout workgroup, so the fp64 weights stay off the
// path of the workgroups that store; workgroup 0 if the grid has no spare)
// and from workgroup r for row r in large mode.
//
// A tagged word is a 32-bit payload plus the tag (epoch + 1) of the call that
// wrote it, stored as one 8-byte store; readers poll the words themselves, so
// no hand-off needs a counter. Every wave reads the epoch before it loads its
// tile; the gate workgroup advances it only after it has seen every partial
// (small mode), workgroup 0 only after every id (large mode), which implies
// that every wave has read it.
// Every wait is bounded by a deadline that sets the workspace error word.
#pragma once

#include "device.h"
#include "gate.h"
#include "gemv.h"
#include "sortq.h"

namespace rgt {

// Control words at the head of the workspace, 128 bytes apart.
enum : int { kCtlErr = 0, kCtlEpoch = kCtrStride };

// LDS of the tail, in ints: s_e[P], s_key[P], s_pos[64], s_cnt[N], s_pre[N],
// s_off[N+1], then the gathered logits (16-byte aligned).
__host__ __device__ constexpr int fused_log_offset(int P, int n) { return (2 * P + 64 + 3 * n + 1 + 3) & ~3; }
__host__ __device__ constexpr int fused_tail_ints(int P, int n, int rows) { return fused_log_offset(P, n) + rows * n; }

// Positions of a workgroup's own pairs, indexed by pair number.
struct OffsetPos {
  const int* s_pos;
  int p0;
  __device__ __forceinline__ int operator[](int p) const { return s_pos[p - p0]; }
};

struct FusedArgs {
  GemvArgs g;          // g.logits, g.part and g.ctr unused here
  const float* bias;   // [N] or null
  int topk, block;
  int small;           // 1: small mode, 0: large mode (chosen by the host)
  int fp4;             // 1: MXFP4 rows (K/2 bytes of packed e2m1 codes), 0: MXFP8
  int upw_log;         // log2 of the quant units per quant workgroup (6, 7 or 8)
  u32 cpr_magic;       // ceil(2^32 / (K/16)): token of a quant unit by multiplication
  float* logits_out;   // [M][N] or null
  int32_t* topk_ids;
  float* topk_w;
  int32_t* sorted_ids;
  int32_t* expert_ids;
  int32_t* offsets;
  uint8_t* a_q;
  uint8_t* a_scale;
  u32* ctl;
  u64* tpart;          // [S][M][N] tagged partials (workspace)
  u64* tids;           // [M*topk] tagged expert ids (workspace, padded to 16 bytes)
  u64 budget;          // deadline of each wait, in 100 MHz ticks
  int fault_skip;      // host-forced fault: 1 = no partial is ever published
  u64* trace;          // phase stamps (trace build only), 16 per workgroup
};

// The call's tag, read by every wave on its own (no barrier): epoch + 1,
// skipping 0 so zero-filled words never look ready. It stays a per-lane
// value (every lane loads the same word): moving it to a scalar register
// would make the wave wait for this load before issuing the tile's loads.
__device__ __forceinline__ u32 call_tag(const u32* ctl) {
  const u32 t = ld_agent(ctl + kCtlEpoch) + 1u;
  return t ? t : 1u;
}

__device__ __forceinline__ void set_timeout(const FusedArgs& a) { or_agent(a.ctl + kCtlErr, kErrTimeout); }

// 16-byte loads one thread keeps in flight per poll.
constexpr int kPollLoads = 16;

// The workgroup gathers rows [r0, r0 + rows) of the logits from the tagged
// partials into s_log[(row - r0) * n + col]. An item is one column pair of
// one row: item it of the gathered rows sits at byte 16*it of every k-slice
// and lands at s_log[2*it]. Thread t takes items t, t + 256, ... and their S
// slices, nl <= NL loads in all (a thread with fewer items repeats its last
// one). Each thread polls its own loads until every word carries the tag,
// re-issuing them as soon as they return short of it (one poll in flight: a
// second poll issued with the first sees the same memory state, and the loads
// it leaves in flight at the exit cost a wait at the next register reuse),
// then sums each item's slices in k-slice order. Returns false (error word
// set) if the deadline passes.
template <int NL>
__device__ __forceinline__ bool gather_logits(const FusedArgs& a, int r0, int rows, u32 tag, float* s_log) {
  __shared__ u32 s_bad;
  const int n = a.g.n, S = a.g.s_count;
  const int items = rows * (n >> 1);
  const u32 slice = (u32)a.g.m * (u32)n * 8u;
  const u32 row_base = (u32)r0 * (u32)n * 8u;
  const int t = threadIdx.x;
  if (t == 0) s_bad = 0u;
  __syncthreads();
  if (t < items) {
    const auto rsrc = coherent_rsrc(a.tpart, slice * (u32)S);
    u32 off[NL];
    {
      int it = t, s = 0;
#pragma unroll
      for (int l = 0; l < NL; ++l) {
        off[l] = row_base + 16u * (u32)it + (u32)s * slice;
        if (++s == S) {
          s = 0;
          if (it + 256 < items) it += 256;
        }
      }
    }
    auto issue = [&](u32x4_t (&v)[NL]) {
#pragma unroll
      for (int l = 0; l < NL; ++l) v[l] = ld_agent16(rsrc, off[l]);
    };
    auto ready = [&](const u32x4_t (&v)[NL]) {
      bool ok = true;
#pragma unroll
      for (int l = 0; l < NL; ++l) ok = ok & (v[l].y == tag) & (v[l].w == tag);
      return ok;
    };
    auto take = [&](const u32x4_t (&v)[NL]) {
      int s = 0, it = t;
      float2 acc = make_float2(0.f, 0.f);
#pragma unroll
      for (int l = 0; l < NL; ++l) {
        acc.x += __uint_as_float(v[l].x);
        acc.y += __uint_as_float(v[l].z);
        if (++s == S) {
          if (it < items) *reinterpret_cast<float2*>(s_log + 2 * it) = acc;
          acc = make_float2(0.f, 0.f);
          s = 0;
          it += 256;
        }
      }
    };
    const u64 t0 = rt_clock();
    u32x4_t va[NL];
    issue(va);
#ifdef RGT_TRACE
    int polls = 0;
#endif
    for (;;) {
#ifdef RGT_TRACE
      ++polls;
#endif
      if (ready(va)) { take(va); break; }
      issue(va);
      if (rt_clock() - t0 > a.budget) {
        set_timeout(a);
        s_bad = 1u;
        break;
      }
    }
#ifdef RGT_TRACE
    if (t == 0 && a.trace) {  // poll rounds and the gather's start time
      a.trace[blockIdx.x * 16 + 10] = (u64)polls;
      a.trace[blockIdx.x * 16 + 11] = t0;
    }
#endif
  }
  __syncthreads();
  return s_bad == 0u;
}

// Loads per thread that a gather of `rows` rows needs.
__host__ __device__ constexpr int gather_loads(int rows, int n, int s) { return (rows * (n / 2) + 255) / 256 * s; }

__device__ __forceinline__ bool gather_any(const FusedArgs& a, int r0, int rows, u32 tag, float* s_log) {
  const int nl = gather_loads(rows, a.g.n, a.g.s_count);
  if (nl <= 4) return gather_logits<4>(a, r0, rows, tag, s_log);
  if (nl <= 8) return gather_logits<8>(a, r0, rows, tag, s_log);
  return gather_logits<kPollLoads>(a, r0, rows, tag, s_log);
}

// The workgroup polls the P tagged ids (16-byte loads, two words each; thread
// t takes word pairs t, t + 256, ...) until every word carries the tag, then
// leaves the experts in s_e.
template <int NL>
__device__ __forceinline__ bool poll_ids(const FusedArgs& a, int P, u32 tag, int* s_e, int p0, int* s_cnt,
                                         int* s_pre) {
  __shared__ u32 s_bad;
  const int t = threadIdx.x;
  const int pairs = (P + 1) >> 1;
  if (t == 0) s_bad = 0u;
  __syncthreads();
  if (t < pairs) {
    const auto rsrc = coherent_rsrc(a.tids, (u32)pairs * 16u);
    auto pair_of = [&](int l) { return min(t + 256 * l, pairs - 1); };
    auto issue = [&](u32x4_t (&v)[NL]) {
#pragma unroll
      for (int l = 0; l < NL; ++l) v[l] = ld_agent16(rsrc, (u32)pair_of(l) * 16u);
    };
    auto ready = [&](const u32x4_t (&v)[NL]) {
      bool ok = true;
#pragma unroll
      for (int l = 0; l < NL; ++l) ok = ok & (v[l].y == tag) & ((2 * pair_of(l) + 1 >= P) | (v[l].w == tag));
      return ok;
    };
    auto take = [&](const u32x4_t (&v)[NL]) {
#pragma unroll
      for (int l = 0; l < NL; ++l) {
        const int q = t + 256 * l;
        if (q < pairs) {
          s_e[2 * q] = (int)v[l].x;
          hist_add((int)v[l].x, 2 * q, p0, a.g.n, s_cnt, s_pre);
          if (2 * q + 1 < P) {
            s_e[2 * q + 1] = (int)v[l].z;
            hist_add((int)v[l].z, 2 * q + 1, p0, a.g.n, s_cnt, s_pre);
          }
        }
      }
    };
    const u64 t0 = rt_clock();
    u32x4_t va[NL];
    issue(va);
    for (;;) {
      if (ready(va)) { take(va); break; }
      issue(va);
      if (rt_clock() - t0 > a.budget) {
        set_timeout(a);
        s_bad = 1u;
        break;
      }
    }
  }
  __syncthreads();
  return s_bad == 0u;
}

__device__ __forceinline__ bool poll_ids_any(const FusedArgs& a, int P, u32 tag, int* s_e, int p0, int* s_cnt,
                                             int* s_pre) {
  if (P <= 512) return poll_ids<1>(a, P, tag, s_e, p0, s_cnt, s_pre);
  return poll_ids<4>(a, P, tag, s_e, p0, s_cnt, s_pre);
}

// One wave selects the top-k of R rows held in LDS (lane-major loads);
// rows[r] is the row's logits.
template <int NV, int R>
__device__ __forceinline__ void row_select(const FusedArgs& a, const float* const (&rows)[R], int (&id)[R],
                                           u32 (&key)[R]) {
  __shared__ __align__(16) int s_slot[4][64 * R];
  const int n = a.g.n, c0 = lane_id() * NV;
  float sv[R][NV];
#pragma unroll
  for (int r = 0; r < R; ++r) {
#pragma unroll
    for (int i = 0; i < NV; ++i) sv[r][i] = rows[r][min(c0 + i, n - 1)];
    add_bias<NV>(sv[r], a.bias, n);
  }
  wave_select_rows<NV, R>(sv, n, a.topk, id, key, s_slot[threadIdx.x >> 6]);
}

// Workgroup 0 of small mode: the weights of rows r0, r0 + step, ... from the
// selected keys in s_key (one wave per row at a time).
__device__ __forceinline__ void rows_weights(const FusedArgs& a, const u32* s_key, int r0, int step) {
  const int k = a.topk, lane = lane_id();
  for (int row = r0; row < a.g.m; row += step) {
    const float w = wave_weights(s_key[row * k + min(lane, k - 1)], k);
    if (lane < k) a.topk_w[row * k + lane] = w;
  }
}

template <int NV>
__device__ __forceinline__ void fused_tail(const FusedArgs& a, int* smem, u32 tag, bool have_unit, int unit,
                                           const uint4& codes_in, u32 sb_in) {
  const GemvArgs& g = a.g;
  const int m = g.m, n = g.n, k = a.topk;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int units = m * (g.k >> 4);
  // Layout workgroups (one per 256 experts, after the last one with quant
  // units if the grid has room) write offsets, expert_ids and pads.
  const int n_layout = (n + 255) >> 8;
  const int layout_wg = min((int)gridDim.x - n_layout, ((units - 1) >> a.upw_log) + 1);
  const int li = (int)blockIdx.x - layout_wg;  // this workgroup's layout share, if 0 <= li < n_layout
  // Small mode: the gate workgroup (topk_ids, topk_w, logits, epoch) is the
  // first one past the layout workgroups if the grid has it, else 0.
  const int q_wgs = ((units - 1) >> a.upw_log) + 1;
  const int gate_wg = (a.small && layout_wg + n_layout < (int)gridDim.x) ? layout_wg + n_layout : 0;
  const bool gate_here = (int)blockIdx.x == gate_wg;
  const bool quant_wg = (int)blockIdx.x < q_wgs;
  const bool participant = gate_here || quant_wg || (li >= 0 && li < n_layout);
  const int P = m * k;
  int* s_e = smem;
  u32* s_key = reinterpret_cast<u32*>(s_e + P);
  int* s_pos = s_e + 2 * P;   // 64 entries
  int* s_cnt = s_pos + 64;
  int* s_pre = s_cnt + n;
  int* s_off = s_pre + n;
  float* s_log = reinterpret_cast<float*>(smem + fused_log_offset(P, n));
  // This workgroup's tokens (those its quant units touch) and their pairs.
  const int cpr = g.k >> 4;
  const int u0 = (int)blockIdx.x << a.upw_log;
  const int t0 = min(m, div_magic(u0, a.cpr_magic)), t1 = min(m, div_magic(u0 + (1 << a.upw_log) - 1, a.cpr_magic) + 1);
  const int p0 = u0 < units ? t0 * k : 0, p1 = u0 < units ? t1 * k : 0;
  // The expert histograms are filled as the ids become known (zeroed here;
  // the barriers of the gather or of the id poll come before any add).
  if (participant)
    for (int e = threadIdx.x; e < n; e += 256) {
      s_cnt[e] = 0;
      s_pre[e] = 0;
    }
  if (a.small) {
    // Step 2 (small): each participant gathers every row and runs every gate;
    // wave w takes rows w, w + 4, ...
    if (!participant) return;
    if (!gather_any(a, 0, m, tag, s_log)) return;
    RGT_STAMP(a.trace, 5);
    // (The weights only feed topk_w: workgroup 0 computes them off the
    // sort-and-store path, below.)
    auto keep = [&](int row, int id, u32 key) {
      if (lane < k) {
        s_e[row * k + lane] = id;
        s_key[row * k + lane] = key;
        hist_add(id, row * k + lane, p0, n, s_cnt, s_pre);
        if (gate_here) a.topk_ids[row * k + lane] = id;
      }
    };
    for (int row = wave; row < m; row += 4) {
      const float* rows[1] = {s_log + row * n};
      int id[1];
      u32 key[1];
      row_select<NV, 1>(a, rows, id, key);
      keep(row, id[0], key[0]);
    }
    if (gate_here && a.logits_out)
      for (int i = threadIdx.x; i < m * n; i += 256) a.logits_out[i] = s_log[i];
    __syncthreads();
    if (gate_here && gate_wg != 0) {
      // Every partial has been seen, so every wave has read the epoch.
      if (threadIdx.x == 0) st_agent(a.ctl + kCtlEpoch, tag);
      rows_weights(a, s_key, wave, 4);
      return;
    }
    RGT_STAMP(a.trace, 6);
  } else {
    // Step 2 (large): workgroup r gathers row r, runs its gate and publishes
    // the ids; then every participant polls all ids.
    if ((int)blockIdx.x < m) {
      const int row = blockIdx.x;
      if (!gather_any(a, row, 1, tag, s_log)) return;
      RGT_STAMP(a.trace, 5);
      if (wave == 0) {
        const float* rows[1] = {s_log};
        int ids[1];
        u32 keys[1];
        row_select<NV, 1>(a, rows, ids, keys);
        const int id = ids[0];
        const u32 key = keys[0];
        if (lane < k) {
          st_agent(a.tids + row * k + lane, tag_word((u32)id, tag));
          a.topk_ids[row * k + lane] = id;
        }
        const float w = wave_weights(key, k);  // after the ids are published
        if (lane < k) a.topk_w[row * k + lane] = w;
      }
      if (a.logits_out)
        for (int i = threadIdx.x; i < n; i += 256) a.logits_out[(int64_t)row * n + i] = s_log[i];
      RGT_STAMP(a.trace, 6);
    }
    if (!participant) return;
    if (!poll_ids_any(a, P, tag, s_e, p0, s_cnt, s_pre)) return;
  }
  RGT_STAMP(a.trace, 7);
  // Every wave of the grid has read the epoch (see the top of this file):
  // advance it for the next call (large mode, or small mode without a spare
  // gate workgroup).
  if (gate_here && threadIdx.x == 0) st_agent(a.ctl + kCtlEpoch, tag);
  // Step 3: positions of the pairs of this workgroup's tokens (a counting
  // sort from the expert histogram), then the workgroup stores its quantised
  // chunk to the padded rows of those pairs. The token's pairs' sorted_ids
  // entries are written by the workgroup holding its first quant unit; the
  // layout workgroup writes offsets, expert_ids and the pads.
  if (threadIdx.x < 64) pair_positions<NV>(P, n, a.block, p0, p1, s_e, s_cnt, s_pre, s_off, s_pos);
  else if (a.small && gate_here) rows_weights(a, s_key, wave - 1, 3);  // while wave 0 works
  __syncthreads();
  RGT_STAMP(a.trace, 8);
  if (li >= 0 && li < n_layout)
    write_layout<256>(s_cnt, s_off, n, a.block, P, li << 8, min(n, (li + 1) << 8), a.sorted_ids, a.expert_ids,
                      a.offsets);
  if ((int)threadIdx.x < p1 - p0) {
    const int p = p0 + threadIdx.x, q = s_pos[threadIdx.x];
    const int tok = p / k;
    if (q >= 0 && (tok * cpr) >> a.upw_log == (int)blockIdx.x) a.sorted_ids[q] = p;
  }
  const u32 scales4 = pack_scales(sb_in);  // all lanes: DPP reads neighbouring lanes
  if (have_unit) store_unit(a.a_q, a.a_scale, g.k, k, unit, OffsetPos{s_pos, p0}, codes_in, scales4, a.cpr_magic,
                             a.fp4 != 0);
  RGT_STAMP(a.trace, 9);
}

// Shared head of both kernels: read the tag, run the tile, quantise, then the
// tail. tile(nb, s, sink) computes this workgroup's GEMV tile.
template <int NV, class Tile>
__device__ __forceinline__ void fused_body(const FusedArgs& a, int* smem, Tile tile) {
  const GemvArgs& g = a.g;
  const int units = g.m * (g.k >> 4);
  const int unit = ((int)blockIdx.x << a.upw_log) + threadIdx.x;
  const bool have_unit = (int)threadIdx.x < (1 << a.upw_log) && unit < units;
  const int tile_id = xcd_tile(blockIdx.x, gridDim.x);
  RGT_STAMP(a.trace, 0);
  // Right after the tile's W loads are issued: the call's tag (loads return
  // in order, so issued earlier it would hold up the tile's arithmetic) and
  // the thread's quant chunk of x, quantised once the tile is done.
  u32 tag = 0;
  uint4 xa = make_uint4(0, 0, 0, 0), xb = make_uint4(0, 0, 0, 0);
  auto prefetch = [&]() {
    tag = call_tag(a.ctl);
    if (have_unit) {
      const int cpr = g.k >> 4, t = div_magic(unit, a.cpr_magic), c = unit - t * cpr;
      const u16* src = g.x + (int64_t)t * g.ldx + 16 * c;
      xa = ld16(src);
      xb = ld16(src + 8);
    }
  };
  tile(tile_id, [&](int s, int row, int col, float v) {
    if (!a.fault_skip) st_agent(a.tpart + ((int64_t)s * g.m + row) * g.n + col, tag_word(__float_as_uint(v), tag));
  }, prefetch);
  RGT_STAMP(a.trace, 1);
  u32 sb = 0;
  const uint4 codes = mx_quant16_fmt(xa, xb, sb, a.fp4 != 0);  // all lanes: the scale exchange reads the partner lane
  __syncthreads();  // the tile's LDS is reused below
  RGT_STAMP(a.trace, 4);
  fused_tail<NV>(a, smem, tag, have_unit, unit, codes, sb);
}

// Quant units (16-element chunks of x, row-major) go 2^upw_log to a
// workgroup, to its first threads (the host guarantees M*K/16 <= grid *
// 2^upw_log). Small mode takes the fewest units per workgroup that cover
// them all (the tail's stores spread over more CUs); large mode the most
// whose token pairs fit one wave (fewer quant workgroups; measured faster
// there, slower in small mode).
template <int NV, int MT, int RPW, int L>
__global__ void __launch_bounds__(256) fused_valu_kernel(FusedArgs a) {
  extern __shared__ int smem[];
  fused_body<NV>(a, smem, [&](int t, auto&& sink, auto&& pre) {
    valu_tile<MT, RPW, L>(a.g, t % a.g.nb_count, t / a.g.nb_count, sink, pre);
  });
}

template <int NV, int MT, int KS>
__global__ void __launch_bounds__(256) fused_mfma_kernel(FusedArgs a) {
  extern __shared__ int smem[];
  fused_body<NV>(a, smem, [&](int t, auto&& sink, auto&& pre) {
    const int nb = t % a.g.nb_count;
    const int s = (t / a.g.nb_count) % a.g.s_count;
    const int mb = t / (a.g.nb_count * a.g.s_count);
    mfma_tile<MT, KS>(a.g, mb, nb, s, reinterpret_cast<float*>(smem), sink, pre);
  });
}

}  // namespace rgt
