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
// no hand-off needs a counter. Wave 0 of every workgroup reads the epoch
// before it stores its first partial, and the other waves take its value
// through LDS; the gate workgroup advances the epoch only after it has seen
// every partial (small mode), workgroup 0 only after every id (large mode),
// which implies that every workgroup has read it. Tags repeat after 2^32 - 1
// calls; a rotating window of the tagged-word area outside the call's own
// words is zeroed every call, so no stale word lives that long.
// Every wait is bounded by a deadline that sets the workspace error word; a
// call that finds the error word set waits for nothing and writes defined
// poison outputs (top-k ids -1, weights 0, offsets 0) until the workspace is
// reset.
#pragma once

#include "device.h"
#include "gate.h"
#include "gemv.h"
#include "norm.h"
#include "sortq.h"

namespace rgt {

// Control words at the head of the workspace: the error word and the call
// epoch side by side (one 8-byte load reads both).
enum : int { kCtlErr = 0, kCtlEpoch = 1 };

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
  u64* scrub;          // the workspace past the tile counters (16-byte aligned)
  u32 scrub_units;     // its size in 16-byte units (> 0)
  u32 fp_part0, fp_part1, fp_ids0, fp_ids1;  // this call's tagged words, 16-byte units from scrub
  // The RMSNorm producer in front of the router (instances with the norm
  // only): g.x is the raw x, the router and the quant read xn.
  const u16* res;      // [M][ldr] residual or null
  int64_t ldr;
  const u16* gamma;    // [K]
  float eps;
  u16* xn;             // [M][ldxn] written
  int64_t ldxn;
  u16* res_out;        // [M][ldro] written with h if not null (needs res)
  int64_t ldro;
  float* rstd_out;     // [M] written if not null
  u64* trs;            // [M] tagged rstd words (workspace, after tids)
};

// The fused kernels' scalar arguments ahead of FusedArgs (the tile's
// operands, preloaded into scalar registers; see the kernels below) and the
// byte offset of FusedArgs in the kernarg segment after them.
struct TileParams {
  const u16* x;
  const u16* w;
  int ldx, ldw, m, nbc;
  u32 nbm;
  int mbc;
  u32 mbm;
  int grid;
};
constexpr unsigned kFusedArgsAt = (sizeof(TileParams) + alignof(FusedArgs) - 1) / alignof(FusedArgs) * alignof(FusedArgs);
static_assert(sizeof(TileParams) == 48 && kFusedArgsAt == 48, "kernel argument layout");

// A field of the call's FusedArgs read from the kernarg segment where it is
// used (output pointers of the tail; values whose use must stay behind the
// tile's loads).
#define RGT_ARG(field) \
  ::rgt::kernarg_at<decltype(::rgt::FusedArgs::field)>(::rgt::kFusedArgsAt + offsetof(::rgt::FusedArgs, field))
#define RGT_OUT(field) RGT_ARG(field)

// Set by a wave of the small-mode tail whose own gather expired; zeroed at
// the kernel's start, read by all waves after the tail's mask barrier.
__shared__ u32 s_tail_err;

// The call's tag from the epoch word: epoch + 1, skipping 0 so zero-filled
// words never look ready. The control words stay per-lane values (every lane
// loads the same words): moving them to scalar registers would make the wave
// wait for this load before issuing the tile's loads.
__device__ __forceinline__ u32 call_tag_of(u32 epoch) {
  const u32 t = epoch + 1u;
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
// one). during() runs in every thread once the first poll is issued. Each thread polls its own loads until every word carries the tag,
// re-issuing them as soon as they return short of it (one poll in flight: a
// second poll issued with the first sees the same memory state, and the loads
// it leaves in flight at the exit cost a wait at the next register reuse),
// then sums each item's slices in k-slice order. Returns false (error word
// set) if the deadline passes.
template <int NL, class During>
__device__ __forceinline__ bool gather_logits(const FusedArgs& a, int r0, int rows, u32 tag, float* s_log,
                                              During&& during) {
  __shared__ u32 s_bad;
  const int n = a.g.n, S = a.g.s_count;
  const int items = rows * (n >> 1);
  const u32 slice = (u32)a.g.m * (u32)n * 8u;
  const u32 row_base = (u32)r0 * (u32)n * 8u;
  const int t = threadIdx.x;
  if (t == 0) s_bad = 0u;
  __syncthreads();
  {
    // Only threads with items poll; during() runs in every thread between the
    // first issue and the poll loop (uniform there, so it may exchange values
    // between lanes).
    const bool poller = t < items;
    const auto rsrc = coherent_rsrc(a.tpart, slice * (u32)S);
    u32 off[NL];
    {
      int it = min(t, items - 1), s = 0;
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
    if (poller) issue(va);
    during();  // other work while the first poll is in flight
    RGT_STAMP(a.trace, 11);
    while (poller) {
      if (ready(va)) { take(va); break; }
      issue(va);
      if (rt_clock() - t0 > a.budget) {
        set_timeout(a);
        s_bad = 1u;
        break;
      }
    }
    RGT_STAMP(a.trace, 15);
  }
  __syncthreads();
  return s_bad == 0u;
}

// One row of 128 experts gathered by the calling wave alone (no LDS, no
// barrier): lane l polls the k-slices of column pair l (NL >= S loads, the
// ones past S repeat the last slice) and sums them in k-slice order, the
// same bits as gather_logits. during() runs once the first poll is issued.
// false (error word set) if the deadline passes.
template <int NL, class During>
__device__ __forceinline__ bool wave_gather_pairs(const FusedArgs& a, u32 tag, int row, float (&sv)[2],
                                                  During&& during) {
  const int S = a.g.s_count;
  const u32 slice = (u32)a.g.m * (u32)a.g.n * 8u;
  const auto rsrc = coherent_rsrc(a.tpart, slice * (u32)S);
  const u32 base = (u32)row * (u32)a.g.n * 8u + 16u * (u32)lane_id();
  u32x4_t v[NL];
  auto issue = [&] {
#pragma unroll
    for (int l = 0; l < NL; ++l) v[l] = ld_agent16(rsrc, base + (u32)min(l, S - 1) * slice);
  };
  auto ready = [&] {
    bool ok = true;
#pragma unroll
    for (int l = 0; l < NL; ++l) ok = ok & (v[l].y == tag) & (v[l].w == tag);
    return ok;
  };
  const u64 t0 = rt_clock();
  issue();
  RGT_STAMP(a.trace, 11);
  during();
  bool ok = true;
  for (;;) {
    if (ready()) {
      float x0 = 0.f, x1 = 0.f;
#pragma unroll
      for (int l = 0; l < NL; ++l)
        if (l < S) {
          x0 += __uint_as_float(v[l].x);
          x1 += __uint_as_float(v[l].z);
        }
      sv[0] = x0;
      sv[1] = x1;
      break;
    }
    issue();
    if (rt_clock() - t0 > a.budget) {
      set_timeout(a);
      ok = false;
      break;
    }
  }
  RGT_STAMP(a.trace, 15);
  return ballot64(!ok) == 0ull;
}

// One row gathered by the calling wave alone when the partials are one
// k-slice (no sum): lane l takes experts [l*NV, l*NV + NV) as NV/2 column
// pairs (pairs past the row repeat its last one; their experts are absent),
// polling until every word carries the tag. false (error word set) if the
// deadline passes.
template <int NV>
__device__ __forceinline__ bool wave_gather_row1(const FusedArgs& a, u32 tag, int row, float (&sv)[NV]) {
  static_assert(NV % 2 == 0, "column pairs");
  constexpr int NP = NV / 2;
  const int np = a.g.n >> 1;
  const auto rsrc = coherent_rsrc(a.tpart, (u32)a.g.m * (u32)a.g.n * 8u);
  const u32 base = (u32)row * (u32)a.g.n * 8u;
  const int p0 = lane_id() * NP;
  u32x4_t v[NP];
  auto issue = [&] {
#pragma unroll
    for (int c = 0; c < NP; ++c) v[c] = ld_agent16(rsrc, base + 16u * (u32)min(p0 + c, np - 1));
  };
  auto ready = [&] {
    bool ok = true;
#pragma unroll
    for (int c = 0; c < NP; ++c) ok = ok & (v[c].y == tag) & (v[c].w == tag);
    return ok;
  };
  const u64 t0 = rt_clock();
  issue();
  bool ok = true;
  for (;;) {
    if (ready()) {
#pragma unroll
      for (int c = 0; c < NP; ++c) {
        sv[2 * c] = __uint_as_float(v[c].x);
        sv[2 * c + 1] = __uint_as_float(v[c].z);
      }
      break;
    }
    issue();
    if (rt_clock() - t0 > a.budget) {
      set_timeout(a);
      ok = false;
      break;
    }
  }
  return ballot64(!ok) == 0ull;
}

// Loads per thread that a gather of `rows` rows needs.
__host__ __device__ constexpr int gather_loads(int rows, int n, int s) { return (rows * (n / 2) + 255) / 256 * s; }

// Gather with the (item, slice) loads spread over all 256 threads when the
// items alone would leave most threads idle: items is a power of two below
// 256 and tpi = 256 / items threads share an item, each polling a run of
// consecutive slices; the loaded partials meet in LDS, and the item's thread
// then adds its S slices in k-slice order (the same order as the in-register
// sum, so the same bits). SP: slices a thread polls, at most.
// The staged partials share LDS with s_log, which the host sizes to
// S * rows * n floats in that case: slice s of item it sits at float2 index
// s * items + it, so slice 0 of an item is where its sum goes, and only that
// item's thread reads it before writing the sum.
// (Only for 8 or more slices: with fewer, the extra LDS pass and barrier
// cost more than the shorter polls save; measured at 1 and 2 rows, 3 slices.)
__host__ __device__ constexpr bool fused_gather_staged(int rows, int n, int s) {
  return s >= 8 && rows * (n / 2) < 256 && ((rows * (n / 2)) & (rows * (n / 2) - 1)) == 0 &&
         s * rows * (n / 2) <= 2048;
}
template <int SP, class During>
__device__ __forceinline__ bool gather_staged(const FusedArgs& a, int r0, int rows, u32 tag, float* s_log,
                                              During&& during) {
  __shared__ u32 s_bad;
  float2* s_stage = reinterpret_cast<float2*>(s_log);
  const int n = a.g.n, S = a.g.s_count;
  const int items = rows * (n >> 1);
  const int lg = 31 - __clz(items);
  const int tpi = 256 >> lg;
  const int sp = (S + tpi - 1) / tpi;
  const u32 slice = (u32)a.g.m * (u32)n * 8u;
  const u32 row_base = (u32)r0 * (u32)n * 8u;
  const int t = threadIdx.x;
  const int it = t & (items - 1), sub = t >> lg;
  const int s0 = sub * sp;
  const int ns = max(0, min(sp, S - s0));  // this thread's slices
  if (t == 0) s_bad = 0u;
  __syncthreads();
  const auto rsrc = coherent_rsrc(a.tpart, slice * (u32)S);
  u32 off[SP];
#pragma unroll
  for (int l = 0; l < SP; ++l) off[l] = row_base + 16u * (u32)it + (u32)min(s0 + l, S - 1) * slice;
  u32x4_t va[SP];
  auto issue = [&]() {
#pragma unroll
    for (int l = 0; l < SP; ++l) va[l] = ld_agent16(rsrc, off[l]);
  };
  auto ready = [&]() {
    bool ok = true;
#pragma unroll
    for (int l = 0; l < SP; ++l) ok = ok & ((l >= ns) | ((va[l].y == tag) & (va[l].w == tag)));
    return ok;
  };
  const bool poller = ns > 0;
  const u64 t0 = rt_clock();
  if (poller) issue();
  during();
  while (poller) {
    if (ready()) {
#pragma unroll
      for (int l = 0; l < SP; ++l)
        if (l < ns) s_stage[(s0 + l) * items + it] = make_float2(__uint_as_float(va[l].x), __uint_as_float(va[l].z));
      break;
    }
    issue();
    if (rt_clock() - t0 > a.budget) {
      set_timeout(a);
      s_bad = 1u;
      break;
    }
  }
  __syncthreads();
  if (t < items && s_bad == 0u) {
    float2 acc = make_float2(0.f, 0.f);
    for (int s = 0; s < S; ++s) {
      const float2 v = s_stage[s * items + t];
      acc.x += v.x;
      acc.y += v.y;
    }
    s_stage[t] = acc;  // = s_log[2t], 2t+1
  }
  __syncthreads();
  return s_bad == 0u;
}

template <class During>
__device__ __forceinline__ bool gather_any(const FusedArgs& a, int r0, int rows, u32 tag, float* s_log,
                                           During&& during) {
  const int items = rows * (a.g.n >> 1), S = a.g.s_count;
  if (fused_gather_staged(rows, a.g.n, S)) {
    const int sp = (S + (256 / items) - 1) / (256 / items);
    if (sp <= 2) return gather_staged<2>(a, r0, rows, tag, s_log, during);
    if (sp <= 4) return gather_staged<4>(a, r0, rows, tag, s_log, during);
  }
  const int nl = gather_loads(rows, a.g.n, a.g.s_count);
  if (nl <= 4) return gather_logits<4>(a, r0, rows, tag, s_log, during);
  if (nl <= 8) return gather_logits<8>(a, r0, rows, tag, s_log, during);
  return gather_logits<kPollLoads>(a, r0, rows, tag, s_log, during);
}
__device__ __forceinline__ bool gather_any(const FusedArgs& a, int r0, int rows, u32 tag, float* s_log) {
  return gather_any(a, r0, rows, tag, s_log, [] {});
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

// Owner form of the top-k of one row of logits held in LDS, by the calling
// wave: for each of this lane's NV experts (lane-major, expert lane*NV + i)
// whether it is selected, its slot and its score key. bv: this lane's bias
// values. Up to four experts a lane the threshold selection; above, the
// pruned selection (k rounds of a wave maximum when it cannot prune) whose
// slot-ordered winners are handed to their owners through s_flag (n ints of
// LDS owned by the calling wave). With slots false
// (a caller that only needs the selected set, one position per winner) the
// threshold selection numbers the winners in expert order instead of by rank.
template <int NV>
__device__ __forceinline__ void row_topk_owner(const FusedArgs& a, float (&sv)[NV], const float (&bv)[NV],
                                               bool (&sel)[NV], int (&slot)[NV], u32 (&key)[NV], int* s_flag,
                                               bool slots) {
  const int n = a.g.n, k = a.topk, lane = lane_id(), c0 = lane * NV;
  if (a.bias) {
#pragma unroll
    for (int i = 0; i < NV; ++i) sv[i] = __fadd_rn(sv[i], bv[i]);
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) key[i] = c0 + i < n ? score_key(sv[i]) : 0u;
  RGT_STAMP(a.trace, 12);
  if constexpr (NV <= 4) {
    __shared__ __align__(16) u64 s_c[4][32];
    u64* sc = s_c[threadIdx.x >> 6];
    wave_threshold_select<NV>(key, k, sel);
    if (!slots) wave_select_order<NV>(sel, slot);
    else if (k <= 8) wave_select_slots<NV, 8>(key, sel, slot, sc);
    else if (k <= 16) wave_select_slots<NV, 16>(key, sel, slot, sc);
    else wave_select_slots<NV, 32>(key, sel, slot, sc);
  } else {
    __shared__ __align__(16) int s_slot[4][64];
    float sv1[1][NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) sv1[0][i] = sv[i];
    int id[1];
    u32 kk[1];
    wave_select_rows<NV, 1>(sv1, n, k, id, kk, s_slot[threadIdx.x >> 6]);
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (c0 + i < n) s_flag[c0 + i] = 0;
    if (lane < k) s_flag[id[0]] = lane + 1;  // one wave: after the zeroing
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int f = c0 + i < n ? s_flag[c0 + i] : 0;
      sel[i] = f > 0;
      slot[i] = f - 1;
    }
  }
  RGT_STAMP(a.trace, 13);
}
template <int NV>
__device__ __forceinline__ void row_topk_owner(const FusedArgs& a, const float* row, const float (&bv)[NV],
                                               bool (&sel)[NV], int (&slot)[NV], u32 (&key)[NV], int* s_flag,
                                               bool slots) {
  const int n = a.g.n, c0 = lane_id() * NV;
  float sv[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) sv[i] = row[min(c0 + i, n - 1)];
  row_topk_owner<NV>(a, sv, bv, sel, slot, key, s_flag, slots);
}

// The top-k of one row of logits held in LDS, by the calling wave: scores
// lane-major (expert lane*NV + i), plus the bias (bv: this lane's bias values,
// loaded at the start of the kernel). emit(j, e, key) runs once for each of
// the k selected experts, in the lane holding it: slot j, expert e, score key.
// Up to four experts a lane the threshold selection; above, the pruned
// selection (k rounds of a wave maximum when it cannot prune), slot order.
template <int NV, class Emit>
__device__ __forceinline__ void row_topk(const FusedArgs& a, const float* row, const float (&bv)[NV], Emit&& emit) {
  const int n = a.g.n, k = a.topk, lane = lane_id(), c0 = lane * NV;
  float sv[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) sv[i] = row[min(c0 + i, n - 1)];
  if (a.bias) {
#pragma unroll
    for (int i = 0; i < NV; ++i) sv[i] = __fadd_rn(sv[i], bv[i]);
  }
  RGT_STAMP(a.trace, 12);
  if constexpr (NV <= 4) {
    __shared__ __align__(16) u64 s_c[4][32];
    u64* sc = s_c[threadIdx.x >> 6];
    u32 key[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) key[i] = c0 + i < n ? score_key(sv[i]) : 0u;
    bool sel[NV];
    int slot[NV];
    if (k <= 8) wave_topk_threshold<NV, 8>(key, k, sel, slot, sc);
    else if (k <= 16) wave_topk_threshold<NV, 16>(key, k, sel, slot, sc);
    else wave_topk_threshold<NV, 32>(key, k, sel, slot, sc);
    RGT_STAMP(a.trace, 13);
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (sel[i]) emit(slot[i], c0 + i, key[i]);
  } else {
    __shared__ __align__(16) int s_slot[4][64];
    float sv1[1][NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) sv1[0][i] = sv[i];
    int id[1];
    u32 key[1];
    wave_select_rows<NV, 1>(sv1, n, k, id, key, s_slot[threadIdx.x >> 6]);
    RGT_STAMP(a.trace, 13);
    if (lane < k) emit(lane, id[0], key[0]);
  }
}

// Small mode's gate workgroup: the weights of rows r0, r0 + step, ... from the
// selected keys in s_key (one wave per row at a time).
__device__ __forceinline__ void rows_weights(const FusedArgs& a, const u32* s_key, int r0, int step) {
  const int k = a.topk, lane = lane_id();
  float* const topk_w = RGT_OUT(topk_w);
  for (int row = r0; row < a.g.m; row += step) {
    const float w = wave_weights(s_key[row * k + min(lane, k - 1)], k);
    if (lane < k) topk_w[row * k + lane] = w;
  }
}

// Zero one window of the workspace's tagged-word area per call (all
// workgroups' reads and writes of this call stay inside its footprint, which
// the window skips), so that over a sweep of a few hundred calls every word
// outside the current footprint is rewritten. Tags repeat only after 2^32 - 1
// calls, so no word can keep a tag that long and be mistaken for a fresh one.
// Threads t0, t0 + nt, ... take its 256 units.
__device__ __forceinline__ void scrub_window(const FusedArgs& a, u32 tag, u32 t0 = threadIdx.x, u32 nt = 256u) {
  const u32 units = a.scrub_units;
  const u32 first = (u32)(((u64)tag * 256u) % units);
  for (u32 t = t0; t < 256u; t += nt) {
    const u32 i = first + t >= units ? first + t - units : first + t;
    const bool in_fp = (i >= a.fp_part0 && i < a.fp_part1) || (i >= a.fp_ids0 && i < a.fp_ids1);
    if (t < units && !in_fp) reinterpret_cast<uint4*>(a.scrub)[i] = make_uint4(0, 0, 0, 0);
  }
}

// Outputs of a call made on a workspace whose error word is set (an earlier
// wait expired): every top-k id is -1, every weight 0 and every offset 0
// (a padded total of 0: no row of the sort outputs is valid).
__device__ __forceinline__ void write_poison(const FusedArgs& a) {
  const int P = a.g.m * a.topk;
  int32_t* const topk_ids = RGT_OUT(topk_ids);
  float* const topk_w = RGT_OUT(topk_w);
  int32_t* const offsets = RGT_OUT(offsets);
  for (int i = threadIdx.x; i < P; i += 256) {
    topk_ids[i] = -1;
    topk_w[i] = 0.f;
  }
  for (int e = threadIdx.x; e <= a.g.n; e += 256) offsets[e] = 0;
}

// pos(p) of 64-bit lane masks: the set bits of mask below the calling lane.
__device__ __forceinline__ int mask_below(u64 mask) {
  return (int)__builtin_amdgcn_mbcnt_hi((u32)(mask >> 32), __builtin_amdgcn_mbcnt_lo((u32)mask, 0u));
}
__device__ __forceinline__ u64 uniform_u64(u64 v) {
  return ((u64)(u32)__builtin_amdgcn_readfirstlane((int)(v >> 32)) << 32) |
         (u32)__builtin_amdgcn_readfirstlane((int)(u32)v);
}

// A quant workgroup's chunks stored by all of its 256 threads: thread t
// keeps chunk slot us = t mod 2^upw_log of the workgroup (its codes and
// packed scales read from LDS once) and stores it to the padded rows of
// pairs j = t >> upw_log, + 256 >> upw_log, ... of its token (consecutive
// threads take consecutive chunks of one padded row). All of the thread's
// positions are read before its first store, so the LDS latencies overlap.
// s_codes / s_sc: the chunks' codes and packed scales by chunk slot; s_pos:
// the padded row of pair t*k + j.
template <int JN, bool FP4>
__device__ __forceinline__ void store_chunk_rows(const FusedArgs& a, int t, int c, int j0, int js, const int* s_pos,
                                                 const uint4& cd, u32 sc) {
  const int k = a.topk;
  const u32 row_bytes = FP4 ? (u32)a.g.k >> 1 : (u32)a.g.k;
  const u32 kscale = (u32)a.g.k >> 5;
  uint8_t* q_col = RGT_OUT(a_q) + (FP4 ? 8 * c : 16 * c);
  uint8_t* s_col = RGT_OUT(a_scale) + (c >> 1);
  const bool lead = (c & 7) == 0;
  int r[JN];
#pragma unroll
  for (int i = 0; i < JN; ++i) r[i] = s_pos[t * k + min(j0 + i * js, k - 1)];
  // (Write-through stores, agent-scope or non-temporal, measured no faster.)
#pragma unroll
  for (int i = 0; i < JN; ++i) {
    if (j0 + i * js < k) {
      uint8_t* row = q_col + (u64)(u32)r[i] * row_bytes;
      if (FP4) *reinterpret_cast<uint2*>(row) = make_uint2(cd.x, cd.y);
      else *reinterpret_cast<uint4*>(row) = cd;
      if (lead) *reinterpret_cast<u32*>(s_col + (u64)(u32)r[i] * kscale) = sc;
    }
  }
}
__device__ __forceinline__ void store_chunks_spread(const FusedArgs& a, int u0, const int* s_pos,
                                                    const uint4* s_codes, const u32* s_sc) {
  const int k = a.topk, ul = a.upw_log;
  const int cpr = a.g.k >> 4, units = a.g.m * cpr;
  const int us = (int)threadIdx.x & ((1 << ul) - 1);
  const int j0 = (int)threadIdx.x >> ul, js = 256 >> ul;  // js = 4, 2 or 1
  const int unit = u0 + us;
  if (unit >= units || j0 >= k) return;
  const int t = div_magic(unit, a.cpr_magic), c = unit - t * cpr;
  const uint4 cd = s_codes[us];
  const u32 sc = s_sc[us];
  const int jn = (k - j0 + js - 1) / js;  // this thread's pairs
  if (a.fp4) {
    if (jn <= 2) store_chunk_rows<2, true>(a, t, c, j0, js, s_pos, cd, sc);
    else if (jn <= 4) store_chunk_rows<4, true>(a, t, c, j0, js, s_pos, cd, sc);
    else if (jn <= 8) store_chunk_rows<8, true>(a, t, c, j0, js, s_pos, cd, sc);
    else store_chunk_rows<32, true>(a, t, c, j0, js, s_pos, cd, sc);
  } else {
    if (jn <= 2) store_chunk_rows<2, false>(a, t, c, j0, js, s_pos, cd, sc);
    else if (jn <= 4) store_chunk_rows<4, false>(a, t, c, j0, js, s_pos, cd, sc);
    else if (jn <= 8) store_chunk_rows<8, false>(a, t, c, j0, js, s_pos, cd, sc);
    else store_chunk_rows<32, false>(a, t, c, j0, js, s_pos, cd, sc);
  }
}

// Small mode after the partials are seen: every participant has every row's
// logits; wave r runs row r's gate (M <= 4). With M no larger than the block
// size (block >= 16), an expert holds at most M pairs, so each selected
// expert fills exactly one block: its segment starts at block * (number of
// selected experts below it), and a pair's rank in it is the number of
// earlier rows that chose the same expert. Both come from the rows' selection
// masks (one ballot per key slot), so the sort needs no histogram and no
// scan. The gate workgroup writes topk_ids, the weights, the logits and the
// epoch; the layout workgroup writes offsets, expert_ids and sorted_ids
// (pairs and pads); the quant workgroups store their chunks. With one row
// the pairs' padded rows are 0, B, ..., (k-1)B whichever experts win (the
// row's pair is the first row of each of the k blocks), and the gate
// workgroup, which has the slots, writes the pairs' sorted_ids entries, so
// the layout workgroup needs only the selected set. The instances built for
// one row (ONE) go further: the quant-only workgroups store at once, with no
// gather and no gate, and at 128 experts the gate and layout workgroups run
// on one wave with no LDS pass or barrier. (Only there: the extra code costs
// the other instances scalar-register spills, +0.4 us at two rows.)
template <int NV, bool ONE, class Quant>
__device__ __forceinline__ void small_tail(const FusedArgs& a, int* smem, u32 tag, int role, bool have_unit, int unit,
                                           Quant&& quant, const float (&bv)[NV], bool gate_here, bool layout_here,
                                           bool quant_wg) {
  __shared__ __align__(16) u64 s_mask[4][NV];
  const GemvArgs& g = a.g;
  const int m = g.m, n = g.n, k = a.topk, B = a.block;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int P = m * k, c0 = lane * NV;
  int* s_pos = smem;                                  // [P] padded position of pair r*k + j
  u32* s_key = reinterpret_cast<u32*>(smem + P);      // [P] score key of slot j of row r
  float* s_log = reinterpret_cast<float*>(smem + fused_log_offset(P, n));
  const int stage = fused_gather_staged(m, n, g.s_count) ? (g.s_count - 1) * m * n : 0;
  int* s_flag = smem + fused_tail_ints(P, n, m) + stage + wave * n;  // above four experts a lane only
  // the chunks go to LDS so that all four waves store them
  __shared__ uint4 s_codes[256];
  __shared__ u32 s_sc[256];
  u32 sb_in = 0;
  uint4 codes_in = make_uint4(0, 0, 0, 0);
  if (ONE && m == 1 && quant_wg && !gate_here && !layout_here) {
    codes_in = quant(sb_in);
    const u32 scales4 = pack_scales(sb_in);  // all lanes: DPP reads neighbouring lanes
    if (have_unit) {
      s_codes[threadIdx.x] = codes_in;
      s_sc[threadIdx.x] = scales4;
    }
    if ((int)threadIdx.x < k) s_pos[threadIdx.x] = (int)threadIdx.x * B;
    __syncthreads();
    RGT_STAMP(a.trace, 8);
    store_chunks_spread(a, role << a.upw_log, s_pos, s_codes, s_sc);
#ifdef RGT_TRACE
    vm_drain();  // the stores acknowledged
    RGT_STAMP(a.trace, 2);
#endif
    return;
  }
  if constexpr (ONE && NV == 2) {
    if (m == 1 && n == 128 && !quant_wg && g.s_count <= 8 && !fused_gather_staged(1, n, g.s_count)) {
      // The gate or layout workgroup of one row of 128 experts: its parts run
      // on separate waves, each gathering the row for itself (lane l holds
      // experts 2l and 2l + 1, as its gather leaves them) with no LDS pass
      // and no barrier. Gate: wave 0 the ids, the pairs' sorted_ids entries,
      // the logits and the epoch, wave 1 the weights; layout: one wave the
      // offsets and expert_ids, one the pads (which do not depend on the
      // winners) and the scrub.
      const int wl = wave - (gate_here ? 2 : 0);
      const bool do_ids = gate_here && wave == 0, do_w = gate_here && wave == 1;
      const bool do_off = layout_here && wl == 0, do_pad = layout_here && wl == 1;
      if (do_pad) {
        int32_t* const sorted_ids = RGT_OUT(sorted_ids);
        for (int q = lane; q < k * B; q += 64)
          if (q & (B - 1)) sorted_ids[q] = P;
        if (lane == 0) RGT_OUT(offsets)[n] = k * B;
        scrub_window(a, tag, lane, 64u);
      }
      if (!(do_ids || do_w || do_off)) return;
      float sv[2];
      const bool ok = g.s_count <= 4 ? wave_gather_pairs<4>(a, tag, 0, sv, [] {})
                                     : wave_gather_pairs<8>(a, tag, 0, sv, [] {});
      if (!ok) return;
      RGT_STAMP(a.trace, 5);
      const float lg[2] = {sv[0], sv[1]};  // the logits (the gate adds the bias to sv)
      bool sel[2];
      int slot[2], ord[2];
      u32 key[2];
      row_topk_owner<2>(a, sv, bv, sel, slot, key, nullptr, do_ids || do_w);
      wave_select_order<2>(sel, ord);  // winners below, = the block of each expert
      RGT_STAMP(a.trace, 14);
      if (do_ids) {
        int32_t* const topk_ids = RGT_OUT(topk_ids);
        int32_t* const sorted_ids = RGT_OUT(sorted_ids);
#pragma unroll
        for (int i = 0; i < 2; ++i)
          if (sel[i]) {
            topk_ids[slot[i]] = c0 + i;
            sorted_ids[ord[i] * B] = slot[i];  // the pair of slot j leads its expert's block
          }
        float* const logits_out = RGT_OUT(logits_out);
        if (logits_out) {
          logits_out[c0] = lg[0];
          logits_out[c0 + 1] = lg[1];
        }
        // every partial has been seen, so every workgroup's tag is read
        if (lane == 0) st_agent(a.ctl + kCtlEpoch, tag);
      }
      if (do_w) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
          if (sel[i]) s_key[slot[i]] = key[i];
        const float w = wave_weights(s_key[min(lane, k - 1)], k);  // one wave: after its LDS writes
        if (lane < k) RGT_OUT(topk_w)[lane] = w;
      }
      if (do_off) {
        // the k present experts fill one block each
        int32_t* const offsets = RGT_OUT(offsets);
        int32_t* const expert_ids = RGT_OUT(expert_ids);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          offsets[c0 + i] = ord[i] * B;
          if (sel[i]) expert_ids[ord[i]] = c0 + i;
        }
        RGT_STAMP(a.trace, 7);
      }
#ifdef RGT_TRACE
      vm_drain();  // the stores acknowledged
      RGT_STAMP(a.trace, 2);
#endif
      return;
    }
  }
  // The thread's quant chunk is encoded while the first poll is in flight.
  // With 128 experts and two to four rows each row wave gathers its own row
  // into registers (thread t of a workgroup gather would hold item t, i.e.
  // the same values), so the rows need no LDS pass and the gather no
  // barrier; a wave whose wait expires flags it, and every wave leaves after
  // the mask barrier below.
  const int row = wave;
  float rv[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) rv[i] = 0.f;
  bool wave_rows = false, wave_ok = true;
  if constexpr (!ONE && NV == 2) {
    if (n == 128 && m >= 2 && g.s_count <= 12 && !fused_gather_staged(m, n, g.s_count)) {
      wave_rows = true;
      auto enc = [&] { codes_in = quant(sb_in); };
      if (row < m)
        wave_ok = g.s_count <= 4   ? wave_gather_pairs<4>(a, tag, row, rv, enc)
                  : g.s_count <= 8 ? wave_gather_pairs<8>(a, tag, row, rv, enc)
                                   : wave_gather_pairs<12>(a, tag, row, rv, enc);
      else
        enc();
      if (!wave_ok && lane == 0) s_tail_err = 1u;
    }
  }
  if (!wave_rows && !gather_any(a, 0, m, tag, s_log, [&] { codes_in = quant(sb_in); })) return;
  RGT_STAMP(a.trace, 5);
  bool sel[NV];
  int slot[NV];
  u32 key[NV];
  if (row < m && wave_ok) {
    // quant-only workgroups (and the layout workgroup of one row) need the
    // selected set, not the slots: their positions are indexed by winner
    // order, the same k rows either way
    const bool slots = gate_here || (layout_here && m > 1);
    if (wave_rows) {
      float sv[NV];
#pragma unroll
      for (int i = 0; i < NV; ++i) sv[i] = rv[i];
      row_topk_owner<NV>(a, sv, bv, sel, slot, key, s_flag, slots);
    } else {
      row_topk_owner<NV>(a, s_log + row * n, bv, sel, slot, key, s_flag, slots);
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const u64 mk = ballot64(sel[i]);
      if (m > 1 && lane == 0) s_mask[row][i] = mk;
    }
    if (gate_here) {
      int32_t* const topk_ids = RGT_OUT(topk_ids);
#pragma unroll
      for (int i = 0; i < NV; ++i)
        if (sel[i]) {
          topk_ids[row * k + slot[i]] = c0 + i;
          s_key[row * k + slot[i]] = key[i];
        }
      if (m == 1) {
        // the pair of winner j (expert order) sits at row j * B
        int32_t* const sorted_ids = RGT_OUT(sorted_ids);
        int ord[NV];
        wave_select_order<NV>(sel, ord);
#pragma unroll
        for (int i = 0; i < NV; ++i)
          if (sel[i]) sorted_ids[ord[i] * B] = slot[i];
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      sel[i] = false;
      slot[i] = 0;
    }
  }
  if (gate_here) {
    float* const logits_out = RGT_OUT(logits_out);
    if (logits_out) {
      if (wave_rows) {
        if (row < m)
#pragma unroll
          for (int i = 0; i < NV; ++i) logits_out[row * n + c0 + i] = rv[i];
      } else {
        for (int i = threadIdx.x; i < m * n; i += 256) logits_out[i] = s_log[i];
      }
    }
  }
  // (one row: wave 0 holds everything the positions need, no barrier here)
  if (m > 1) __syncthreads();
  if (wave_rows && s_tail_err) return;  // every wave, after the barrier
  RGT_STAMP(a.trace, 14);
  if (gate_here) {
    // Every partial has been seen, so every workgroup's tag is read.
    if (threadIdx.x == 0) st_agent(a.ctl + kCtlEpoch, tag);
    if (!quant_wg && !layout_here) {
      if (row < m) {
        const float w = wave_weights(s_key[row * k + min(lane, k - 1)], k);
        if (lane < k) RGT_OUT(topk_w)[row * k + lane] = w;
      }
      return;
    }
  }
  // Segment layout from the rows' selection masks mr (uniform): for this
  // lane's experts, the first block (blocks before it: present experts
  // below), the pair count and the rank of row `row`'s pair among them.
  struct Seg {
    int blk[NV], cnt[NV], rk[NV];
    bool present[NV];
    int total;  // present experts
  };
  auto seg_of = [&](const u64 (&mr)[4][NV]) {
    Seg sg;
    u64 un[NV];
    int run = 0;
    sg.total = 0;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      un[i] = mr[0][i] | mr[1][i] | mr[2][i] | mr[3][i];
      run += mask_below(un[i]);
      sg.total += __popcll(un[i]);
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      sg.present[i] = (un[i] >> lane) & 1ull;
      sg.blk[i] = run;
      run += sg.present[i] ? 1 : 0;
      int c = 0, rk = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int bit = (int)((mr[r][i] >> lane) & 1ull);
        c += bit;
        rk += r < row ? bit : 0;
      }
      sg.cnt[i] = c;
      sg.rk[i] = rk;
    }
    return sg;
  };
  // (all rows' words read together, one LDS round trip, and the rows past M
  // masked off afterwards: a read per row behind its own branch waited a
  // round trip each)
  auto masks_lds = [&](u64 (&mr)[4][NV]) {
    u64 v[4][NV];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int i = 0; i < NV; ++i) v[r][i] = s_mask[r][i];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int i = 0; i < NV; ++i) mr[r][i] = uniform_u64(v[r][i]) & (r < m ? ~0ull : 0ull);
  };
  // Positions of this wave's row (one row: wave 0's own ballots, no barrier
  // before). The layout workgroup writes the layout here too, from the same
  // masks, before the chunk exchange: offsets of every expert (an absent
  // one's segment is empty), the block of each present expert and its pads.
  if (row < m || (layout_here && m > 1)) {
    u64 mr[4][NV];
    if (m == 1) {
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        mr[0][i] = ballot64(sel[i]);
        mr[1][i] = mr[2][i] = mr[3][i] = 0ull;
      }
    } else {
      masks_lds(mr);
    }
    const Seg sg = seg_of(mr);
    int32_t* const sorted_ids = layout_here ? RGT_OUT(sorted_ids) : nullptr;
    if (row < m) {
#pragma unroll
      for (int i = 0; i < NV; ++i)
        if (sel[i]) {
          const int q = sg.blk[i] * B + sg.rk[i];
          s_pos[row * k + slot[i]] = q;
          if (layout_here && m > 1) sorted_ids[q] = row * k + slot[i];
        }
    }
    RGT_STAMP(a.trace, 6);
    if (layout_here) {
      if (wave == 0) {
        int32_t* const offsets = RGT_OUT(offsets);
        int32_t* const expert_ids = RGT_OUT(expert_ids);
#pragma unroll
        for (int i = 0; i < NV; ++i) {
          if (c0 + i < n) offsets[c0 + i] = sg.blk[i] * B;
          if (sg.present[i]) expert_ids[sg.blk[i]] = c0 + i;
        }
        if (lane == 0) offsets[n] = sg.total * B;
      }
      if (m == 1) {
        // every block holds one pair (its first row) and B - 1 pads: the
        // rows below k * B that are not a multiple of B (wave 0 alone)
        for (int q = lane; q < sg.total * B; q += 64)
          if (q & (B - 1)) sorted_ids[q] = P;
      } else {
        // Each wave writes the pair count of every block (its lanes hold all
        // the experts) to a table of its own and reads only its own writes,
        // so no barrier; then thread t pads rows t, t + 256, ... of the
        // blocks (a row past its block's pairs).
        __shared__ int s_bcnt[4][128];  // blocks <= M * k <= 4 * 32
        int* bc = s_bcnt[wave];
#pragma unroll
        for (int i = 0; i < NV; ++i)
          if (sg.present[i]) bc[sg.blk[i]] = sg.cnt[i];
        const int lb = __ffs(B) - 1;
        for (int q = threadIdx.x; q < sg.total * B; q += 256)
          if ((q & (B - 1)) >= bc[q >> lb]) sorted_ids[q] = P;
      }
      RGT_STAMP(a.trace, 7);
    }
  }
  const u32 scales4 = pack_scales(sb_in);  // all lanes: DPP reads neighbouring lanes
  if (have_unit) {
    s_codes[threadIdx.x] = codes_in;
    s_sc[threadIdx.x] = scales4;
  }
  __syncthreads();  // s_pos, the chunks and the masks complete
  RGT_STAMP(a.trace, 8);
  if (quant_wg) store_chunks_spread(a, role << a.upw_log, s_pos, s_codes, s_sc);
  RGT_STAMP(a.trace, 9);
  if (gate_here && row < m) {  // the gate workgroup had no spare of its own
    const float w = wave_weights(s_key[row * k + min(lane, k - 1)], k);
    if (lane < k) RGT_OUT(topk_w)[row * k + lane] = w;
  }
  if (layout_here) scrub_window(a, tag);
#ifdef RGT_TRACE
  vm_drain();  // the stores acknowledged
  RGT_STAMP(a.trace, 2);
#endif
}

// quant(sb) returns the thread's encoded quant chunk and its scale byte(s);
// every lane of a wave calls it together.
template <int NV, bool ONE, bool VALU, class Quant>
__device__ __forceinline__ void fused_tail(const FusedArgs& a, int* smem, u32 tag, bool poisoned, int role,
                                           bool have_unit, int unit, Quant&& quant, const float (&bv)[NV]) {
  const GemvArgs& g = a.g;
  const int m = g.m, n = g.n, k = a.topk;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int units = m * (g.k >> 4);
  // Roles. Quant workgroups [0, q_wgs) hold the quant units; the layout
  // workgroups (one per 256 experts) follow them if the grid has room, else
  // they are the last ones; the spare workgroups after them run the gates
  // that feed the others: small mode's gate workgroup (the first spare, else
  // workgroup 0) and large mode's row workgroups (spare ones when all M fit,
  // else workgroup r for row r).
  const int q_wgs = ((units - 1) >> a.upw_log) + 1;
  const int n_layout = (n + 255) >> 8;
  const int layout_wg = min((int)gridDim.x - n_layout, q_wgs);
  const int li = role - layout_wg;  // this workgroup's layout share, if 0 <= li < n_layout
  const int spare0 = layout_wg + n_layout;
  const int gate_wg = (a.small && spare0 < (int)gridDim.x) ? spare0 : 0;
  const bool gate_here = role == gate_wg;
  const bool quant_wg = role < q_wgs;
  const bool layout_here = li >= 0 && li < n_layout;
  const bool participant = gate_here || quant_wg || layout_here;
  const int P = m * k;
  RGT_STAMP(a.trace, 3);
  if (poisoned) {
    // An earlier wait of this workspace expired: no waits, defined outputs.
    if (role == layout_wg) write_poison(a);
    return;
  }
  if (a.small) {
    // one layout workgroup writes the whole layout in small mode
    if (!(gate_here || quant_wg || li == 0)) return;
    small_tail<NV, ONE>(a, smem, tag, role, have_unit, unit, quant, bv, gate_here, li == 0, quant_wg);
    return;
  }
  // Step 2 (large): row workgroups gather their row, run its gate and
  // publish the ids; then every participant polls all ids.
  const int row_wg0 = spare0 + m <= (int)gridDim.x ? spare0 : 0;
  const int row = role - row_wg0;
  u32* s_key1 = reinterpret_cast<u32*>(smem);  // a spare row workgroup's k keys
  if constexpr (NV == 2) {
    if (row >= 0 && row < m && !participant && n == 128 && g.s_count <= 12) {
      // A spare row workgroup at 128 experts: wave 0 alone gathers the row
      // into registers (lane l: experts 2l, 2l + 1), runs its gate and
      // publishes the ids; no LDS pass, no barrier.
      if (wave != 0) return;
      float sv[2];
      const int S = g.s_count;
      const bool ok = S <= 4   ? wave_gather_pairs<4>(a, tag, row, sv, [] {})
                      : S <= 8 ? wave_gather_pairs<8>(a, tag, row, sv, [] {})
                               : wave_gather_pairs<12>(a, tag, row, sv, [] {});
      if (!ok) return;
      RGT_STAMP(a.trace, 5);
      const int c0 = lane * 2;
      const float lg[2] = {sv[0], sv[1]};  // the logits (the gate adds the bias to sv)
      bool sel[2];
      int slot[2];
      u32 key[2];
      row_topk_owner<2>(a, sv, bv, sel, slot, key, nullptr, true);
      int32_t* const topk_ids = RGT_OUT(topk_ids);
#pragma unroll
      for (int i = 0; i < 2; ++i)
        if (sel[i]) {
          st_agent(a.tids + row * k + slot[i], tag_word((u32)(c0 + i), tag));
          topk_ids[row * k + slot[i]] = c0 + i;
          s_key1[slot[i]] = key[i];
        }
      // the pad word of an odd pair count: every word of the call's
      // footprint carries its tag
      if (row == m - 1 && lane == 0 && (P & 1)) st_agent(a.tids + P, tag_word(0u, tag));
      float* const logits_out = RGT_OUT(logits_out);
      if (logits_out) {
        logits_out[(int64_t)row * n + c0] = lg[0];
        logits_out[(int64_t)row * n + c0 + 1] = lg[1];
      }
      const float w = wave_weights(s_key1[min(lane, k - 1)], k);  // one wave: after its LDS writes
      if (lane < k) RGT_OUT(topk_w)[row * k + lane] = w;
      RGT_STAMP(a.trace, 6);
      return;
    }
  }
  if constexpr (VALU && NV > 4 && NV % 2 == 0) {  // (one k-slice: VALU plans only)
    if (row >= 0 && row < m && !participant && g.s_count == 1 && (n & 1) == 0) {
      // A spare row workgroup over more than 256 experts with one k-slice:
      // wave 0 alone gathers the row into registers (lane l: experts
      // [l*NV, l*NV + NV)), selects (lane j ends with slot j: the keys that
      // reach the k-th largest lane maximum, one a lane, by threshold; k
      // rounds of a wave maximum when more than 64 reach it) and publishes
      // the ids; no LDS pass of the row, no barrier.
      if (wave != 0) return;
      float sv[NV];
      if (!wave_gather_row1<NV>(a, tag, row, sv)) return;
      RGT_STAMP(a.trace, 5);
      const int c0 = lane * NV;
      float* const logits_out = RGT_OUT(logits_out);
      if (logits_out) {
#pragma unroll
        for (int i = 0; i < NV; ++i)
          if (c0 + i < n) logits_out[(int64_t)row * n + c0 + i] = sv[i];
      }
      float sb[1][NV];
#pragma unroll
      for (int i = 0; i < NV; ++i) sb[0][i] = a.bias ? __fadd_rn(sv[i], bv[i]) : sv[i];
      __shared__ __align__(16) int s_sel[64];
      int id[1];
      u32 key[1];
      wave_select_rows<NV, 1>(sb, n, k, id, key, s_sel);
      if (lane < k) {
        st_agent(a.tids + row * k + lane, tag_word((u32)id[0], tag));
        RGT_OUT(topk_ids)[row * k + lane] = id[0];
      }
      // the pad word of an odd pair count: every word of the call's
      // footprint carries its tag
      if (row == m - 1 && lane == 0 && (P & 1)) st_agent(a.tids + P, tag_word(0u, tag));
      const float w = wave_weights(key[0], k);
      if (lane < k) RGT_OUT(topk_w)[row * k + lane] = w;
      RGT_STAMP(a.trace, 6);
      return;
    }
  }
  u32 sb_in = 0;
  const uint4 codes_in = quant(sb_in);  // all lanes: the scale exchange reads the partner lane
  int* s_e = smem;
  u32* s_key = reinterpret_cast<u32*>(s_e + P);
  int* s_pos = s_e + 2 * P;   // 64 entries
  int* s_cnt = s_pos + 64;
  int* s_pre = s_cnt + n;
  int* s_off = s_pre + n;
  float* s_log = reinterpret_cast<float*>(smem + fused_log_offset(P, n));
  // This workgroup's tokens (those its quant units touch) and their pairs.
  const int cpr = g.k >> 4;
  const int u0 = role << a.upw_log;
  const int t0 = min(m, div_magic(u0, a.cpr_magic)), t1 = min(m, div_magic(u0 + (1 << a.upw_log) - 1, a.cpr_magic) + 1);
  const int p0 = u0 < units ? t0 * k : 0, p1 = u0 < units ? t1 * k : 0;
  // The expert histograms are filled as the ids become known (zeroed here;
  // the barriers of the gather or of the id poll come before any add).
  if (participant)
    for (int e = threadIdx.x; e < n; e += 256) {
      s_cnt[e] = 0;
      s_pre[e] = 0;
    }
  {
    if (row >= 0 && row < m) {
      if (!gather_any(a, row, 1, tag, s_log)) return;
      RGT_STAMP(a.trace, 5);
      if (wave == 0) {
        // (s_key is free in large mode: its first k entries hold the row's
        // keys in slot order for the weights)
        int32_t* const topk_ids = RGT_OUT(topk_ids);
        row_topk<NV>(a, s_log, bv, [&](int j, int e, u32 key) {
          st_agent(a.tids + row * k + j, tag_word((u32)e, tag));
          topk_ids[row * k + j] = e;
          s_key[j] = key;
        });
        // the pad word of an odd pair count: every word of the call's
        // footprint carries its tag
        if (row == m - 1 && lane == 0 && (P & 1)) st_agent(a.tids + P, tag_word(0u, tag));
        const float w = wave_weights(s_key[min(lane, k - 1)], k);  // after the ids are published
        if (lane < k) RGT_OUT(topk_w)[row * k + lane] = w;
      }
      float* const logits_out = RGT_OUT(logits_out);
      if (logits_out)
        for (int i = threadIdx.x; i < n; i += 256) logits_out[(int64_t)row * n + i] = s_log[i];
      RGT_STAMP(a.trace, 6);
    }
    if (!participant) return;
    if (!poll_ids_any(a, P, tag, s_e, p0, s_cnt, s_pre)) return;
  }
  RGT_STAMP(a.trace, 10);
  // Every workgroup's tag is read (see the top of this file): advance the
  // epoch for the next call (large mode, or small mode without a spare gate
  // workgroup).
  if (gate_here && threadIdx.x == 0) st_agent(a.ctl + kCtlEpoch, tag);
  // Step 3: positions of the pairs of this workgroup's tokens (a counting
  // sort from the expert histogram), then the workgroup stores its quantised
  // chunk to the padded rows of those pairs. The token's pairs' sorted_ids
  // entries are written by the workgroup holding its first quant unit; the
  // layout workgroup writes offsets, expert_ids and the pads.
  if (threadIdx.x < 64) pair_positions<NV>(P, n, a.block, p0, p1, s_e, s_cnt, s_pre, s_off, s_pos);
  __syncthreads();
  RGT_STAMP(a.trace, 8);
  int32_t* const sorted_ids = RGT_OUT(sorted_ids);
  if (layout_here)
    write_layout<256>(s_cnt, s_off, n, a.block, P, li << 8, min(n, (li + 1) << 8), sorted_ids,
                      RGT_OUT(expert_ids), RGT_OUT(offsets));
  if ((int)threadIdx.x < p1 - p0) {
    const int p = p0 + threadIdx.x, q = s_pos[threadIdx.x];
    const int tok = p / k;
    if (q >= 0 && (tok * cpr) >> a.upw_log == role) sorted_ids[q] = p;
  }
  RGT_STAMP(a.trace, 7);
  const u32 scales4 = pack_scales(sb_in);  // all lanes: DPP reads neighbouring lanes
  if (have_unit)
    store_unit(RGT_OUT(a_q), RGT_OUT(a_scale), g.k, k, unit, OffsetPos{s_pos, p0}, codes_in, scales4, a.cpr_magic,
               a.fp4 != 0);
  RGT_STAMP(a.trace, 9);
  if (li == 0) scrub_window(a, tag);
#ifdef RGT_TRACE
  vm_drain();  // the stores acknowledged
  RGT_STAMP(a.trace, 2);
#endif
}

// The router behind the RMSNorm producer ("route on the norm's scale",
// MiniMax-M3.1 FFN monokernel page, Modifications): workgroup r < M is row
// r's norm workgroup; it loads that row of x (and the residual) before its
// tile's loads, and once its tile's loads are out takes the row's rstd with
// the norm kernel's own reduction and publishes it as a tagged word. Every
// tile loads the raw x, residual and gamma chunks of its own columns, takes
// its rows' rstd words and normalises those columns itself (h, then xn, as
// the norm kernel computes them), so its products are those of the router
// fed the norm's xn. The norm workgroups publish before they wait, and the
// launch is co-resident, so every wait ends. With one row every workgroup
// takes the row's rstd itself (the same reduction, so the same bits) and
// nothing is published or waited for: the row is 2K bytes (4K with the
// residual) served by L2, cheaper than a hand-off.
constexpr int kNormChunks = 4;  // 8-element chunks a thread holds of a norm row: K <= 8192

struct NormX {
  static constexpr bool kOn = true;
  const FusedArgs& a;
  const u32& tag;  // the wave's control words, read by prefetch before row_work
  u32& err;
  float& rs_own;   // the rstd this workgroup took (its norm row's)
  const int role;  // the workgroup's role index (see fused_body)
  uint4 hv[kNormChunks];
  uint4 rv[kNormChunks];

  __device__ __forceinline__ NormX(const FusedArgs& args, const u32& t, u32& e, float& r, int ro)
      : a(args), tag(t), err(e), rs_own(r), role(ro) {}

  __device__ __forceinline__ bool local() const { return a.g.m == 1; }
  __device__ __forceinline__ bool norm_wg() const { return local() || role < a.g.m; }
  __device__ __forceinline__ int norm_row() const { return local() ? 0 : role; }

  // Before the tile's loads: the norm row's x and residual.
  __device__ __forceinline__ void begin() {
    if (!norm_wg()) return;
    const int nch = a.g.k >> 3, row = norm_row();
#pragma unroll
    for (int c = 0; c < kNormChunks; ++c) {
      const int idx = min((int)threadIdx.x + 256 * c, nch - 1);
      hv[c] = ld16(a.g.x + (int64_t)row * a.g.ldx + 8 * idx);
      if (a.res) rv[c] = ld16(a.res + (int64_t)row * a.ldr + 8 * idx);
    }
  }
  __device__ __forceinline__ uint4 res(int row, int k) const {
    return a.res ? ld16(a.res + (int64_t)row * a.ldr + k) : make_uint4(0, 0, 0, 0);
  }
  __device__ __forceinline__ uint4 gamma(int k) const { return ld16(a.gamma + k); }
  // The norm workgroup's rstd, published (whole workgroup: one barrier).
  __device__ __forceinline__ void row_work() {
    if (!norm_wg()) return;
    if (a.res) {
#pragma unroll
      for (int c = 0; c < kNormChunks; ++c) hv[c] = add_bf16x8(hv[c], rv[c]);
    }
    const float rs = row_rstd<kNormChunks>(hv, a.g.k >> 3, a.g.k, a.eps);
    rs_own = rs;
    if (threadIdx.x == 0) {
      if (!local() && !a.fault_skip && err == 0u) {
        st_agent(a.trs + role, tag_word(__float_as_uint(rs), tag));
        // the pad word of an odd M: every word of the call's footprint
        // carries its tag
        if (role == a.g.m - 1 && (a.g.m & 1)) st_agent(a.trs + a.g.m, tag_word(0u, tag));
      }
      if (a.rstd_out && role < a.g.m) a.rstd_out[role] = rs;
    }
    RGT_STAMP(a.trace, 11);
  }
  // The rows' published rstd (lanes may ask for different rows), all words
  // polled together. On an expired wait the error word is set and this wave
  // publishes nothing; a workspace already in error waits for nothing (no
  // word is published).
  template <int R>
  __device__ __forceinline__ void rstd_rows(const int (&rows)[R], float (&out)[R]) {
    if (local()) {
#pragma unroll
      for (int i = 0; i < R; ++i) out[i] = rs_own;
      return;
    }
    u64 v[R];
    auto issue = [&]() {
#pragma unroll
      for (int i = 0; i < R; ++i) v[i] = ld_agent(a.trs + rows[i]);
    };
    auto ready = [&]() {
      bool ok = true;
#pragma unroll
      for (int i = 0; i < R; ++i) ok = ok & tag_ok(v[i], tag);
      return ok;
    };
    issue();
    if (err == 0u && ballot64(!ready())) {
      const u64 t0 = rt_clock();
      for (;;) {
        issue();
        if (!ballot64(!ready())) break;
        if (rt_clock() - t0 > a.budget) {
          set_timeout(a);
          err = kErrTimeout;
          break;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < R; ++i) out[i] = __uint_as_float((u32)v[i]);
    RGT_STAMP(a.trace, 15);
  }
  __device__ __forceinline__ uint4 residual(uint4 x, uint4 r) const { return a.res ? add_bf16x8(x, r) : x; }
  __device__ __forceinline__ uint4 apply(uint4 h, uint4 g, float rs) const { return norm_bf16x8(h, g, rs); }
};

// A quant unit of the norm variant: its chunk of xn (and h), from the raw x
// and residual chunks and the token's rstd (with one row the workgroup's
// own, else the published word: it is out before any tile of the token ends,
// so it is there by the tail); stores both. One lane's wait; false if it
// expired.
__device__ __forceinline__ bool norm_unit(const FusedArgs& a, int unit, u32 tag, float rs_own, uint4& xa, uint4& xb,
                                          const uint4& ra, const uint4& rb, const uint4& ga, const uint4& gb) {
  const int cpr = a.g.k >> 4, t = div_magic(unit, a.cpr_magic), c = unit - t * cpr;
  float rs = rs_own;
  if (a.g.m > 1) {
    u64 v = ld_agent(a.trs + t);
    if (!tag_ok(v, tag)) {
      const u64 t0 = rt_clock();
      while (!tag_ok(v = ld_agent(a.trs + t), tag)) {
        if (rt_clock() - t0 > a.budget) {
          set_timeout(a);
          return false;
        }
      }
    }
    rs = __uint_as_float((u32)v);
  }
  if (a.res) {
    xa = add_bf16x8(xa, ra);
    xb = add_bf16x8(xb, rb);
    if (a.res_out) {
      uint4* ro = reinterpret_cast<uint4*>(a.res_out + (int64_t)t * a.ldro + 16 * c);
      ro[0] = xa;
      ro[1] = xb;
    }
  }
  xa = norm_bf16x8(xa, ga, rs);
  xb = norm_bf16x8(xb, gb, rs);
  uint4* xo = reinterpret_cast<uint4*>(a.xn + (int64_t)t * a.ldxn + 16 * c);
  xo[0] = xa;
  xo[1] = xb;
  return true;
}

// Shared head of the kernels: read the control words, run the tile, then the
// tail. tile(t, sink, pre, xf) computes this workgroup's GEMV tile; with NORM
// the tile and the quant units read the RMSNorm of x (NormX).
template <int NV, bool NORM, bool ONE, bool VALU, class Tile>
__device__ __forceinline__ void fused_body(const FusedArgs& a, int* smem, int grid, Tile tile) {
  __shared__ u32 s_ctl[2];
  const GemvArgs& g = a.g;
  // The workgroup's place among the quant, layout, gate, row and norm
  // workgroups: its block index, so the tail's workgroups spread over the
  // XCDs (block b runs on XCD b % 8). (The XCDs' first workgroups start up to
  // ~0.55 us apart, XCD 0 first; placing the tail's roles on the first XCDs
  // instead, all on XCD 0 or spread over XCDs 0-3, measured slower at one
  // and at 64 rows, faster at 8-16, +-0.1-0.4 us.)
  const int role = (int)blockIdx.x;
  const int tile_id = xcd_tile(blockIdx.x, grid);  // grid = gridDim.x
  // The thread's quant unit, set once the tile's loads are out (its inputs
  // are read from the argument block there, so no wait for them comes
  // ahead of those loads).
  int unit = 0;
  bool have_unit = false;
  RGT_STAMP(a.trace, 0);
  // Right after the tile's W loads are issued: the control words (loads
  // return in order, so issued earlier they would hold up the tile's
  // arithmetic), the thread's quant chunk of x (with the norm: and of the
  // residual and gamma), quantised once the tile is done, and the lane's bias
  // values for the gate.
  u32 tag = 0, err = 0;
  uint4 xa = make_uint4(0, 0, 0, 0), xb = make_uint4(0, 0, 0, 0);
  [[maybe_unused]] uint4 ra = xa, rb = xa, ga = xa, gb = xa;
  float bv[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) bv[i] = 0.f;
  auto prefetch = [&]() {
    const int ul = RGT_ARG(upw_log), units = RGT_ARG(g.m) * (RGT_ARG(g.k) >> 4);
    unit = (role << ul) + threadIdx.x;
    have_unit = (int)threadIdx.x < (1 << ul) && unit < units;
    const u64 cw = ld_agent(reinterpret_cast<const u64*>(a.ctl));
    err = (u32)cw;
    tag = call_tag_of((u32)(cw >> 32));
    if (have_unit) {
      const int cpr = g.k >> 4, t = div_magic(unit, a.cpr_magic), c = unit - t * cpr;
      const u16* src = g.x + (int64_t)t * g.ldx + 16 * c;
      xa = ld16(src);
      xb = ld16(src + 8);
      if constexpr (NORM) {
        if (a.res) {
          const u16* rsrc = a.res + (int64_t)t * a.ldr + 16 * c;
          ra = ld16(rsrc);
          rb = ld16(rsrc + 8);
        }
        ga = ld16(a.gamma + 16 * c);
        gb = ld16(a.gamma + 16 * c + 8);
      }
    }
    if (a.bias) {
      const int c0 = lane_id() * NV;
#pragma unroll
      for (int i = 0; i < NV; ++i) bv[i] = a.bias[min(c0 + i, g.n - 1)];
    }
  };
  auto sink = [&](int s, int row, int col, float v) {
    if (!a.fault_skip && err == 0u)
      st_agent(a.tpart + ((int64_t)s * g.m + row) * g.n + col, tag_word(__float_as_uint(v), tag));
  };
  [[maybe_unused]] float rs_own = 0.f;
  if constexpr (NORM) {
    NormX xf(a, tag, err, rs_own, role);
    xf.begin();
    tile(tile_id, sink, prefetch, xf);
  } else {
    tile(tile_id, sink, prefetch, NoNorm());
  }
  RGT_STAMP(a.trace, 1);
  // Every wave takes wave 0's control words. Wave 0 stores at least one
  // partial (row 0 of its tile) with its tag, so once every partial of the
  // call has been seen, every workgroup's read of the epoch is complete and
  // it may advance; the other waves may store no partial (rows past M), and
  // a read of their own could return the advanced epoch.
  if (threadIdx.x == 0) {
    s_ctl[0] = tag;
    s_ctl[1] = err;
    s_tail_err = 0u;
  }
  __syncthreads();  // also: the tile's LDS is reused below
  tag = s_ctl[0];
  err = s_ctl[1];
  RGT_STAMP(a.trace, 4);
  auto quant = [&](u32& sb) {
    uint4 c0 = xa, c1 = xb;
    if constexpr (NORM) {
      if (have_unit) norm_unit(a, unit, tag, rs_own, c0, c1, ra, rb, ga, gb);
    }
    return mx_quant16_fmt(c0, c1, sb, a.fp4 != 0);
  };
  fused_tail<NV, ONE, VALU>(a, smem, tag, err != 0u, role, have_unit, unit, quant, bv);
}

// Quant units (16-element chunks of x, row-major) go 2^upw_log to a
// workgroup, to its first threads (the host guarantees M*K/16 <= grid *
// 2^upw_log). Small mode takes the fewest units per workgroup that cover
// them all (the tail's stores spread over more CUs); large mode the most
// whose token pairs fit one wave (fewer quant workgroups; measured faster
// there, slower in small mode).
// The kernels take the operands of the tile's first loads as scalar
// arguments ahead of FusedArgs: built with the first ten arguments
// preloaded into scalar registers when the workgroup starts, the tile's
// loads go out without waiting for the argument block (a kernarg-segment
// load takes ~0.2 us at a workgroup's start), and the tile index is split
// with host-computed reciprocals instead of runtime divisions. x, w, ldx,
// ldw, m are a.g's; nbc = a.g.nb_count; mbc = the row blocks of the MFMA
// plan; nbm, mbm = 2^32 / nbc, 2^32 / mbc rounded up (unused for 1); grid = gridDim.x (a
// hidden argument otherwise, loaded from the segment).
#define RGT_TILE_PARAMS                                                                                   \
  const u16 *__restrict__ x, const u16 *__restrict__ w, int ldx, int ldw, int m, int nbc, u32 nbm, int mbc, \
      u32 mbm, int grid
// t / d by the host's reciprocal (d = 1 has none that fits 32 bits).
__device__ __forceinline__ int div_by(int t, int d, u32 magic) { return d == 1 ? t : div_magic(t, magic); }
__device__ __forceinline__ GemvArgs tile_args(const FusedArgs& a, const u16* x, const u16* w, int ldx, int ldw,
                                              int m) {
  GemvArgs g = a.g;
  g.x = x;
  g.w = w;
  g.ldx = ldx;
  g.ldw = ldw;
  g.m = m;
  return g;
}

template <int NV, bool NORM, int MT, int RPW, int L>
__global__ void __launch_bounds__(256) fused_valu_kernel(RGT_TILE_PARAMS, FusedArgs a) {
  extern __shared__ int smem[];
  fused_body<NV, NORM, MT == 1, true>(a, smem, grid, [&](int t, auto&& sink, auto&& pre, auto&& xf) {
    const int s = div_by(t, nbc, nbm);
    valu_tile<MT, RPW, L>(tile_args(a, x, w, ldx, ldw, m), t - s * nbc, s, sink, pre, xf);
  });
}

template <int NV, bool NORM, int MT, int KS>
__global__ void __launch_bounds__(256) fused_mfma_kernel(RGT_TILE_PARAMS, FusedArgs a) {
  extern __shared__ int smem[];
  fused_body<NV, NORM, false, false>(a, smem, grid, [&](int t, auto&& sink, auto&& pre, auto&& xf) {
    // row block fastest: the row blocks of one W tile run side by side
    const int r = div_by(t, mbc, mbm), mb = t - r * mbc;
    const int s = div_by(r, nbc, nbm), nb = r - s * nbc;
    mfma_tile<MT, KS>(tile_args(a, x, w, ldx, ldw, m), mb, nb, s, reinterpret_cast<float*>(smem), sink, pre, xf);
  });
}
#undef RGT_TILE_PARAMS

}  // namespace rgt
