// rgt.hip - host side of the routing front-end library (C ABI in rgt.h).
//
// Validation happens before any HIP call, so every argument error is reported
// without touching the GPU. Plans (tile kind and split) are picked per M
// bucket, in the spirit of the per-M-bucket configs of "MiniMax-M3: Triton
// split-K router GEMV with in-kernel split-K fixup" (opening summary), but
// sized for 256 CUs in 8 XCDs.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "rgt.h"
#include "device.h"
#include "diag.h"
#include "fused.h"
#include "fused_pick.h"
#include "gate.h"
#include "gemm.h"
#include "gemv.h"
#include "norm.h"
#include "shared.h"
#include "shared_pick.h"
#include "sortq.h"
#include "sortq_kernels.h"
#include "stage1.h"

using namespace rgt;

namespace {

constexpr int kVersion = 100;  // 0.1.0
constexpr size_t kAlign = 256;
constexpr size_t kCtlBytes = 512;          // control words (error, phase counters), 128 B apart
constexpr int kMaxTileCounters = 8192;     // arrival counters for GEMV tiles
constexpr int kSmallSortMaxP = 8192;       // one-workgroup sort up to this many pairs
constexpr int kLargeSortChunk = 512;       // pairs per workgroup in the large sort
constexpr int kFusedMaxM = 64;

thread_local int g_last_launches = 0;
std::atomic<bool> g_sort_lds_set{false};  // the one-workgroup sort may use more than 64 KB of LDS
constexpr int kSortSmallMaxLds = 120 * 1024;

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int env_int(const char* name, int dflt) {
  const char* v = std::getenv(name);
  return v && *v ? std::atoi(v) : dflt;
}

// Environment settings, read at the first call and again by rgt_reload_env
// (so that no call pays for getenv):
//   RGT_WAIT_BUDGET_US  deadline of each device-side wait (default 100000)
//   RGT_NO_FUSE=1       never the one-launch form
//   RGT_NORM_IN_LAUNCH  1: the norm joins the launch whenever it fits, 0: never
//   RGT_FORCE_BUCKET    comma-separated: valu | mfma (router tile, M <= 8 for
//                       valu), small | large (the one-launch tail's mode)
//   RGT_LOG=1           one stderr line per new shape with the plan chosen
//   RGT_FAULT_INJECT=1  host-forced fault: nothing is published (tests)
enum { kForceNone = 0, kForceValu = 1, kForceMfma = 2 };
enum { kModeAuto = 0, kModeSmall = 1, kModeLarge = 2 };
struct Config {
  long wait_budget_us = 100000;
  int no_fuse = 0;
  int norm_in_launch = -1;
  int force_tile = kForceNone;
  int force_mode = kModeAuto;
  int log = 0;
  int fault_inject = 0;
  unsigned gen = 0;  // bumped by every reload (plan cache key)
};
Config g_cfg;
std::once_flag g_cfg_once;
std::mutex g_cfg_mu;

void load_config() {
  Config c;
  c.wait_budget_us = env_int("RGT_WAIT_BUDGET_US", 100000);
  c.no_fuse = env_int("RGT_NO_FUSE", 0);
  c.norm_in_launch = env_int("RGT_NORM_IN_LAUNCH", -1);
  c.log = env_int("RGT_LOG", 0);
  c.fault_inject = env_int("RGT_FAULT_INJECT", 0);
  if (const char* f = std::getenv("RGT_FORCE_BUCKET")) {
    const char* q = f;
    while (*q) {
      const char* e = q;
      while (*e && *e != ',') ++e;
      const size_t len = (size_t)(e - q);
      auto is = [&](const char* w) { return std::strlen(w) == len && std::strncmp(q, w, len) == 0; };
      if (is("valu")) c.force_tile = kForceValu;
      else if (is("mfma")) c.force_tile = kForceMfma;
      else if (is("small")) c.force_mode = kModeSmall;
      else if (is("large")) c.force_mode = kModeLarge;
      q = *e ? e + 1 : e;
    }
  }
  c.gen = g_cfg.gen + 1;
  g_cfg = c;
}

const Config& config() {
  std::call_once(g_cfg_once, [] {
    std::lock_guard<std::mutex> lk(g_cfg_mu);
    load_config();
  });
  return g_cfg;
}

bool covered(int m, int n, int k) {
  return m >= 0 && m <= 8192 && n >= 16 && n <= 1024 && n % 16 == 0 && k >= 512 && k % 512 == 0;
}

bool gate_covered(int n, int topk) { return topk >= 1 && topk <= 32 && topk <= n; }

bool block_covered(int b) { return b == 16 || b == 32 || b == 64; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// ---------------------------------------------------------------------------
// GEMV plan for one call.
// ---------------------------------------------------------------------------
struct Plan {
  bool gemm;     // large batches: LDS-tiled MFMA GEMM, no split-K
  bool valu;     // VALU tile (M <= 8) or MFMA tile
  int mt;        // VALU: rows in the template (1,2,4,8); MFMA: 16-row tiles (1..4)
  int rpw;       // VALU rows of W per wave
  int l;         // VALU 512-element k-chunks per lane (1, 2, 4 or 7)
  int ks;        // MFMA k-steps of 32 per wave (2, 4 or 8)
  int nb;        // n-blocks
  int s;         // k-slices
  int mb;        // row blocks (MFMA)
  int grid;      // workgroups
  int bn;        // experts per n-block
};

int pow2_at_least(int v) {
  int p = 1;
  while (p < v) p <<= 1;
  return p;
}

// Fewest k-slices that still give this many workgroups: every k-slice is one
// more partial per output for the fixup to read, and every workgroup one
// more to dispatch, so decode shapes aim at about a third of the CUs.
#ifndef RGT_MIN_GRID
#define RGT_MIN_GRID 96
#endif
#ifndef RGT_MFMA_ROWS_GRID
#define RGT_MFMA_ROWS_GRID 192
#endif

// The stage-1 GEMM splits K over a workgroup's waves below this many
// (row tile, 64-column group) pairs, and gives each wave two column tiles
// from this many (row tile, 128-column group) pairs. Measured (N = 128,
// K = 6144, top-8, I = 768): at M = 8 the K split beats one column tile a
// wave (62 against 73 us); at M = 64 two column tiles a wave beat one (146-150
// against 158-160 us) and the K split (157-159 us); at N = 896, K = 3584,
// top-16, I = 384, M = 32 one column tile would be 3 us faster (124 against
// 127-129 us).
#ifndef RGT_STAGE1_KSPLIT_BELOW
#define RGT_STAGE1_KSPLIT_BELOW 1024
#endif
#ifndef RGT_STAGE1_JT2_FROM
#define RGT_STAGE1_JT2_FROM 512
#endif

// Batches with at least this many 128 x 128 output tiles use the GEMM.
constexpr int kGemmMinTiles = 256;

Plan make_plan(int m, int n, int k) {
  Plan p{};
  if (m > kFusedMaxM && ((m + kGemmBM - 1) / kGemmBM) * ((n + kGemmBN - 1) / kGemmBN) >= kGemmMinTiles) {
    p.gemm = true;
    p.s = 1;
    p.mb = (m + kGemmBM - 1) / kGemmBM;
    p.nb = (n + kGemmBN - 1) / kGemmBN;
    p.bn = kGemmBN;
    p.grid = p.mb * p.nb;
    return p;
  }
  const int force = config().force_tile;
  // VALU tile to 8 rows; at most 128 experts the 16-row MFMA tile from 5 rows
  // (12 k-slices, 96 workgroups: M = 5 / 6 / 7 / 8 in 7.41 / 7.55 / 7.65 /
  // 7.53 us against 7.56 / 7.76 / 7.88 / 7.99 with the 8-row VALU tile; at
  // 3-4 rows the two are within 0.1 us, at 2 rows the MFMA plan's 12
  // k-slices cost 1.5 us in the small-mode gather).
  if (m <= 8 && force != kForceMfma && (force == kForceValu || m <= 4 || n > 128)) {
    p.valu = true;
    p.mt = pow2_at_least(std::max(m, 1));
    p.rpw = 1;
    p.bn = 4;
    p.nb = n / 4;
    p.mb = 1;
    const int chunks = k / 512;
    // The 8-row tile (M = 5..8) streams twice the grid: measured at M = 8,
    // N = 128, K = 6144, 192 workgroups of six k-slices beat 96 of three
    // (8.9 vs 9.4 us), while at M <= 4 the 96 win (6.5 vs 6.7 us at M = 1).
    const int min_grid = p.mt >= 8 ? 2 * RGT_MIN_GRID : RGT_MIN_GRID;
    p.l = 1;
    for (int l : {7, 4, 2}) {
      if (chunks % l == 0 && p.nb * (chunks / l) >= min_grid) {
        p.l = l;
        break;
      }
    }
    p.s = chunks / p.l;
  } else {
    // Fewest k-slices that give RGT_MIN_GRID workgroups with the tallest row
    // tile; then shorter row tiles while the grid stays under
    // RGT_MFMA_ROWS_GRID (each workgroup streams 16*MT rows of x from L2).
    // The row blocks of one W tile are neighbouring workgroups on one XCD
    // (the kernels take the row block as the fastest index), so the second
    // block's W loads are served by that XCD's L2 and W still streams from
    // HBM once.
    p.valu = false;
    p.bn = 16;
    p.nb = n / 16;
    p.mt = std::min(4, (m + 15) / 16);
    p.mb = (m + 16 * p.mt - 1) / (16 * p.mt);
    p.ks = 2;
    for (int ks : {8, 4}) {
      if (k % (128 * ks) == 0 && p.nb * p.mb * (k / (128 * ks)) >= RGT_MIN_GRID) {
        p.ks = ks;
        break;
      }
    }
    p.s = k / (128 * p.ks);
    while (p.mt > 1 && p.nb * p.s * p.mb < RGT_MFMA_ROWS_GRID) {
      p.mt = p.mt == 4 ? 2 : 1;
      p.mb = (m + 16 * p.mt - 1) / (16 * p.mt);
    }
  }
  p.grid = p.nb * p.s * p.mb;
  return p;
}

// Wide batches (more than 64 rows, too few 128 x 128 tiles to fill the chip)
// whose router runs as the k-split GEMM: from 384 rows at 128 experts, or
// more than 128 experts (where the split-K GEMV's 16-expert tiles re-read
// each x row N/16 times). Below, at N = 128, the split-K GEMV with its
// in-launch fixup measured faster (M = 128: 12 vs 13.5 us router + gate).
bool wide_gemm(int m, int n) {
  const int tiles = ((m + kGemmBM - 1) / kGemmBM) * ((n + kGemmBN - 1) / kGemmBN);
  return m > kFusedMaxM && tiles < kGemmMinTiles && (m >= 384 || n > 128);
}

// k-slices of the router GEMM for a wide batch: the most slices that still
// leave each workgroup four k-steps (at most 32), so a handful of 128 x 128
// tiles spread over more CUs; the gate (or a sum launch) adds the slices.
int chain_gemm_slices(int m, int n, int k) {
  const int tiles = ((m + kGemmBM - 1) / kGemmBM) * ((n + kGemmBN - 1) / kGemmBN);
  if (tiles >= kGemmMinTiles) return 1;
  const int steps = k / kGemmBK;
  for (int d = 32; d > 1; --d)
    if (steps % d == 0 && steps / d >= 4) return d;
  return 1;
}

// ---------------------------------------------------------------------------
// Workspace layout for one call (offsets depend on the call's own shape,
// except the control words and tile counters, which sit at fixed offsets and
// are the only state that must stay zero between calls).
// ---------------------------------------------------------------------------
struct Layout {
  size_t ctl, ctr, part, logits, tpart, tids, trs, pos, ghist, offws, trace, total;
};

int even_up(int v) { return (v + 1) & ~1; }

int large_sort_groups(int P) { return (P + kLargeSortChunk - 1) / kLargeSortChunk; }

Layout make_layout(int m, int n, int k, int topk) {
  Layout L{};
  const Plan p = make_plan(m, n, k);
  const int P = m * topk;
  size_t o = 0;
  L.ctl = o; o += kCtlBytes;
  L.ctr = o; o = align_up(o + sizeof(u32) * kCtrStride * (size_t)kMaxTileCounters, kAlign);
  const int part_slices = std::max(p.s, wide_gemm(m, n) ? chain_gemm_slices(m, n, k) : 1);
  L.part = o; o = align_up(o + sizeof(float) * (size_t)part_slices * m * n, kAlign);
  L.logits = o; o = align_up(o + sizeof(float) * (size_t)m * n, kAlign);
  L.tpart = L.tids = L.trs = o;
  if (m <= kFusedMaxM) {  // tagged hand-off words of the one-launch path
    L.tpart = o; o = align_up(o + sizeof(u64) * (size_t)p.s * m * n, kAlign);
    // the expert ids, then (behind the RMSNorm producer) the rows' rstd, each
    // padded to whole 16-byte units (the pad words are written too)
    L.tids = o;
    L.trs = o + sizeof(u64) * (size_t)even_up(P);
    o = align_up(L.trs + sizeof(u64) * (size_t)even_up(m), kAlign);
  }
  L.pos = o; o = align_up(o + sizeof(int32_t) * (size_t)P, kAlign);
  L.ghist = o;
  if (P > kSmallSortMaxP) o = align_up(o + sizeof(int32_t) * (size_t)large_sort_groups(P) * n, kAlign);
  L.offws = o; o = align_up(o + sizeof(int32_t) * (size_t)(2 * n + 1), kAlign);  // offsets, then counts
#ifdef RGT_TRACE
  L.trace = o; o = align_up(o + sizeof(u64) * 16 * (size_t)p.grid, kAlign);
#endif
  L.total = o;
  return L;
}

size_t ws_need(int m, int n, int k, int topk) { return make_layout(m, n, k, topk).total; }

// ---------------------------------------------------------------------------
// Device facts, cached per device.
// ---------------------------------------------------------------------------
struct DevInfo {
  int cus = 0;
  bool init = false;
};
std::mutex g_mu;
DevInfo g_dev[64];

bool dev_info(DevInfo& out) {
  int d = 0;
  if (hipGetDevice(&d) != hipSuccess || d < 0 || d >= 64) return false;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_dev[d].init) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, d) != hipSuccess) return false;
    g_dev[d].cus = prop.multiProcessorCount;
    g_dev[d].init = true;
  }
  out = g_dev[d];
  return true;
}

u64 wait_budget_ticks() {
  return (u64)std::max(1L, config().wait_budget_us) * 100ull;  // 100 MHz clock
}

rgt_status launched() {
  return hipGetLastError() == hipSuccess ? RGT_OK : RGT_ERR_HIP;
}

// ---------------------------------------------------------------------------
// Kernel dispatch helpers (template instantiation by switch).
// ---------------------------------------------------------------------------
int nv_bucket(int n) {
  const int nv = (n + 63) / 64;
  if (nv <= 2) return 2;
  if (nv <= 4) return 4;
  if (nv <= 8) return 8;
  if (nv <= 14) return 14;
  return 16;
}

template <int MT>
void launch_router_valu_rpw(const GemvArgs& a, const Plan& p, hipStream_t st) {
  switch (p.l) {
    case 1: hipLaunchKernelGGL((router_valu_kernel<MT, 1, 1>), dim3(p.grid), dim3(256), 0, st, a); break;
    case 2: hipLaunchKernelGGL((router_valu_kernel<MT, 1, 2>), dim3(p.grid), dim3(256), 0, st, a); break;
    case 4: hipLaunchKernelGGL((router_valu_kernel<MT, 1, 4>), dim3(p.grid), dim3(256), 0, st, a); break;
    default: hipLaunchKernelGGL((router_valu_kernel<MT, 1, 7>), dim3(p.grid), dim3(256), 0, st, a); break;
  }
}

template <int MT>
void launch_router_mfma(const GemvArgs& a, const Plan& p, hipStream_t st) {
  switch (p.ks) {
    case 2: hipLaunchKernelGGL((router_mfma_kernel<MT, 2>), dim3(p.grid), dim3(256), 0, st, a); break;
    case 4: hipLaunchKernelGGL((router_mfma_kernel<MT, 4>), dim3(p.grid), dim3(256), 0, st, a); break;
    default: hipLaunchKernelGGL((router_mfma_kernel<MT, 8>), dim3(p.grid), dim3(256), 0, st, a); break;
  }
}

// The prefill GEMM with 32*NJ experts a tile (its two LDS buffers need more
// than the default 64 KB of dynamic LDS: allowed once per instance).
template <int NJ>
bool launch_gemm_big(const GemvArgs& a, hipStream_t st) {
  static std::atomic<bool> lds_set{false};
  constexpr int bytes = gemm_big_lds_bytes<NJ>();
  if (bytes > 65536 && !lds_set.load()) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(router_gemm_big_kernel<NJ>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, bytes) != hipSuccess)
      return false;
    lds_set.store(true);
  }
  const int tiles = ((a.m + kGemmBM - 1) / kGemmBM) * ((a.n + 32 * NJ - 1) / (32 * NJ));
  hipLaunchKernelGGL(router_gemm_big_kernel<NJ>, dim3(tiles), dim3(512), bytes, st, a.x, a.ldx, a.w, a.ldw, a.logits,
                     a.m, a.n, a.k);
  return true;
}

void launch_router(const GemvArgs& a, const Plan& p, hipStream_t st) {
  if (p.gemm) {
    // 224 experts a tile where N is a multiple of it (N = 896: four tiles a
    // row block), 256 where N is one of that, 128 otherwise
    if (a.n % 224 == 0) launch_gemm_big<7>(a, st);
    else if (a.n % 256 == 0) launch_gemm_big<8>(a, st);
    else launch_gemm_big<4>(a, st);
    return;
  }
  if (p.valu) {
    switch (p.mt) {
      case 1: launch_router_valu_rpw<1>(a, p, st); break;
      case 2: launch_router_valu_rpw<2>(a, p, st); break;
      case 4: launch_router_valu_rpw<4>(a, p, st); break;
      default: launch_router_valu_rpw<8>(a, p, st); break;
    }
  } else {
    switch (p.mt) {
      case 1: launch_router_mfma<1>(a, p, st); break;
      case 2: launch_router_mfma<2>(a, p, st); break;
      case 3: launch_router_mfma<3>(a, p, st); break;
      default: launch_router_mfma<4>(a, p, st); break;
    }
  }
}

void launch_gate(const float* logits, const float* bias, int m, int n, int k, int32_t* ids, float* w,
                 hipStream_t st) {
  const dim3 grid((m + 3) / 4), blk(256);
  switch (nv_bucket(n)) {
    case 2: hipLaunchKernelGGL((topk_gate_kernel<2>), grid, blk, 0, st, logits, bias, m, n, k, ids, w); break;
    case 4: hipLaunchKernelGGL((topk_gate_kernel<4>), grid, blk, 0, st, logits, bias, m, n, k, ids, w); break;
    case 8: hipLaunchKernelGGL((topk_gate_kernel<8>), grid, blk, 0, st, logits, bias, m, n, k, ids, w); break;
    case 14: hipLaunchKernelGGL((topk_gate_kernel<14>), grid, blk, 0, st, logits, bias, m, n, k, ids, w); break;
    default: hipLaunchKernelGGL((topk_gate_kernel<16>), grid, blk, 0, st, logits, bias, m, n, k, ids, w); break;
  }
}

// The router GEMM of wide batches: k-slice partials to a.part (or the
// logits directly for one slice). Returns the number of launches (1).
int launch_chain_gemm(const GemvArgs& a, int m, int n, int k, hipStream_t st) {
  const int S = chain_gemm_slices(m, n, k);
  const int tiles = ((m + kGemmBM - 1) / kGemmBM) * ((n + kGemmBN - 1) / kGemmBN);
  float* out = S > 1 ? a.part : a.logits;
  if (k / S == 4 * kGemmBK)
    hipLaunchKernelGGL(router_gemm_kernel<4>, dim3(tiles * S), dim3(256), 0, st, a.x, a.ldx, a.w, a.ldw, out, m, n,
                       k / S);
  else
    hipLaunchKernelGGL(router_gemm_kernel<1>, dim3(tiles * S), dim3(256), 0, st, a.x, a.ldx, a.w, a.ldw, out, m, n,
                       k / S);
  return 1;
}

void launch_gate_partials(const float* part, int S, float* logits, const float* bias, int m, int n, int k,
                          int32_t* ids, float* w, hipStream_t st) {
  const dim3 grid((m + 3) / 4), blk(256);
  switch (nv_bucket(n)) {
    case 2: hipLaunchKernelGGL((topk_gate_partials_kernel<2>), grid, blk, 0, st, part, S, logits, bias, m, n, k, ids, w); break;
    case 4: hipLaunchKernelGGL((topk_gate_partials_kernel<4>), grid, blk, 0, st, part, S, logits, bias, m, n, k, ids, w); break;
    case 8: hipLaunchKernelGGL((topk_gate_partials_kernel<8>), grid, blk, 0, st, part, S, logits, bias, m, n, k, ids, w); break;
    case 14: hipLaunchKernelGGL((topk_gate_partials_kernel<14>), grid, blk, 0, st, part, S, logits, bias, m, n, k, ids, w); break;
    default: hipLaunchKernelGGL((topk_gate_partials_kernel<16>), grid, blk, 0, st, part, S, logits, bias, m, n, k, ids, w); break;
  }
}

// Sort + quant as separate launches. Returns the number of launches, or -1
// if the sort's LDS allowance could not be set (nothing launched).
bool wave_sort_fits(int P, int n) { return P <= std::min(kWaveSortMaxP, std::max(128, 5 * n / 8)); }

int launch_sort_quant(const int32_t* ids, const uint16_t* x, int64_t ldx, int m, int n, int k, int topk, int block,
                      int32_t* sorted_ids, int32_t* expert_ids, int32_t* offsets, uint8_t* a_q, uint8_t* a_scale,
                      bool fp4, char* ws, const Layout& L, hipStream_t st) {
  const int P = m * topk;
  int32_t* pos = reinterpret_cast<int32_t*>(ws + L.pos);
  int launches = 0;
  if (P <= kSmallSortMaxP) {
    // One wave sorts up to max(128, 5N/8) pairs, every wave above. Measured
    // (sort + quant, us, one wave vs sixteen): N = 128: P = 128: 8.4 / 8.5,
    // P = 256: 9.9 / 8.8, P = 512: 12.6 / 8.9; N = 896: P = 512: 15.2 / 16.5,
    // P = 1024: 17.1 / 17.1. The sixteen waves' per-expert scans grow with N.
    const int threads = wave_sort_fits(P, n) ? 256 : 1024;
    const size_t lds =
        sizeof(int) * ((size_t)P + std::max<size_t>(P, (size_t)(threads / 64) * n) + n + (n + 1) + threads);
    // Above 64 KB of dynamic LDS the kernel must be allowed more: the largest
    // need (P = 8192, N = 1024, sixteen waves) is 110.6 KB, which with the
    // kernel's static LDS stays under the 160 KB of a CU.
    if (lds > 65536 && !g_sort_lds_set.load()) {
      if (hipFuncSetAttribute(reinterpret_cast<const void*>(sort_small_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, kSortSmallMaxLds) != hipSuccess)
        return -1;
      g_sort_lds_set.store(true);
    }
    hipLaunchKernelGGL(sort_small_kernel, dim3(1), dim3(threads), lds, st, ids, P, n, block, sorted_ids, expert_ids,
                       offsets, pos);
    ++launches;
  } else {
    const int G = large_sort_groups(P);
    int32_t* ghist = reinterpret_cast<int32_t*>(ws + L.ghist);
    int32_t* offws = reinterpret_cast<int32_t*>(ws + L.offws);
    hipLaunchKernelGGL(sort_hist_kernel, dim3(G), dim3(256), sizeof(int) * n, st, ids, P, n, kLargeSortChunk,
                       ghist);
    hipLaunchKernelGGL(sort_colscan_kernel, dim3((n + 63) / 64), dim3(64 * kColscanWaves), 0, st, ghist, G, n,
                       offws);
    hipLaunchKernelGGL(sort_scan_kernel, dim3(1), dim3(1024), sizeof(int) * ((size_t)(n + 1) + 1024), st, n, block,
                       offws);
    hipLaunchKernelGGL(sort_scatter_kernel, dim3(G), dim3(256), sizeof(int) * (4 * (size_t)n + n + (n + 1) + n), st,
                       ids, P, n, block, kLargeSortChunk, ghist, offws, sorted_ids, expert_ids, offsets, pos);
    launches += 4;
  }
  const int units = m * (k / 16);
  hipLaunchKernelGGL(quant_kernel, dim3((units + 255) / 256), dim3(256), 0, st, x, ldx, m, k, topk, pos, a_q,
                     a_scale, fp4 ? 1 : 0);
  return launches + 1;
}

// ---------------------------------------------------------------------------
// Fused launch (M <= 64).
// ---------------------------------------------------------------------------
// Small mode when one gather of every row fits the per-thread loads, every
// wave has at most one row's gate to run, and a lane holds at most two
// experts. Measured on MI355X (small vs large mode, us, M = 1 / 2 / 4, W
// rotating through 8 copies): N = 128, K = 6144: 5.3 / 6.0 / 7.2 vs 6.6 /
// 6.9 / 7.9; N = 256: 8.8 / 9.6 / 11.0 vs 8.4 / 8.6 / 9.7; N = 896, K = 3584,
// top-16: 15.9 / 18.5 / 21.4 vs 11.4 / 11.7 / 12.5. With more experts every
// participant's gate of the whole row costs more than the ids hand-off.
bool fused_small(const Plan& p, int m, int n) {
  const int mode = config().force_mode;
  if (mode == kModeLarge) return false;
  return m <= 4 && (n <= 128 || mode == kModeSmall) && gather_loads(m, n, p.s) <= kPollLoads;
}

size_t fused_lds_bytes(const Plan& p, int m, int n, int topk, bool small) {
  const int P = m * topk;
  const int rows = small ? m : 1;
  // small mode above four experts a lane: n ints a wave to hand the winners
  // to their owner lanes
  const size_t flags = (small && n > 256) ? 4 * (size_t)n : 0;
  // a staged gather keeps every slice's partials in the logits' place
  const size_t stage = fused_gather_staged(rows, n, p.s) ? (size_t)(p.s - 1) * rows * n : 0;
  const size_t tail = sizeof(int) * ((size_t)fused_tail_ints(P, n, rows) + stage + flags);
  const size_t tile = p.valu ? 0 : sizeof(float) * 4 * p.mt * 256;
  return std::max(tail, tile);
}

const void* fused_kernel_for(const Plan& p, int n, bool norm) {
  if (norm) {
    switch (nv_bucket(n)) {
      case 2: return fused_norm_pick_nv2(p.valu, p.mt, p.l, p.ks);
      case 4: return fused_norm_pick_nv4(p.valu, p.mt, p.l, p.ks);
      case 8: return fused_norm_pick_nv8(p.valu, p.mt, p.l, p.ks);
      case 14: return fused_norm_pick_nv14(p.valu, p.mt, p.l, p.ks);
      default: return fused_norm_pick_nv16(p.valu, p.mt, p.l, p.ks);
    }
  }
  switch (nv_bucket(n)) {
    case 2: return fused_pick_nv2(p.valu, p.mt, p.l, p.ks);
    case 4: return fused_pick_nv4(p.valu, p.mt, p.l, p.ks);
    case 8: return fused_pick_nv8(p.valu, p.mt, p.l, p.ks);
    case 14: return fused_pick_nv14(p.valu, p.mt, p.l, p.ks);
    default: return fused_pick_nv16(p.valu, p.mt, p.l, p.ks);
  }
}

// Largest co-resident grid for a kernel at this dynamic LDS size (cached).
struct OccKey {
  const void* fn;
  size_t lds;
  int dev;
  int blocks;
};
OccKey g_occ[256];
int g_occ_n = 0;

int coresident_blocks(const void* fn, size_t lds, int cus) {
  int d = 0;
  if (hipGetDevice(&d) != hipSuccess) d = 0;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    for (int i = 0; i < g_occ_n; ++i)
      if (g_occ[i].fn == fn && g_occ[i].lds == lds && g_occ[i].dev == d) return g_occ[i].blocks;
  }
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 256, lds) != hipSuccess) per_cu = 0;
  const int blocks = per_cu * cus;
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_occ_n < 256) g_occ[g_occ_n++] = OccKey{fn, lds, d, blocks};
  return blocks;
}

// ---------------------------------------------------------------------------
// Allocation-free variant of rgt_route_sort_quant: its workspace is this
// file-scope device array, one copy per GPU, held until the process ends.
// Host code never passes the array's name to the device: the address comes
// from hipGetSymbolAddress, taken once per device with that device current.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = 8u << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

void* g_scratch_ptr[64];

__global__ void __launch_bounds__(256) fill_zero_kernel(uint4* p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
    p[i] = make_uint4(0, 0, 0, 0);
}

// This device's scratch address. The first call on a device takes the
// symbol's address and zero-fills the array with a kernel on `stream` (one
// launch, counted in *launches).
rgt_status scratch_for(hipStream_t stream, void** out, int* launches) {
  int d = 0;
  if (hipGetDevice(&d) != hipSuccess || d < 0 || d >= 64) return RGT_ERR_HIP;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_scratch_ptr[d]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return RGT_ERR_HIP;
    hipLaunchKernelGGL(fill_zero_kernel, dim3(256), dim3(256), 0, stream, static_cast<uint4*>(p),
                       kScratchBytes / 16);
    if (hipGetLastError() != hipSuccess) return RGT_ERR_HIP;
    g_scratch_ptr[d] = p;
    ++*launches;
  }
  *out = g_scratch_ptr[d];
  return RGT_OK;
}

}  // namespace

// ===========================================================================
// C ABI
// ===========================================================================
extern "C" {

const char* rgt_status_string(rgt_status s) {
  switch (s) {
    case RGT_OK: return "ok";
    case RGT_ERR_UNSUPPORTED: return "shape outside coverage";
    case RGT_ERR_INVALID: return "invalid argument";
    case RGT_ERR_WORKSPACE: return "workspace null, misaligned or too small";
    case RGT_ERR_HIP: return "HIP runtime error";
    case RGT_ERR_TIMEOUT: return "device-side wait timed out";
  }
  return "unknown status";
}

int rgt_version(void) { return kVersion; }

int rgt_last_launch_count(void) { return g_last_launches; }

int64_t rgt_sort_capacity(int m, int n, int topk, int block) {
  if (m < 0 || m > 8192 || n < 1 || n > 1024 || !gate_covered(n, topk) || !block_covered(block)) return -1;
  const int64_t P = (int64_t)m * topk;
  const int64_t cap = P + std::min<int64_t>(n, P) * (block - 1);
  return (cap + block - 1) / block * block;
}

size_t rgt_workspace_bytes(int max_m, int n, int k, int topk, int block) {
  if (max_m < 1 || !covered(max_m, n, k) || !gate_covered(n, topk) || !block_covered(block)) return 0;
  size_t need = 0;
  for (int m = 1; m <= max_m; ++m) need = std::max(need, ws_need(m, n, k, topk));
  return need;
}

rgt_status rgt_router_supported(int m, int n, int k) {
  return covered(m, n, k) ? RGT_OK : RGT_ERR_UNSUPPORTED;
}

rgt_status rgt_reset_workspace(void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!ws || !aligned(ws, kAlign) || ws_bytes < kCtlBytes) return RGT_ERR_WORKSPACE;
  g_last_launches = 0;
  return hipMemsetAsync(ws, 0, ws_bytes, stream) == hipSuccess ? RGT_OK : RGT_ERR_HIP;
}

rgt_status rgt_check_workspace(const void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!ws || !aligned(ws, kAlign) || ws_bytes < kCtlBytes) return RGT_ERR_WORKSPACE;
  if (hipStreamSynchronize(stream) != hipSuccess) return RGT_ERR_HIP;
  u32 err = 0;
  if (hipMemcpy(&err, ws, sizeof(err), hipMemcpyDeviceToHost) != hipSuccess) return RGT_ERR_HIP;
  return (err & kErrTimeout) ? RGT_ERR_TIMEOUT : RGT_OK;
}

static rgt_status check_gemv_args(const void* x, int64_t ldx, const void* w, int64_t ldw, int m, int n, int k) {
  if (!covered(m, n, k)) return RGT_ERR_UNSUPPORTED;
  if (m == 0) return RGT_OK;
  if (!x || !w || !aligned(x, 16) || !aligned(w, 16)) return RGT_ERR_INVALID;
  if (ldx < k || ldw < k || ldx % 8 || ldw % 8) return RGT_ERR_INVALID;
  return RGT_OK;
}

static rgt_status check_ws(const void* ws, size_t ws_bytes, size_t need) {
  if (!ws || !aligned(ws, kAlign) || ws_bytes < need) return RGT_ERR_WORKSPACE;
  return RGT_OK;
}

rgt_status rgt_router_logits(const void* x, int64_t ldx, const void* w, int64_t ldw, float* logits, int m, int n,
                             int k, void* ws, size_t ws_bytes, hipStream_t stream) {
  g_last_launches = 0;
  rgt_status st = check_gemv_args(x, ldx, w, ldw, m, n, k);
  if (st != RGT_OK || m == 0) return st;
  if (!logits || !aligned(logits, 4)) return RGT_ERR_INVALID;
  const Layout L = make_layout(m, n, k, 1);
  if ((st = check_ws(ws, ws_bytes, L.total)) != RGT_OK) return st;
  const Plan p = make_plan(m, n, k);
  if (p.mb * p.nb > kMaxTileCounters) return RGT_ERR_UNSUPPORTED;
  char* base = static_cast<char*>(ws);
  GemvArgs a{static_cast<const u16*>(x), ldx, static_cast<const u16*>(w), ldw, logits,
             reinterpret_cast<float*>(base + L.part), reinterpret_cast<u32*>(base + L.ctr), m, n, k, p.s, p.nb};
  if (wide_gemm(m, n)) {
    // Wide batch: the same k-slice partials as the launch chain of
    // rgt_route_sort_quant, summed in the same order (same bits).
    g_last_launches = launch_chain_gemm(a, m, n, k, stream);
    const int S = chain_gemm_slices(m, n, k);
    if (S > 1) {
      const int64_t count = (int64_t)m * n;
      hipLaunchKernelGGL(sum_partials_kernel, dim3((unsigned)((count / 4 + 255) / 256)), dim3(256), 0, stream, a.part,
                         S, count, logits);
      ++g_last_launches;
    }
    return launched();
  }
  launch_router(a, p, stream);
  g_last_launches = 1;
  return launched();
}

rgt_status rgt_topk_gate(const float* logits, const float* bias, int m, int n, int topk, int32_t* topk_ids,
                         float* topk_w, hipStream_t stream) {
  g_last_launches = 0;
  if (m < 0 || m > 8192 || n < 16 || n > 1024 || n % 16 || !gate_covered(n, topk)) return RGT_ERR_UNSUPPORTED;
  if (m == 0) return RGT_OK;
  if (!logits || !topk_ids || !topk_w || !aligned(logits, 4) || !aligned(topk_ids, 4) || !aligned(topk_w, 4) ||
      (bias && !aligned(bias, 4)))
    return RGT_ERR_INVALID;
  launch_gate(logits, bias, m, n, topk, topk_ids, topk_w, stream);
  g_last_launches = 1;
  return launched();
}

rgt_status rgt_topk_gate_partials(const float* part, int s, const float* bias, int m, int n, int topk,
                                  float* logits, int32_t* topk_ids, float* topk_w, hipStream_t stream) {
  g_last_launches = 0;
  if (m < 0 || m > 8192 || n < 16 || n > 1024 || n % 16 || !gate_covered(n, topk) || s < 1 || s > 1024)
    return RGT_ERR_UNSUPPORTED;
  if (m == 0) return RGT_OK;
  if (!part || !topk_ids || !topk_w || !aligned(part, 4) || !aligned(topk_ids, 4) || !aligned(topk_w, 4) ||
      (bias && !aligned(bias, 4)) || (logits && !aligned(logits, 4)))
    return RGT_ERR_INVALID;
  launch_gate_partials(part, s, logits, bias, m, n, topk, topk_ids, topk_w, stream);
  g_last_launches = 1;
  return launched();
}

static rgt_status check_norm_args(const void* x, int64_t ldx, const void* residual, int64_t ldr, const void* gamma,
                                  float eps, int m, int k, const void* xn, int64_t ldxn, const void* residual_out,
                                  int64_t ldro, const float* rstd) {
  if (m < 0 || m > 65535 || k < 8 || k > 16384 || k % 8) return RGT_ERR_UNSUPPORTED;
  if (m == 0) return RGT_OK;
  if (!x || !gamma || !xn || !aligned(x, 16) || !aligned(gamma, 16) || !aligned(xn, 16)) return RGT_ERR_INVALID;
  if (ldx < k || ldx % 8 || ldxn < k || ldxn % 8 || !(eps >= 0.f)) return RGT_ERR_INVALID;
  if (residual && (!aligned(residual, 16) || ldr < k || ldr % 8)) return RGT_ERR_INVALID;
  if (residual_out && (!residual || !aligned(residual_out, 16) || ldro < k || ldro % 8)) return RGT_ERR_INVALID;
  if (rstd && !aligned(rstd, 4)) return RGT_ERR_INVALID;
  return RGT_OK;
}

static void launch_rmsnorm(const uint16_t* xs, int64_t ldx, const uint16_t* rs, int64_t ldr, const uint16_t* gs,
                           float eps, int m, int k, uint16_t* xo, int64_t ldxn, uint16_t* ro, int64_t ldro, float* rstd,
                           hipStream_t stream) {
  const int ch = (k + 2047) / 2048;  // 8-element chunks per thread
  const dim3 grid(m), blk(256);
  if (ch <= 1) hipLaunchKernelGGL(rmsnorm_kernel<1>, grid, blk, 0, stream, xs, ldx, rs, ldr, gs, eps, k, xo, ldxn, ro, ldro, rstd);
  else if (ch <= 2) hipLaunchKernelGGL(rmsnorm_kernel<2>, grid, blk, 0, stream, xs, ldx, rs, ldr, gs, eps, k, xo, ldxn, ro, ldro, rstd);
  else if (ch <= 4) hipLaunchKernelGGL(rmsnorm_kernel<4>, grid, blk, 0, stream, xs, ldx, rs, ldr, gs, eps, k, xo, ldxn, ro, ldro, rstd);
  else hipLaunchKernelGGL(rmsnorm_kernel<8>, grid, blk, 0, stream, xs, ldx, rs, ldr, gs, eps, k, xo, ldxn, ro, ldro, rstd);
}

void rgt_reload_env(void) {
  config();
  std::lock_guard<std::mutex> lk(g_cfg_mu);
  load_config();
}

rgt_status rgt_rmsnorm(const void* x, int64_t ldx, const void* residual, int64_t ldr, const void* gamma, float eps,
                       int m, int k, void* xn, int64_t ldxn, void* residual_out, int64_t ldro, float* rstd,
                       hipStream_t stream) {
  g_last_launches = 0;
  const rgt_status st = check_norm_args(x, ldx, residual, ldr, gamma, eps, m, k, xn, ldxn, residual_out, ldro, rstd);
  if (st != RGT_OK || m == 0) return st;
  launch_rmsnorm(static_cast<const uint16_t*>(x), ldx, static_cast<const uint16_t*>(residual), ldr,
                 static_cast<const uint16_t*>(gamma), eps, m, k, static_cast<uint16_t*>(xn), ldxn,
                 static_cast<uint16_t*>(residual_out), ldro, rstd, stream);
  g_last_launches = 1;
  return launched();
}

int rgt_router_partial_slices(int m, int n, int k) {
  if (m < 1 || m > kSharedMaxM || k > kSharedMaxK || !covered(m, n, k)) return 0;
  return make_plan(m, n, k).s;
}

rgt_status rgt_router_shared_swiglu(const void* x, int64_t ldx, const void* w, int64_t ldw, int m, int n, int k,
                                    float* part, int s, const uint8_t* wsh_q, const uint8_t* wsh_scale, int inter,
                                    void* h, int64_t ldh, hipStream_t stream) {
  g_last_launches = 0;
  if (m < 0 || m > kSharedMaxM || k > kSharedMaxK || inter < 1 || inter > (1 << 20)) return RGT_ERR_UNSUPPORTED;
  rgt_status st = check_gemv_args(x, ldx, w, ldw, m, n, k);
  if (st != RGT_OK || m == 0) return st;
  const Plan p = make_plan(m, n, k);
  if (s != p.s || !part || !aligned(part, 16)) return RGT_ERR_INVALID;
  if (!wsh_q || !aligned(wsh_q, 16) || !wsh_scale || !h || !aligned(h, 2) || ldh < inter) return RGT_ERR_INVALID;
  if (ldx > INT32_MAX) return RGT_ERR_UNSUPPORTED;  // passed to the kernel as a 32-bit scalar
  const void* fn = shared_pick(p.valu, p.mt, p.l, p.ks, m);
  if (!fn) return RGT_ERR_UNSUPPORTED;
  GemvArgs a{static_cast<const u16*>(x), ldx, static_cast<const u16*>(w), ldw, nullptr, part, nullptr, m, n, k,
             p.s, p.nb};
  SharedArgs b{static_cast<const u16*>(x), ldx, wsh_q, wsh_scale, static_cast<u16*>(h), ldh, m, k, inter};
  // the shared part's operands, preloaded into scalar registers (shared.h)
  int router_wgs = p.grid, sldx = (int)ldx, sk = k, sinter = inter, sm = m;
  const uint8_t* swq = wsh_q;
  const uint8_t* sws = wsh_scale;
  const u16* sx = static_cast<const u16*>(x);
  void* args[] = {&router_wgs, &swq, &sws, &sx, &sldx, &sk, &sinter, &sm, &a, &b};
  // shared-expert columns per workgroup, for the shared part's rows (the
  // VALU form of 8 rows up to 8, as shared_pick chooses)
  const int cols = shared_cols_per_wg(p.valu ? p.mt : (m <= 8 ? 8 : 16));
  const int grid = p.grid + (inter + cols - 1) / cols;
  if (hipLaunchKernel(fn, dim3(grid), dim3(256), args, 0, stream) != hipSuccess) return RGT_ERR_HIP;
  g_last_launches = 1;
  return launched();
}

static rgt_status check_sort_args(const void* x, int64_t ldx, int m, int n, int k, int topk, int block,
                                  const void* sorted_ids, const void* expert_ids, const void* offsets,
                                  const void* a_q, const void* a_scale) {
  if (!covered(m, n, k) || !gate_covered(n, topk) || !block_covered(block)) return RGT_ERR_UNSUPPORTED;
  if (m == 0) return RGT_OK;
  if (!x || !aligned(x, 16) || ldx < k || ldx % 8) return RGT_ERR_INVALID;
  if (!sorted_ids || !expert_ids || !offsets || !a_q || !a_scale) return RGT_ERR_INVALID;
  if (!aligned(sorted_ids, 4) || !aligned(expert_ids, 4) || !aligned(offsets, 4) || !aligned(a_q, 16) ||
      !aligned(a_scale, 4))
    return RGT_ERR_INVALID;
  return RGT_OK;
}

static rgt_status moe_sort_quant_impl(const int32_t* topk_ids, const void* x, int64_t ldx, int m, int n, int k,
                                      int topk, int block, int32_t* sorted_ids, int32_t* expert_ids,
                                      int32_t* offsets, uint8_t* a_q, uint8_t* a_scale, bool fp4, void* ws,
                                      size_t ws_bytes, hipStream_t stream) {
  g_last_launches = 0;
  rgt_status st = check_sort_args(x, ldx, m, n, k, topk, block, sorted_ids, expert_ids, offsets, a_q, a_scale);
  if (st != RGT_OK || m == 0) return st;
  if (!topk_ids || !aligned(topk_ids, 4)) return RGT_ERR_INVALID;
  const Layout L = make_layout(m, n, k, topk);
  if ((st = check_ws(ws, ws_bytes, L.total)) != RGT_OK) return st;
  const int nl = launch_sort_quant(topk_ids, static_cast<const uint16_t*>(x), ldx, m, n, k, topk, block, sorted_ids,
                                   expert_ids, offsets, a_q, a_scale, fp4, static_cast<char*>(ws), L, stream);
  if (nl < 0) return RGT_ERR_HIP;
  g_last_launches = nl;
  return launched();
}

rgt_status rgt_moe_sort_quant(const int32_t* topk_ids, const void* x, int64_t ldx, int m, int n, int k, int topk,
                              int block, int32_t* sorted_ids, int32_t* expert_ids, int32_t* offsets, uint8_t* a_q,
                              uint8_t* a_scale, void* ws, size_t ws_bytes, hipStream_t stream) {
  return moe_sort_quant_impl(topk_ids, x, ldx, m, n, k, topk, block, sorted_ids, expert_ids, offsets, a_q, a_scale,
                             false, ws, ws_bytes, stream);
}

rgt_status rgt_moe_sort_quant_mxfp4(const int32_t* topk_ids, const void* x, int64_t ldx, int m, int n, int k,
                                    int topk, int block, int32_t* sorted_ids, int32_t* expert_ids, int32_t* offsets,
                                    uint8_t* a_q, uint8_t* a_scale, void* ws, size_t ws_bytes, hipStream_t stream) {
  return moe_sort_quant_impl(topk_ids, x, ldx, m, n, k, topk, block, sorted_ids, expert_ids, offsets, a_q, a_scale,
                             true, ws, ws_bytes, stream);
}

// Everything a route call decides from its shape, computed once per (device,
// M, N, K, top-k, norm in the launch, settings) and kept: the plan, the
// workspace layout and, for the one-launch form, the kernel, its LDS, the
// tail's mode and quant units per workgroup, and whether it fits at all
// (co-residency, per-thread loads, quant units, wave-sized pair lists).
struct ShapeEntry {
  int dev, m, n, k, topk;
  bool want_norm;
  unsigned gen;
  Plan p;
  Layout L;
  bool fuse, norm_in, small;
  int upw_log;
  const void* fn;
  size_t lds;
};
constexpr int kShapeCache = 1024;
static ShapeEntry g_shapes[kShapeCache];
static int g_shapes_n = 0;

static ShapeEntry compute_shape(int dev, int m, int n, int k, int topk, bool want_norm) {
  const Config& cfg = config();
  ShapeEntry e{};
  e.dev = dev, e.m = m, e.n = n, e.k = k, e.topk = topk, e.want_norm = want_norm, e.gen = cfg.gen;
  e.p = make_plan(m, n, k);
  e.L = make_layout(m, n, k, topk);
  const Plan& p = e.p;
  e.fuse = m <= kFusedMaxM && !cfg.no_fuse;
  e.norm_in = want_norm && e.fuse && m <= p.grid;
  e.small = fused_small(p, m, n);
  e.upw_log = 8;
  if (e.fuse) {
    DevInfo di;
    if (!dev_info(di)) {
      e.fuse = e.norm_in = false;
      return e;
    }
    e.fn = fused_kernel_for(p, n, e.norm_in);
    e.lds = fused_lds_bytes(p, m, n, topk, e.small);
    const int units = m * (k / 16);
    // A workgroup's quant units cover at most this many tokens; their pairs
    // must fit one wave.
    const int cpr = k / 16;
    auto pairs_fit_at = [&](int ul) {
      return (((1 << ul) - 1) / cpr + 2) * topk <= 64 &&
             (uint64_t)(p.grid << ul) * (uint64_t)cpr < (1ull << 32);  // exact magic division
    };
    if (e.small) {
      // the fewest units per workgroup that cover every unit
      e.upw_log = 6;
      while (e.upw_log < 8 && ((units + (1 << e.upw_log) - 1) >> e.upw_log) > p.grid) ++e.upw_log;
    } else {
      // large mode: the most units per workgroup whose pairs fit one wave
      // (fewer, fuller quant workgroups; measured faster at M >= 16)
      while (e.upw_log > 6 && !pairs_fit_at(e.upw_log) && units <= (p.grid << (e.upw_log - 1))) --e.upw_log;
    }
    // Co-residency is required for the device-side waits; each thread owns at
    // most one quant unit; in large mode workgroup r gathers row r.
    if (p.grid > coresident_blocks(e.fn, e.lds, di.cus) || units > (p.grid << e.upw_log) ||
        !pairs_fit_at(e.upw_log) || (!e.small && (m > p.grid || gather_loads(1, n, p.s) > kPollLoads)))
      e.fuse = false;
  }
  if (!e.fuse) e.norm_in = false;
  if (cfg.log) {
    if (e.fuse)
      std::fprintf(stderr,
                   "rgt: route M=%d N=%d K=%d top-%d%s: one launch, %s tile (mt %d, %s %d), %d k-slices, grid %d, "
                   "%s mode, %d quant units a workgroup\n",
                   m, n, k, topk, want_norm ? (e.norm_in ? " behind the norm" : " (norm launch first)") : "",
                   p.valu ? "VALU" : "MFMA", p.mt, p.valu ? "l" : "ks", p.valu ? p.l : p.ks, p.s, p.grid,
                   e.small ? "small" : "large", 1 << e.upw_log);
    else
      std::fprintf(stderr, "rgt: route M=%d N=%d K=%d top-%d%s: launch chain (%s)\n", m, n, k, topk,
                   want_norm ? " (norm launch first)" : "", wide_gemm(m, n) ? "GEMM" : p.valu ? "VALU tile" : "MFMA tile");
  }
  return e;
}

// The cached entry (entries are never changed once in the table), or one
// held in a thread-local slot when the table is full.
static const ShapeEntry* shape_entry(int m, int n, int k, int topk, bool want_norm) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = -1;  // no device: no one-launch form (argument checks still run)
  const unsigned gen = config().gen;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    for (int i = 0; i < g_shapes_n; ++i) {
      const ShapeEntry& e = g_shapes[i];
      if (e.m == m && e.n == n && e.k == k && e.topk == topk && e.want_norm == want_norm && e.dev == dev &&
          e.gen == gen)
        return &e;
    }
  }
  const ShapeEntry e = compute_shape(dev, m, n, k, topk, want_norm);
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_shapes_n < kShapeCache) {
    g_shapes[g_shapes_n] = e;
    return &g_shapes[g_shapes_n++];
  }
  thread_local ShapeEntry spill;
  spill = e;
  return &spill;
}

// The RMSNorm producer in front of the router: x is the raw input; xn, h and
// rstd are written as rgt_rmsnorm writes them, and the router reads xn.
struct NormIn {
  const uint16_t* res;
  int64_t ldr;
  const uint16_t* gamma;
  float eps;
  uint16_t* xn;
  int64_t ldxn;
  uint16_t* res_out;
  int64_t ldro;
  float* rstd;
};

static rgt_status route_sort_quant_impl(const void* x, int64_t ldx, const void* w, int64_t ldw, const float* bias,
                                        int m, int n, int k, int topk, int block, float* logits, int32_t* topk_ids,
                                        float* topk_w, int32_t* sorted_ids, int32_t* expert_ids, int32_t* offsets,
                                        uint8_t* a_q, uint8_t* a_scale, bool fp4, void* ws, size_t ws_bytes,
                                        hipStream_t stream, const NormIn* nrm = nullptr) {
  g_last_launches = 0;
  rgt_status st = check_gemv_args(x, ldx, w, ldw, m, n, k);
  if (st != RGT_OK) return st;
  st = check_sort_args(x, ldx, m, n, k, topk, block, sorted_ids, expert_ids, offsets, a_q, a_scale);
  if (st != RGT_OK || m == 0) return st;
  if (nrm && (st = check_norm_args(x, ldx, nrm->res, nrm->ldr, nrm->gamma, nrm->eps, m, k, nrm->xn, nrm->ldxn,
                                   nrm->res_out, nrm->ldro, nrm->rstd)) != RGT_OK)
    return st;
  if (!topk_ids || !topk_w || !aligned(topk_ids, 4) || !aligned(topk_w, 4)) return RGT_ERR_INVALID;
  if ((logits && !aligned(logits, 4)) || (bias && !aligned(bias, 4))) return RGT_ERR_INVALID;
  const Config& cfg = config();
  // Behind the norm: inside the launch the first M workgroups are the rows'
  // norm workgroups and hold a row in registers (kNormChunks 8-element chunks
  // a thread); otherwise the norm's own launch comes first and the route
  // reads its xn. By default the norm joins the launch for one row only:
  // there every workgroup takes the row's rstd itself, measured faster than
  // the two launches (7.5 vs 8.4 us at N = 128, K = 6144); with more rows the
  // tiles of every n-block normalise the same columns again and wait for the
  // published rstd, measured slower than the norm's own launch (M = 2..64:
  // +0.4..+2.7 us). RGT_NORM_IN_LAUNCH = 1 takes the one launch whenever it
  // fits, 0 never.
  const bool want_norm = nrm && m <= kFusedMaxM && !cfg.no_fuse && k <= 2048 * kNormChunks &&
                         (cfg.norm_in_launch > 0 || (cfg.norm_in_launch < 0 && m == 1));
  const ShapeEntry* se = shape_entry(m, n, k, topk, want_norm);
  if (!se) return RGT_ERR_HIP;
  const Plan& p = se->p;
  const Layout& L = se->L;
  if ((st = check_ws(ws, ws_bytes, L.total)) != RGT_OK) return st;
  if (p.mb * p.nb > kMaxTileCounters) return RGT_ERR_UNSUPPORTED;
  char* base = static_cast<char*>(ws);
  float* lg = logits ? logits : reinterpret_cast<float*>(base + L.logits);
  GemvArgs g{static_cast<const u16*>(x), ldx, static_cast<const u16*>(w), ldw, lg,
             reinterpret_cast<float*>(base + L.part), reinterpret_cast<u32*>(base + L.ctr), m, n, k, p.s, p.nb};
  const bool fuse = se->fuse;
  bool norm_in = se->norm_in;
  int n_norm = 0;
  auto norm_first = [&]() {
    norm_in = false;
    if (!nrm || n_norm) return;
    launch_rmsnorm(g.x, ldx, nrm->res, nrm->ldr, nrm->gamma, nrm->eps, m, k, nrm->xn, nrm->ldxn, nrm->res_out,
                   nrm->ldro, nrm->rstd, stream);
    n_norm = 1;
    g.x = nrm->xn;
    g.ldx = nrm->ldxn;
    x = nrm->xn;
    ldx = nrm->ldxn;
  };
  if (!norm_in) norm_first();
  const bool small = se->small;
  const int upw_log = se->upw_log;
  const void* fn = se->fn;
  const size_t lds = se->lds;
  // (the one-launch kernels take the row strides as 32-bit scalars)
  if (fuse && ldx <= INT32_MAX && ldw <= INT32_MAX) {
    const u32 cpr_magic = 0xFFFFFFFFu / (u32)(k / 16) + 1u;  // exact for unit * (K/16) < 2^32
    // The scrub sweeps the workspace past the tile counters (in the trace
    // build, up to the phase stamps); this call's tagged words are skipped.
#ifdef RGT_TRACE
    const size_t scrub_end = L.trace;
#else
    const size_t scrub_end = ws_bytes / 16 * 16;
#endif
    // This call's footprint: the words it writes with its tag, all of them
    // (the scrub leaves them alone; a word in the footprint left unwritten
    // would keep an old tag for good): the partials; in large mode the
    // expert ids; behind the norm the rstd words (contiguous with the ids;
    // none with one row, whose rstd every workgroup takes itself).
    const u32 part0 = (u32)((L.tpart - L.part) / 16);
    const u32 ids0 = (u32)(((small ? L.trs : L.tids) - L.part) / 16);
    const u32 ids1 = (u32)((L.trs - L.part) / 16) + (norm_in && m > 1 ? (u32)(even_up(m) / 2) : 0u);
    FusedArgs a{g, bias, topk, block, small ? 1 : 0, fp4 ? 1 : 0, upw_log, cpr_magic, logits, topk_ids, topk_w, sorted_ids, expert_ids, offsets,
                a_q, a_scale, reinterpret_cast<u32*>(base + L.ctl), reinterpret_cast<u64*>(base + L.tpart),
                reinterpret_cast<u64*>(base + L.tids), wait_budget_ticks(), cfg.fault_inject,
#ifdef RGT_TRACE
                reinterpret_cast<u64*>(base + L.trace),
#else
                nullptr,
#endif
                reinterpret_cast<u64*>(base + L.part), (u32)((scrub_end - L.part) / 16),
                part0, part0 + (u32)(((size_t)p.s * m * n * 8 + 15) / 16),
                ids0, std::max(ids0, ids1)};
    if (norm_in) {
      a.res = nrm->res;
      a.ldr = nrm->ldr;
      a.gamma = nrm->gamma;
      a.eps = nrm->eps;
      a.xn = nrm->xn;
      a.ldxn = nrm->ldxn;
      a.res_out = nrm->res_out;
      a.ldro = nrm->ldro;
      a.rstd_out = nrm->rstd;
      a.trs = reinterpret_cast<u64*>(base + L.trs);
    }
    // the tile's operands, preloaded into scalar registers (fused.h)
    const u16* tx = a.g.x;
    const u16* tw = a.g.w;
    int tldx = (int)a.g.ldx, tldw = (int)a.g.ldw, tm = a.g.m, nbc = p.nb, mbc = p.valu ? 1 : p.mb;
    // reciprocals, exact for t * d < 2^32 (a divisor of 1 is not divided by)
    u32 nbm = nbc > 1 ? 0xFFFFFFFFu / (u32)nbc + 1u : 0u, mbm = mbc > 1 ? 0xFFFFFFFFu / (u32)mbc + 1u : 0u;
    int tgrid = p.grid;
    void* args[] = {&tx, &tw, &tldx, &tldw, &tm, &nbc, &nbm, &mbc, &mbm, &tgrid, &a};
    if (hipLaunchKernel(fn, dim3(p.grid), dim3(256), args, lds, stream) != hipSuccess) return RGT_ERR_HIP;
    g_last_launches = n_norm + 1;
    return launched();
  }
  norm_first();  // the one-launch form did not fit: the norm's launch, then the chain
  if (wide_gemm(m, n)) {
    // Wide batch: the router GEMM writes k-slice partials, the gate sums them
    // in slice order and writes the logits.
    const int S = chain_gemm_slices(m, n, k);
    launch_chain_gemm(g, m, n, k, stream);
    if (S > 1) launch_gate_partials(g.part, S, logits, bias, m, n, topk, topk_ids, topk_w, stream);
    else launch_gate(lg, bias, m, n, topk, topk_ids, topk_w, stream);
  } else {
    launch_router(g, p, stream);
    launch_gate(lg, bias, m, n, topk, topk_ids, topk_w, stream);
  }
  const int nl = launch_sort_quant(topk_ids, static_cast<const uint16_t*>(x), ldx, m, n, k, topk, block, sorted_ids,
                                   expert_ids, offsets, a_q, a_scale, fp4, base, L, stream);
  if (nl < 0) return RGT_ERR_HIP;
  g_last_launches = n_norm + 2 + nl;
  return launched();
}

rgt_status rgt_route_sort_quant(const void* x, int64_t ldx, const void* w, int64_t ldw, const float* bias, int m,
                                int n, int k, int topk, int block, float* logits, int32_t* topk_ids, float* topk_w,
                                int32_t* sorted_ids, int32_t* expert_ids, int32_t* offsets, uint8_t* a_q,
                                uint8_t* a_scale, void* ws, size_t ws_bytes, hipStream_t stream) {
  return route_sort_quant_impl(x, ldx, w, ldw, bias, m, n, k, topk, block, logits, topk_ids, topk_w, sorted_ids,
                               expert_ids, offsets, a_q, a_scale, false, ws, ws_bytes, stream);
}

rgt_status rgt_route_sort_quant_mxfp4(const void* x, int64_t ldx, const void* w, int64_t ldw, const float* bias,
                                      int m, int n, int k, int topk, int block, float* logits, int32_t* topk_ids,
                                      float* topk_w, int32_t* sorted_ids, int32_t* expert_ids, int32_t* offsets,
                                      uint8_t* a_q, uint8_t* a_scale, void* ws, size_t ws_bytes,
                                      hipStream_t stream) {
  return route_sort_quant_impl(x, ldx, w, ldw, bias, m, n, k, topk, block, logits, topk_ids, topk_w, sorted_ids,
                               expert_ids, offsets, a_q, a_scale, true, ws, ws_bytes, stream);
}

static rgt_status rmsnorm_route_impl(const void* x, int64_t ldx, const void* residual, int64_t ldr,
                                     const void* gamma, float eps, const void* w, int64_t ldw, const float* bias,
                                     int m, int n, int k, int topk, int block, void* xn, int64_t ldxn,
                                     void* residual_out, int64_t ldro, float* rstd, float* logits, int32_t* topk_ids,
                                     float* topk_w, int32_t* sorted_ids, int32_t* expert_ids, int32_t* offsets,
                                     uint8_t* a_q, uint8_t* a_scale, bool fp4, void* ws, size_t ws_bytes,
                                     hipStream_t stream) {
  const NormIn nrm{static_cast<const uint16_t*>(residual), ldr, static_cast<const uint16_t*>(gamma), eps,
                   static_cast<uint16_t*>(xn), ldxn, static_cast<uint16_t*>(residual_out), ldro, rstd};
  return route_sort_quant_impl(x, ldx, w, ldw, bias, m, n, k, topk, block, logits, topk_ids, topk_w, sorted_ids,
                               expert_ids, offsets, a_q, a_scale, fp4, ws, ws_bytes, stream, &nrm);
}

rgt_status rgt_rmsnorm_route_sort_quant(const void* x, int64_t ldx, const void* residual, int64_t ldr,
                                        const void* gamma, float eps, const void* w, int64_t ldw, const float* bias,
                                        int m, int n, int k, int topk, int block, void* xn, int64_t ldxn,
                                        void* residual_out, int64_t ldro, float* rstd, float* logits,
                                        int32_t* topk_ids, float* topk_w, int32_t* sorted_ids, int32_t* expert_ids,
                                        int32_t* offsets, uint8_t* a_q, uint8_t* a_scale, void* ws, size_t ws_bytes,
                                        hipStream_t stream) {
  return rmsnorm_route_impl(x, ldx, residual, ldr, gamma, eps, w, ldw, bias, m, n, k, topk, block, xn, ldxn,
                            residual_out, ldro, rstd, logits, topk_ids, topk_w, sorted_ids, expert_ids, offsets, a_q,
                            a_scale, false, ws, ws_bytes, stream);
}

rgt_status rgt_rmsnorm_route_sort_quant_mxfp4(const void* x, int64_t ldx, const void* residual, int64_t ldr,
                                              const void* gamma, float eps, const void* w, int64_t ldw,
                                              const float* bias, int m, int n, int k, int topk, int block, void* xn,
                                              int64_t ldxn, void* residual_out, int64_t ldro, float* rstd,
                                              float* logits, int32_t* topk_ids, float* topk_w, int32_t* sorted_ids,
                                              int32_t* expert_ids, int32_t* offsets, uint8_t* a_q, uint8_t* a_scale,
                                              void* ws, size_t ws_bytes, hipStream_t stream) {
  return rmsnorm_route_impl(x, ldx, residual, ldr, gamma, eps, w, ldw, bias, m, n, k, topk, block, xn, ldxn,
                            residual_out, ldro, rstd, logits, topk_ids, topk_w, sorted_ids, expert_ids, offsets, a_q,
                            a_scale, true, ws, ws_bytes, stream);
}

rgt_status rgt_route_sort_quant_noalloc(const void* x, int64_t ldx, const void* w, int64_t ldw, const float* bias,
                                        int m, int n, int k, int topk, int block, float* logits, int32_t* topk_ids,
                                        float* topk_w, int32_t* sorted_ids, int32_t* expert_ids, int32_t* offsets,
                                        uint8_t* a_q, uint8_t* a_scale, hipStream_t stream) {
  g_last_launches = 0;
  rgt_status st = check_gemv_args(x, ldx, w, ldw, m, n, k);
  if (st != RGT_OK) return st;
  st = check_sort_args(x, ldx, m, n, k, topk, block, sorted_ids, expert_ids, offsets, a_q, a_scale);
  if (st != RGT_OK || m == 0) return st;
  if (!topk_ids || !topk_w || !aligned(topk_ids, 4) || !aligned(topk_w, 4)) return RGT_ERR_INVALID;
  if ((logits && !aligned(logits, 4)) || (bias && !aligned(bias, 4))) return RGT_ERR_INVALID;
  if (ws_need(m, n, k, topk) > kScratchBytes) return RGT_ERR_UNSUPPORTED;  // beyond the scratch array
  void* ws = nullptr;
  int fills = 0;
  if ((st = scratch_for(stream, &ws, &fills)) != RGT_OK) return st;
  st = route_sort_quant_impl(x, ldx, w, ldw, bias, m, n, k, topk, block, logits, topk_ids, topk_w, sorted_ids,
                             expert_ids, offsets, a_q, a_scale, false, ws, kScratchBytes, stream);
  g_last_launches += fills;
  return st;
}

rgt_status rgt_moe_stage1_swiglu(const uint8_t* a_q, const uint8_t* a_scale, const int32_t* sorted_ids,
                                 const int32_t* expert_ids, const int32_t* offsets, int m, int n, int k, int topk,
                                 int block, const uint8_t* w_q, const uint8_t* w_scale, int inter, void* h,
                                 int64_t ldh, hipStream_t stream) {
  g_last_launches = 0;
  if (!covered(m, n, k) || !gate_covered(n, topk) || !block_covered(block) || inter < 16 || inter > (1 << 16) ||
      inter % 16)
    return RGT_ERR_UNSUPPORTED;
  if (m == 0) return RGT_OK;
  if (!a_q || !a_scale || !sorted_ids || !expert_ids || !offsets || !w_q || !w_scale || !h) return RGT_ERR_INVALID;
  if (!aligned(a_q, 16) || !aligned(w_q, 16) || !aligned(sorted_ids, 4) || !aligned(expert_ids, 4) ||
      !aligned(offsets, 4) || !aligned(h, 2) || ldh < inter)
    return RGT_ERR_INVALID;
  const int64_t cap = rgt_sort_capacity(m, n, topk, block);
  Stage1Args a{a_q, a_scale, sorted_ids, expert_ids, offsets, w_q, w_scale, static_cast<uint16_t*>(h), ldh,
               n, k, inter, block, m * topk};
  // Few row tiles (small batches): the four waves of a workgroup split K for
  // 16 columns. Else two column tiles a wave (the A fragment feeds four MFMAs)
  // once the grid has enough workgroups without it, one below.
  const unsigned tiles = (unsigned)(cap / 16);
  if ((int64_t)tiles * ((inter + 63) / 64) < RGT_STAGE1_KSPLIT_BELOW)
    hipLaunchKernelGGL(moe_stage1_ksplit_kernel, dim3(tiles, (unsigned)((inter + 15) / 16)), dim3(256), 0, stream, a);
  else if ((int64_t)tiles * ((inter + 127) / 128) >= RGT_STAGE1_JT2_FROM)
    hipLaunchKernelGGL(moe_stage1_kernel<2>, dim3(tiles, (unsigned)((inter + 127) / 128)), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(moe_stage1_kernel<1>, dim3(tiles, (unsigned)((inter + 63) / 64)), dim3(256), 0, stream, a);
  g_last_launches = 1;
  return launched();
}

#ifdef RGT_TRACE
// Trace build only: byte offset of the phase stamps inside the workspace for a
// fused call of this shape, and the number of workgroups that write them.
size_t rgt_trace_offset(int m, int n, int k, int topk, int* grid) {
  if (grid) *grid = make_plan(m, n, k).grid;
  return make_layout(m, n, k, topk).trace;
}
#endif

rgt_status rgt_diag_read(const void* src, size_t bytes, uint32_t* sink, int grid, hipStream_t stream) {
  g_last_launches = 0;
  if (!src || !sink || !aligned(src, 16) || !aligned(sink, 4) || bytes % 16 || grid < 1 || grid > 65536)
    return RGT_ERR_INVALID;
  hipLaunchKernelGGL(diag_read_kernel, dim3(grid), dim3(256), 0, stream, static_cast<const uint4*>(src), bytes / 16,
                     sink);
  g_last_launches = 1;
  return launched();
}

rgt_status rgt_diag_copy(const void* src, void* dst, size_t bytes, int grid, hipStream_t stream) {
  g_last_launches = 0;
  if (!src || !dst || !aligned(src, 16) || !aligned(dst, 16) || bytes % 16 || grid < 1 || grid > 65536)
    return RGT_ERR_INVALID;
  hipLaunchKernelGGL(diag_copy_kernel, dim3(grid), dim3(256), 0, stream, static_cast<const uint4*>(src),
                     static_cast<uint4*>(dst), bytes / 16);
  g_last_launches = 1;
  return launched();
}

}  // extern "C"
