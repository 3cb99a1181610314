// stage1.h - the routed experts' stage-1 GEMM on the sorted segments.
//
// The sorted, quantised activations of the front end feed the routed
// experts' first GEMM ("Kimi-K3: fused MoE routing, sort, quant and
// epilogue", Modifications: the A8W4 fused MoE runs on the sort's outputs;
// MiniMax-M3.1-Flash MoE/GEMM kernels, Summary: MoE sorting + quant, the
// stage-1 activations). Every padded row p of the sort whose sorted_ids entry
// is a real pair is an MXFP8 row a (a_q[p], a_scale[p]); its block's expert e
// (expert_ids[p / B]) has MXFP4 gate_up weights W_e [2I][K] (e2m1 codes two a
// byte, low nibble first; one e8m0 scale per 32 along K; gate rows first):
//
//   g = a . W_e[j],  u = a . W_e[I + j],  h[p][j] = bf16( silu(g) * u ),
//   silu(g) = g / (1 + exp(-g)), fp32.
//
// gfx950's block-scaled MFMA does the contraction in its native formats:
// v_mfma_scale_f32_16x16x128_f8f6f4 with A = e4m3 (16 rows of a), B = e2m1
// (16 weight rows), each 32-element block of either side scaled by its e8m0
// byte. Its operand layout (checked on the chip): for a 128-wide k step, lane
// l with r = l % 16, g = l / 16 holds A row r at k [16g, 16g + 16) and
// [64 + 16g, 80 + 16g) (two 16-byte halves), B row r at k [32g, 32g + 32)
// (16 bytes of packed codes), and the scale bytes of row r's k block g
// [32g, 32g + 32) for both sides; D lane l holds rows 4g + i, column r.
//
// A workgroup takes one 16-row tile of padded rows (inside one expert's
// segment: block sizes are multiples of 16) and 64 * JT output columns; wave
// w takes JT column tiles of 16, each as two MFMA tiles, the gate rows and the
// up rows, so g and u of an output land in the same lane and register and the
// SwiGLU needs no exchange (JT = 2 when the grid is large enough: the A
// fragment then feeds four MFMAs). Weights stream once per tile of rows; the
// 16 rows of a come from L2. Loads go four k steps (512 elements) at a time,
// the next group's loads issued before the current group's MFMAs.
#pragma once

#include "device.h"
#include "norm.h"

namespace rgt {

typedef int i32x8_t __attribute__((ext_vector_type(8)));

struct Stage1Args {
  const uint8_t* a_q;       // [cap][K] e4m3
  const uint8_t* a_scale;   // [cap][K/32] e8m0
  const int32_t* sorted_ids;
  const int32_t* expert_ids;
  const int32_t* offsets;   // [N+1]: offsets[N] the padded total
  const uint8_t* w_q;       // [N][2I][K/2] e2m1, two a byte
  const uint8_t* w_scale;   // [N][2I][K/32] e8m0
  uint16_t* h;              // [cap][ldh] bf16
  int64_t ldh;
  int n, k, inter, block, pairs;  // pairs = M * topk (the sentinel)
};

constexpr int kStage1Group = 4;  // k steps of 128 per load group (512 elements, 16 scale blocks)

// Step S of a load group: every tile's MFMA on the step's A fragment; op_sel
// S picks byte S of the scale words.
template <int S, int JT>
__device__ __forceinline__ void stage1_step(const uint4& a0, const uint4& a1, const uint4 (&b)[2 * JT][kStage1Group],
                                            u32 sa, const u32 (&sw)[2 * JT], floatx4_t (&acc)[2 * JT]) {
  const i32x8_t av = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
#pragma unroll
  for (int t = 0; t < 2 * JT; ++t) {
    const i32x8_t bv = {(int)b[t][S].x, (int)b[t][S].y, (int)b[t][S].z, (int)b[t][S].w, 0, 0, 0, 0};
    acc[t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc[t], 0, 4, S, (int)sa, S, (int)sw[t]);
  }
}

// One wave: 16 padded rows (p0 ..) x JT column tiles of 16 outputs (j, j + 16,
// ...), each tile a gate MFMA and an up MFMA on the same A fragment.
//
// K order inside a load group (any order works as long as A, B and the
// scales agree): at step s, hardware k block hb (the MFMA's k [32hb,
// 32hb + 32)) carries data block 4hb + s of the group. Then a lane's B bytes
// for the four steps are one contiguous 64-byte run, its scale bytes for the
// four steps one 4-byte word (the MFMA picks byte s with op_sel), and its A
// bytes two runs of four 16-byte chunks 32 bytes apart.
//
// Pad rows (sorted_ids = the sentinel) have no output, so their lanes read
// the tile's first row instead of their own (same addresses within the wave:
// one fetch), which at decode sizes, where most rows of a block are pads,
// cuts the A traffic from L2 several times over; their products are dropped.
// PF: load groups in flight ahead of the one being multiplied (1 or 2).
template <int JT, int PF = 1>
__device__ __forceinline__ void stage1_tile(const Stage1Args& a, int p0, int e, int j, int g0, int g1,
                                            floatx4_t (&acc)[2 * JT], int sid_r) {
  static_assert(PF == 1 || PF == 2, "one or two load groups ahead");
  const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
  const int K = a.k;
  const int prow = sid_r < a.pairs ? p0 + r : p0;  // sid_r = sorted_ids[p0 + r]
  const uint8_t* arow = a.a_q + (int64_t)prow * K + 128 * (g >> 1) + 16 * (g & 1);
  const u32* asc = reinterpret_cast<const u32*>(a.a_scale + (int64_t)prow * (K >> 5)) + g;
  const int64_t wrows = 2 * (int64_t)a.inter;
  const uint8_t* wb[2 * JT];
  const u32* sb[2 * JT];
#pragma unroll
  for (int t = 0; t < JT; ++t) {
    const int64_t rg = (int64_t)e * wrows + j + 16 * t + r, ru = rg + a.inter;
    wb[2 * t] = a.w_q + rg * (K >> 1) + 64 * g;
    wb[2 * t + 1] = a.w_q + ru * (K >> 1) + 64 * g;
    sb[2 * t] = reinterpret_cast<const u32*>(a.w_scale + rg * (K >> 5)) + g;
    sb[2 * t + 1] = reinterpret_cast<const u32*>(a.w_scale + ru * (K >> 5)) + g;
  }
#pragma unroll
  for (int t = 0; t < 2 * JT; ++t) acc[t] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  if (g0 >= g1) return;
  // The current group's operands and the next group's, as plain register
  // arrays with constant indices (a struct passed around by reference ends up
  // in scratch memory); the next group's loads go out before this group's
  // MFMAs, then the registers move over.
  uint4 a0[kStage1Group], a1[kStage1Group], b[2 * JT][kStage1Group];
  uint4 na0[kStage1Group], na1[kStage1Group], nb[2 * JT][kStage1Group];
  [[maybe_unused]] uint4 qa0[kStage1Group], qa1[kStage1Group], qb[2 * JT][kStage1Group];
  u32 sa, sw[2 * JT], nsa = 0, nsw[2 * JT];
  [[maybe_unused]] u32 qsa = 0, qsw[2 * JT];
#define RGT_STAGE1_LOAD(A0, A1, B, SA, SW, GRP)                                              \
  do {                                                                                     \
    const uint8_t* ar_ = arow + 512 * (GRP);                                               \
    _Pragma("unroll") for (int s_ = 0; s_ < kStage1Group; ++s_) {                          \
      A0[s_] = *reinterpret_cast<const uint4*>(ar_ + 32 * s_);                             \
      A1[s_] = *reinterpret_cast<const uint4*>(ar_ + 256 + 32 * s_);                       \
    }                                                                                      \
    SA = asc[4 * (GRP)];                                                                   \
    _Pragma("unroll") for (int t_ = 0; t_ < 2 * JT; ++t_) {                                \
      _Pragma("unroll") for (int s_ = 0; s_ < kStage1Group; ++s_)                          \
        B[t_][s_] = *reinterpret_cast<const uint4*>(wb[t_] + 256 * (GRP) + 16 * s_);        \
      SW[t_] = sb[t_][4 * (GRP)];                                                          \
    }                                                                                      \
  } while (0)
  RGT_STAGE1_LOAD(a0, a1, b, sa, sw, g0);
  if constexpr (PF == 2) {
    if (g0 + 1 < g1) RGT_STAGE1_LOAD(na0, na1, nb, nsa, nsw, g0 + 1);
  }
  for (int grp = g0; grp < g1; ++grp) {
    if constexpr (PF == 2) {
      if (grp + 2 < g1) RGT_STAGE1_LOAD(qa0, qa1, qb, qsa, qsw, grp + 2);
    } else {
      if (grp + 1 < g1) RGT_STAGE1_LOAD(na0, na1, nb, nsa, nsw, grp + 1);
    }
    stage1_step<0, JT>(a0[0], a1[0], b, sa, sw, acc);
    stage1_step<1, JT>(a0[1], a1[1], b, sa, sw, acc);
    stage1_step<2, JT>(a0[2], a1[2], b, sa, sw, acc);
    stage1_step<3, JT>(a0[3], a1[3], b, sa, sw, acc);
#pragma unroll
    for (int s = 0; s < kStage1Group; ++s) {
      a0[s] = na0[s];
      a1[s] = na1[s];
#pragma unroll
      for (int t = 0; t < 2 * JT; ++t) b[t][s] = nb[t][s];
      if constexpr (PF == 2) {
        na0[s] = qa0[s];
        na1[s] = qa1[s];
#pragma unroll
        for (int t = 0; t < 2 * JT; ++t) nb[t][s] = qb[t][s];
      }
    }
    sa = nsa;
#pragma unroll
    for (int t = 0; t < 2 * JT; ++t) sw[t] = nsw[t];
    if constexpr (PF == 2) {
      nsa = qsa;
#pragma unroll
      for (int t = 0; t < 2 * JT; ++t) nsw[t] = qsw[t];
    }
  }
#undef RGT_STAGE1_LOAD
}

// SwiGLU of a finished tile pair and the store of the pair rows. D lane l:
// rows 4g + i, column r of each tile. Which rows are pairs comes from the
// head's sorted ids (lane r of the wave holds row r's), as a wave ballot:
// no second read of sorted_ids before the stores. The whole wave calls it.
template <int JT>
__device__ __forceinline__ void stage1_store(const Stage1Args& a, int p0, int j, const floatx4_t (&acc)[2 * JT],
                                             int sid_r) {
  const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
  const u64 real = ballot64(sid_r < a.pairs);  // bit r (lanes 0..15): row p0 + r is a pair
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = p0 + 4 * g + i;
    if ((real >> (4 * g + i)) & 1) {
#pragma unroll
      for (int t = 0; t < JT; ++t) {
        const int col = j + 16 * t + r;
        if (col < a.inter) {
          const float gv = acc[2 * t][i], uv = acc[2 * t + 1][i];
          const float sgl = gv / (1.f + expf(-gv));
          a.h[(int64_t)p * a.ldh + col] = (uint16_t)bf16_rne(sgl * uv);
        }
      }
    }
  }
}

// Grid: (cap / 16) row tiles x ceil(I / (64 * JT)) column groups, 256
// threads; wave w takes output columns j0 + 16 * JT * w ...
// The tile's sort entries, loaded together ahead of any branch (they are in
// bounds for every row tile of the grid; past the padded total their values
// are not used): the padded total, the tile's first sorted id, its block's
// expert and the lane's row's sorted id: one memory round trip instead of
// four dependent ones.
struct Stage1Head {
  int total, sid0, e, sid_r;
};
__device__ __forceinline__ Stage1Head stage1_head(const Stage1Args& a, int p0) {
  Stage1Head h;
  h.total = a.offsets[a.n];
  h.sid0 = a.sorted_ids[p0];
  h.e = a.expert_ids[p0 >> (__ffs(a.block) - 1)];
  h.sid_r = a.sorted_ids[p0 + (threadIdx.x & 15)];
  return h;
}

template <int JT>
__global__ void __launch_bounds__(256) moe_stage1_kernel(Stage1Args a) {
  const int p0 = (int)blockIdx.x * 16;
  const Stage1Head h = stage1_head(a, p0);
  if (p0 >= h.total) return;    // past the padded total: no segment here
  if (h.sid0 >= a.pairs) return;  // pads only (pairs come first in a segment)
  const int j = ((int)blockIdx.y * 4 + (threadIdx.x >> 6)) * 16 * JT;
  if (j >= a.inter) return;
  floatx4_t acc[2 * JT];
  stage1_tile<JT, 2>(a, p0, h.e, j, 0, a.k / 512, acc, h.sid_r);
  stage1_store<JT>(a, p0, j, acc, h.sid_r);
}

// Small grids: the four waves of a workgroup split K (load groups w*G/4 ..
// (w+1)*G/4) for the same 16 output columns, and wave 0 adds the four parts
// in wave order through LDS (fixed order: deterministic). Grid: (cap / 16)
// row tiles x ceil(I / 16) column tiles.
__global__ void __launch_bounds__(256) moe_stage1_ksplit_kernel(Stage1Args a) {
  __shared__ floatx4_t s_part[3][2][64];
  const int p0 = (int)blockIdx.x * 16;
  const Stage1Head h = stage1_head(a, p0);
  if (p0 >= h.total) return;
  if (h.sid0 >= a.pairs) return;  // pads only
  const int j = (int)blockIdx.y * 16;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int G = a.k / 512;
  floatx4_t acc[2];
  stage1_tile<1, 2>(a, p0, h.e, j, wave * G / 4, (wave + 1) * G / 4, acc, h.sid_r);
  if (wave > 0) {
    s_part[wave - 1][0][lane] = acc[0];
    s_part[wave - 1][1][lane] = acc[1];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int w = 0; w < 3; ++w) {
      acc[0] += s_part[w][0][lane];
      acc[1] += s_part[w][1][lane];
    }
    stage1_store<1>(a, p0, j, acc, h.sid_r);
  }
}

}  // namespace rgt
