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
// segment: block sizes are multiples of 16) and 64 output columns; wave w
// takes the columns j0 + 16w .. + 16 as two MFMA tiles, the gate rows and the
// up rows, so g and u of an output land in the same lane and register and the
// SwiGLU needs no exchange. Weights stream once per tile of rows; the 16 rows
// of a come from L2. Loads go four k steps (512 elements) at a time, the next
// group's loads issued before the current group's MFMAs.
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

constexpr int kStage1Group = 4;  // k steps of 128 per load group

template <int NG>
__device__ __forceinline__ void stage1_tile(const Stage1Args& a, int p0, int e, int j) {
  const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
  const int K = a.k;
  const uint8_t* arow = a.a_q + (int64_t)(p0 + r) * K;
  const uint8_t* asc = a.a_scale + (int64_t)(p0 + r) * (K >> 5);
  const int64_t wrows = 2 * (int64_t)a.inter;
  const uint8_t* wg = a.w_q + ((int64_t)e * wrows + j + r) * (K >> 1);
  const uint8_t* wu = a.w_q + ((int64_t)e * wrows + a.inter + j + r) * (K >> 1);
  const uint8_t* sg = a.w_scale + ((int64_t)e * wrows + j + r) * (K >> 5);
  const uint8_t* su = a.w_scale + ((int64_t)e * wrows + a.inter + j + r) * (K >> 5);
  floatx4_t accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
  // one group: 4 steps of A (two 16-byte halves each), B gate and up (16
  // bytes each), and the scale byte of block 4s + g of every side
  struct Grp {
    uint4 a0[kStage1Group], a1[kStage1Group], bg[kStage1Group], bu[kStage1Group];
    uint8_t sa[kStage1Group], sg[kStage1Group], su[kStage1Group];
  };
  auto load = [&](Grp& q, int grp) {
#pragma unroll
    for (int s = 0; s < kStage1Group; ++s) {
      const int k0 = (grp * kStage1Group + s) * 128;
      q.a0[s] = *reinterpret_cast<const uint4*>(arow + k0 + 16 * g);
      q.a1[s] = *reinterpret_cast<const uint4*>(arow + k0 + 64 + 16 * g);
      q.bg[s] = *reinterpret_cast<const uint4*>(wg + (k0 >> 1) + 16 * g);
      q.bu[s] = *reinterpret_cast<const uint4*>(wu + (k0 >> 1) + 16 * g);
      const int blk = (k0 >> 5) + g;
      q.sa[s] = asc[blk];
      q.sg[s] = sg[blk];
      q.su[s] = su[blk];
    }
  };
  auto mma = [&](const Grp& q) {
#pragma unroll
    for (int s = 0; s < kStage1Group; ++s) {
      const i32x8_t av = {(int)q.a0[s].x, (int)q.a0[s].y, (int)q.a0[s].z, (int)q.a0[s].w,
                          (int)q.a1[s].x, (int)q.a1[s].y, (int)q.a1[s].z, (int)q.a1[s].w};
      const i32x8_t bgv = {(int)q.bg[s].x, (int)q.bg[s].y, (int)q.bg[s].z, (int)q.bg[s].w, 0, 0, 0, 0};
      const i32x8_t buv = {(int)q.bu[s].x, (int)q.bu[s].y, (int)q.bu[s].z, (int)q.bu[s].w, 0, 0, 0, 0};
      accg = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bgv, accg, 0, 4, 0, (int)q.sa[s], 0,
                                                             (int)q.sg[s]);
      accu = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, buv, accu, 0, 4, 0, (int)q.sa[s], 0,
                                                             (int)q.su[s]);
    }
  };
  const int groups = K / (128 * kStage1Group);
  Grp q[2];
  load(q[0], 0);
  for (int grp = 0; grp < groups; ++grp) {
    if (grp + 1 < groups) load(q[(grp + 1) & 1], grp + 1);
    mma(q[grp & 1]);
  }
  // D lane l: rows 4g + i, column r: output column j + r of padded rows p0 + 4g + i
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = p0 + 4 * g + i;
    if (a.sorted_ids[p] < a.pairs) {
      const float gv = accg[i], uv = accu[i];
      const float sgl = gv / (1.f + expf(-gv));
      a.h[(int64_t)p * a.ldh + j + r] = (uint16_t)bf16_rne(sgl * uv);
    }
  }
}

// Grid: (cap / 16) row tiles x ceil(I / 64) column groups, 256 threads.
__global__ void __launch_bounds__(256) moe_stage1_kernel(Stage1Args a) {
  const int p0 = (int)blockIdx.x * 16;
  const int total = a.offsets[a.n];
  if (p0 >= total) return;  // past the padded total: no segment here
  const int e = a.expert_ids[p0 >> (__ffs(a.block) - 1)];
  const int j = ((int)blockIdx.y * 4 + (threadIdx.x >> 6)) * 16;
  if (j >= a.inter) return;
  stage1_tile<kStage1Group>(a, p0, e, j);
}

}  // namespace rgt
