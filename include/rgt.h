/*
 * rgt.h - C ABI of the MI355X (gfx950) MoE routing front-end.
 *
 * The library computes, on one GPU:
 *   1. router logits   logits[M][N] fp32 = x[M][K] bf16 . W[N][K]^T bf16,
 *      as a split-K GEMV whose split-K reduction is finished inside the same
 *      launch by the last workgroup to arrive at each output tile, which then
 *      resets its arrival counter ("MiniMax-M3: Triton split-K router GEMV with
 *      in-kernel split-K fixup", sglang PR #36557, opening summary);
 *   2. a softmax top-k gate with renormalised weights (the gate of the
 *      MiniMax-M3.1-Flash MoE/GEMM kernels page, sglang PR #46691, Summary:
 *      Router; the routing step of "Kimi-K3: fused MoE routing, sort, quant
 *      and epilogue", sglang PR #46652, Modifications);
 *   3. the token -> expert sort into block-padded expert segments
 *      (sglang PR #46691, Summary: MoE sorting + quant; sglang PR #46652,
 *      review snippet: a pair's rank counts pairs of earlier tokens on the
 *      same expert);
 *   4. MXFP8 quantisation of the gathered activations: e4m3 codes plus one
 *      e8m0 scale per 32 elements (OCP Microscaling Formats v1.0; group-32
 *      scales as in the MXFP8 shared-expert commit of sgl-amd-mono PR #56).
 *
 * Conventions shared by every entry point
 *   - All data pointers are DEVICE pointers owned by the caller. The library
 *     never allocates device memory and never synchronises the stream, except
 *     rgt_check_workspace, which synchronises to read the error word.
 *   - bf16 tensors are passed as const void* holding IEEE bf16 bit patterns.
 *     x is row-major [M][ldx] with the K used elements of each row contiguous;
 *     W is row-major [N][ldw]. ldx, ldw count elements and must be >= K and
 *     multiples of 8 (16-byte aligned rows).
 *   - Every entry point is asynchronous on `stream` (0 = the null stream).
 *   - The workspace is caller-owned device memory of at least
 *     rgt_workspace_bytes(...) bytes, aligned to 256 bytes. It must be
 *     zero-filled ONCE when created (rgt_reset_workspace does this); every
 *     call leaves it ready for the next one (arrival counters back at zero;
 *     one phase counter only grows and is read relative to its value at the
 *     start of each call), so no memset is needed between calls. One
 *     workspace serves one stream: two calls that overlap in time on one
 *     workspace race on its counters.
 *   - Coverage. A shape outside coverage returns RGT_ERR_UNSUPPORTED and the
 *     caller may fall back to another implementation; this is the only status
 *     meant for fallback. Covered: 1 <= K, K % 512 == 0; 1 <= N <= 1024,
 *     N % 16 == 0; 1 <= topk <= min(N, 32); block in {16, 32, 64};
 *     0 <= M <= 8192.
 *   - M == 0 is a no-op returning RGT_OK (outputs untouched).
 *   - Null required pointers, misaligned pointers (x, W: 16 bytes; fp32/int32
 *     outputs and a_scale: 4 bytes; a_q: 16 bytes), ld < K or ld % 8 != 0 return
 *     RGT_ERR_INVALID. A workspace that is null, misaligned or too small
 *     returns RGT_ERR_WORKSPACE. A failed kernel launch returns RGT_ERR_HIP.
 *     Argument checks happen before any HIP call, so they never touch the GPU.
 *   - Inputs must be finite (no NaN or Inf in x, W, bias); results for
 *     non-finite inputs are unspecified.
 */
#ifndef RGT_H
#define RGT_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RGT_OK = 0,
  RGT_ERR_UNSUPPORTED = 1, /* shape outside coverage: caller may fall back   */
  RGT_ERR_INVALID = 2,     /* bad pointer, stride or argument                  */
  RGT_ERR_WORKSPACE = 3,   /* workspace null, misaligned or too small          */
  RGT_ERR_HIP = 4,         /* a HIP runtime call or kernel launch failed       */
  RGT_ERR_TIMEOUT = 5      /* a device-side wait passed its deadline           */
} rgt_status;

/* Static string naming a status code. */
const char* rgt_status_string(rgt_status s);

/* Library version as major*10000 + minor*100 + patch. */
int rgt_version(void);

/* Bytes of workspace needed for every call with 1 <= M <= max_m at this
 * (N, K, topk, block). Returns 0 when the shape is outside coverage. */
size_t rgt_workspace_bytes(int max_m, int n, int k, int topk, int block);

/* Sort capacity `cap`: an upper bound on the padded total, equal to
 * P + min(N, P)*(block-1) rounded up to a multiple of block, with P = M*topk.
 * Callers size sorted_ids to cap, expert_ids to cap/block, a_q to cap*K
 * bytes and a_scale to cap*K/32 bytes. Returns -1 outside coverage. */
int64_t rgt_sort_capacity(int m, int n, int topk, int block);

/* RGT_OK when (m, n, k) is inside the router's coverage, else
 * RGT_ERR_UNSUPPORTED. Host-only; never touches the GPU. */
rgt_status rgt_router_supported(int m, int n, int k);

/* Zero-fill a workspace on `stream` (recovery after RGT_ERR_TIMEOUT or an
 * interrupted call, and first-time initialisation). */
rgt_status rgt_reset_workspace(void* ws, size_t ws_bytes, hipStream_t stream);

/* Synchronise `stream`, then read the workspace's error word: RGT_OK or
 * RGT_ERR_TIMEOUT (a device-side wait expired; outputs of that call are
 * undefined and the workspace must be reset before reuse). */
rgt_status rgt_check_workspace(const void* ws, size_t ws_bytes, hipStream_t stream);

/* Router logits (split-K GEMV; split-K GEMV split-K fixup page, opening
 * summary). logits[m][n] = fp32 sum over i < K of x[m][i]*W[n][i], accumulated
 * in fp32 in a fixed order (deterministic: equal inputs give equal bits).
 *   x      : bf16 [M][ldx], device          w      : bf16 [N][ldw], device
 *   logits : fp32 [M][N] row-major, device, written
 * One launch for M <= 64 (the split-K partials are reduced in order by the
 * last workgroup to arrive at each output tile, which then zeroes its
 * counter). Larger M uses an LDS-tiled MFMA GEMM: one launch when its
 * 128 x 128 tiles fill the chip, else two (the GEMM writes k-slice partials
 * to the workspace and a second launch sums them in slice order, the order
 * the launch chain of rgt_route_sort_quant uses, so the bits agree). */
rgt_status rgt_router_logits(const void* x, int64_t ldx, const void* w, int64_t ldw,
                             float* logits, int m, int n, int k,
                             void* ws, size_t ws_bytes, hipStream_t stream);

/* Softmax top-k gate. For each row: s = fp32(logits + bias) (bias may be
 * NULL); ids = the topk experts by (s descending, expert index ascending,
 * -0 == +0), slot 0 the largest; w_j = exp(s_j - s_0) / sum_i exp(s_i - s_0)
 * over the selected slots, evaluated in fp64 by a fixed operation sequence
 * and rounded once to fp32.
 *   logits   : fp32 [M][N], device       bias : fp32 [N], device, or NULL
 *   topk_ids : int32 [M][topk], written  topk_w : fp32 [M][topk], written */
rgt_status rgt_topk_gate(const float* logits, const float* bias, int m, int n, int topk,
                         int32_t* topk_ids, float* topk_w, hipStream_t stream);

/* Softmax top-k gate fed the router's split-K partials (MiniMax-M3.1-Flash
 * MoE/GEMM kernels page, Summary: Router: the gate can take the partials; the
 * sum is the split-K reduction of the split-K GEMV page, opening summary).
 * For each row: logits = ((p_0 + p_1) + p_2) + ... + p_{S-1} in fp32, one IEEE
 * add per k-slice in ascending slice order; then exactly rgt_topk_gate.
 *   part     : fp32 [S][M][N], device (slice s at part + s*M*N)
 *   logits   : fp32 [M][N], device, written if not NULL
 *   bias, topk_ids, topk_w : as rgt_topk_gate
 * One launch. S in [1, 1024]; otherwise as rgt_topk_gate. */
rgt_status rgt_topk_gate_partials(const float* part, int s, const float* bias, int m, int n, int topk,
                                  float* logits, int32_t* topk_ids, float* topk_w, hipStream_t stream);

/* Number of k-slices S of the router partials rgt_router_shared_swiglu
 * writes for this shape (each slice K/S consecutive elements), or 0 for a
 * shape it does not cover (M outside 1..16, K above 8192, or outside the
 * router's shapes). Size part as S*M*N floats. */
int rgt_router_partial_slices(int m, int n, int k);

/* Router split-K partials and the shared expert's gate/up SwiGLU in one
 * launch (MiniMax-M3.1-Flash MoE/GEMM kernels page, Summary: Router: the
 * router's split-K partials, summed in order by the gate, fused with the
 * shared expert's fp8 SwiGLU; Summary: GEMM: the 1536 x 6144 gate_up;
 * MXFP8 shared-expert weights: monokernel page, MXFP8 shared-expert commit).
 *   x         : bf16 [M][ldx], device (read by both parts)
 *   w         : bf16 [N][ldw], device (router weights)
 *   part      : fp32 [S][M][N], device, 16-byte aligned, written:
 *               part[s][m][n] = fp32 sum over k in [s*K/S, (s+1)*K/S) of
 *               x[m][k]*W[n][k]; S must equal rgt_router_partial_slices(M, N,
 *               K). Feed it to rgt_topk_gate_partials.
 *   wsh_q     : uint8 [2I][K] e4m3fn codes, device, 16-byte aligned, rows
 *               K bytes apart: rows 0..I-1 the gate projection, I..2I-1 up.
 *   wsh_scale : uint8 [2I][K/32] e8m0 scale bytes (element (r, i) is
 *               e4m3(code) * 2^(scale[r][i/32] - 127)), device.
 *   h         : bf16 [M][ldh], device, written for columns < I:
 *               h[m][j] = bf16_rne( silu(g) * u ), g = x[m].Wg[j],
 *               u = x[m].Wu[j], silu(g) = g / (1 + exp(-g)), fp32 sums.
 * 0 <= M <= 16, K <= 8192 and the router's shape rules (N a multiple of 16
 * in [16, 1024], K a multiple of 512), 1 <= I <= 2^20, ldh >= I; otherwise
 * RGT_ERR_UNSUPPORTED or RGT_ERR_INVALID and nothing is launched.
 * Covered weight scales: scale bytes 10..246. There every scaled weight is
 * zero or a normal fp32 and bf16 value (at least 2^-126, below 2^128), and
 * the two forms of the kernel (up to 8 rows: codes times x in fp32, then the
 * scale; 9 to 16 rows: the scale folded into bf16 weights) are exact in the
 * weights and agree within the summation bound. Bytes 0..9 and 247..254 are
 * accepted but their results are unspecified, as are results whose g, u or h
 * leave the fp32 / bf16 range. NaN codes or a 255 scale give NaN outputs.
 * One launch, no workspace. */
rgt_status rgt_router_shared_swiglu(const void* x, int64_t ldx, const void* w, int64_t ldw, int m, int n, int k,
                                    float* part, int s, const uint8_t* wsh_q, const uint8_t* wsh_scale, int inter,
                                    void* h, int64_t ldh, hipStream_t stream);

/* Sort (token, slot) pairs into block-padded expert segments and quantise
 * the gathered activations to MXFP8. Pair p = m*topk + j has expert
 * topk_ids[m][j] (each in [0, N)).
 *   sorted_ids : int32 [cap]; segment e occupies [offsets[e], offsets[e+1]);
 *                its first cnt[e] entries are the pair ids on expert e in
 *                ascending order, the rest the sentinel P = M*topk.
 *   expert_ids : int32 [cap/block]; expert of each block of sorted_ids.
 *   offsets    : int32 [N+1]; offsets[N] is the padded total. Entries of
 *                sorted_ids / expert_ids / a_q / a_scale at or past the total
 *                are not written.
 *   a_q        : uint8 [cap][K]; row p (for a non-sentinel entry) holds the
 *                e4m3fn codes of x[sorted_ids[p] / topk]; pad rows are not
 *                written.
 *   a_scale    : uint8 [cap][K/32]; e8m0 scale byte of each 32-element block:
 *                se + 127 with se = clamp(floor(log2 amax) - 8, -127, 127),
 *                0 for an all-zero block. Codes are e4m3(v / 2^se), round to
 *                nearest even, saturating at +-448, sign kept. */
rgt_status rgt_moe_sort_quant(const int32_t* topk_ids, const void* x, int64_t ldx,
                              int m, int n, int k, int topk, int block,
                              int32_t* sorted_ids, int32_t* expert_ids, int32_t* offsets,
                              uint8_t* a_q, uint8_t* a_scale,
                              void* ws, size_t ws_bytes, hipStream_t stream);

/* The whole front end: router logits -> top-k gate -> sort -> MXFP8 quant.
 * Outputs are bit-identical to rgt_router_logits, rgt_topk_gate and
 * rgt_moe_sort_quant chained on the same inputs. `logits` may be NULL (then
 * the logits stay in the workspace). For M <= 64 this is ONE kernel launch
 * whose workgroups wait for one another on device counters; the grid is
 * sized to be co-resident, and every wait is bounded by a deadline (expiry
 * sets the workspace error word, see rgt_check_workspace). */
rgt_status rgt_route_sort_quant(const void* x, int64_t ldx, const void* w, int64_t ldw,
                                const float* bias, int m, int n, int k, int topk, int block,
                                float* logits, int32_t* topk_ids, float* topk_w,
                                int32_t* sorted_ids, int32_t* expert_ids, int32_t* offsets,
                                uint8_t* a_q, uint8_t* a_scale,
                                void* ws, size_t ws_bytes, hipStream_t stream);

/* rgt_route_sort_quant without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). The workspace is an 8 MiB array inside
 * the library, one per GPU, held until the process ends; the call allocates
 * nothing and frees nothing. Arguments, outputs, launch counts and errors are
 * those of rgt_route_sort_quant, plus: a shape whose workspace
 * (rgt_workspace_bytes at M = m) exceeds 8 MiB returns RGT_ERR_UNSUPPORTED
 * and launches nothing (every shape with M <= 64 fits: 2.2 MiB at N = 128,
 * K = 6144, top-8; 5.9 MiB at N = 896, K = 3584, top-16; 7.3 MiB at
 * N = 1024, K = 8192, top-32). The first call on a GPU also zero-fills the
 * array with one kernel on `stream` (counted in rgt_last_launch_count).
 * Every call on a GPU shares that GPU's array: calls that overlap in time on
 * one GPU (two streams, two threads) race and give undefined results; run
 * them in one stream. A device-side deadline expiry poisons the array: every
 * later call on that GPU writes the poison outputs (top-k ids -1, weights 0,
 * offsets 0) for the rest of the process. */
rgt_status rgt_route_sort_quant_noalloc(const void* x, int64_t ldx, const void* w, int64_t ldw,
                                        const float* bias, int m, int n, int k, int topk, int block,
                                        float* logits, int32_t* topk_ids, float* topk_w,
                                        int32_t* sorted_ids, int32_t* expert_ids, int32_t* offsets,
                                        uint8_t* a_q, uint8_t* a_scale, hipStream_t stream);

/* MXFP4 variants (the stage-1 activation quant of the MoE sort; MiniMax-M3.1-
 * Flash MoE/GEMM kernels page, Summary: MoE sorting + quant, and "Changes to
 * existing kernels": 128-expert top-4 routing at hidden 6144 sorted in one
 * launch with the stage-1 MXFP4 activation quant). Arguments, sort outputs,
 * coverage, errors and launch counts are those of rgt_moe_sort_quant and
 * rgt_route_sort_quant; only the element format and the a_q layout differ:
 *   a_q     : uint8 [cap][K/2]; byte j of row p holds the e2m1 codes of
 *             elements 2j (low nibble) and 2j+1 (high nibble) of
 *             x[sorted_ids[p] / topk]; pad rows are not written.
 *   a_scale : uint8 [cap][K/32]; se + 127 with se = clamp(floor(log2 amax) - 2,
 *             -127, 127) (OCP MX v1.0, e2m1 emax 2), 0 for an all-zero block.
 *             Codes are e2m1(v / 2^se): values 0, 0.5, 1, 1.5, 2, 3, 4, 6, round
 *             to nearest even, saturating at +-6, sign in bit 3 (-0 -> 0x8). */
rgt_status rgt_moe_sort_quant_mxfp4(const int32_t* topk_ids, const void* x, int64_t ldx,
                                    int m, int n, int k, int topk, int block,
                                    int32_t* sorted_ids, int32_t* expert_ids, int32_t* offsets,
                                    uint8_t* a_q, uint8_t* a_scale,
                                    void* ws, size_t ws_bytes, hipStream_t stream);
rgt_status rgt_route_sort_quant_mxfp4(const void* x, int64_t ldx, const void* w, int64_t ldw,
                                      const float* bias, int m, int n, int k, int topk, int block,
                                      float* logits, int32_t* topk_ids, float* topk_w,
                                      int32_t* sorted_ids, int32_t* expert_ids, int32_t* offsets,
                                      uint8_t* a_q, uint8_t* a_scale,
                                      void* ws, size_t ws_bytes, hipStream_t stream);

/* Stage-1 GEMM of the routed experts on the sorted segments (the A8W4 fused
 * MoE that runs on the sort's outputs: "Kimi-K3: fused MoE routing, sort,
 * quant and epilogue", Modifications; the stage-1 activations of the
 * MiniMax-M3.1-Flash MoE/GEMM kernels page, Summary: MoE sorting + quant).
 * Reads the outputs of rgt_moe_sort_quant / rgt_route_sort_quant (MXFP8) in
 * place. For every padded row p < offsets[N] whose sorted_ids entry is a
 * pair (not the sentinel M*topk), with e = expert_ids[p / block]:
 *   g = a . W_e[j], u = a . W_e[I + j]  (a: the row's MXFP8 values; W_e:
 *       expert e's gate_up weights, fp32 sums in the MFMA's own order),
 *   h[p][j] = bf16_rne( silu(g) * u ), silu(g) = g / (1 + exp(-g)), j < I.
 *   a_q, a_scale, sorted_ids, expert_ids, offsets : as rgt_moe_sort_quant
 *                 wrote them (M, N, K, topk, block: that call's arguments)
 *   w_q     : uint8 [N][2I][K/2] e2m1 codes, byte i of a row holding
 *             elements 2i (low nibble) and 2i+1 (high nibble); rows 0..I-1 of
 *             an expert the gate projection, I..2I-1 up; 16-byte aligned
 *   w_scale : uint8 [N][2I][K/32] e8m0 scales (element (r, i) of expert e is
 *             e2m1(code) * 2^(w_scale[e][r][i/32] - 127))
 *   h       : bf16 [cap][ldh], device, written for the pair rows and j < I;
 *             pad rows and rows at or past offsets[N] are not written
 * Coverage: the sort's shapes (K % 512 == 0, N <= 1024, topk <= 32, block in
 * {16, 32, 64}, M <= 8192) and 16 <= I <= 65536, I % 16 == 0; otherwise
 * RGT_ERR_UNSUPPORTED. One launch, no workspace. Scale bytes 255 or NaN
 * activation codes give NaN outputs; results whose g, u or h leave the fp32 /
 * bf16 range are unspecified. */
rgt_status rgt_moe_stage1_swiglu(const uint8_t* a_q, const uint8_t* a_scale, const int32_t* sorted_ids,
                                 const int32_t* expert_ids, const int32_t* offsets, int m, int n, int k,
                                 int topk, int block, const uint8_t* w_q, const uint8_t* w_scale, int inter,
                                 void* h, int64_t ldh, hipStream_t stream);

/* RMSNorm producer in front of the router (the Gemma RMSNorm (+ residual)
 * producers of the MiniMax-M3.1-Flash MoE/GEMM kernels page, Summary: fp8
 * producers; the per-token rstd it publishes is the scale the "route on the
 * norm's scale" commit of the MiniMax-M3.1 FFN monokernel page routes on).
 * For each row m:
 *   h    = bf16(fp32(x) + fp32(residual)) with one fp32 add and round to
 *          nearest even, or h = x when residual is NULL
 *   rstd = 1 / sqrt(sum_i h_i^2 / K + eps), fp32 (the sum in this library's
 *          order: compared with a reference within its rounding, not bit for bit)
 *   xn_i = bf16(fp32(fp32(h_i * rstd) * fp32(1 + gamma_i)))   (Gemma weights)
 *   x, residual : bf16 [M][ld], device, 16-byte aligned, ld >= K, ld % 8 == 0
 *   gamma       : bf16 [K], device, 16-byte aligned
 *   xn          : bf16 [M][ldxn], written (the router's input)
 *   residual_out: bf16 [M][ldro], written with h if not NULL (needs residual)
 *   rstd        : fp32 [M], written if not NULL
 * Coverage: 8 <= K <= 16384, K % 8 == 0, M <= 65535. One launch. The sum of
 * squares is accumulated in fp32: rows whose sum of squares overflows fp32
 * (|h| beyond ~1e17) are outside the contract. */
rgt_status rgt_rmsnorm(const void* x, int64_t ldx, const void* residual, int64_t ldr, const void* gamma, float eps,
                       int m, int k, void* xn, int64_t ldxn, void* residual_out, int64_t ldro, float* rstd,
                       hipStream_t stream);

/* The front end behind its RMSNorm producer: rgt_rmsnorm, then
 * rgt_route_sort_quant (or _mxfp4) on its xn, with every output bit-identical
 * to that two-call chain on the same inputs (xn, residual_out and rstd as
 * rgt_rmsnorm writes them; logits, gate, sort and quant as the route call
 * writes them from xn). The router routes on the norm's scale ("route on the
 * norm's scale", MiniMax-M3.1 FFN monokernel page, Modifications): in the
 * one-launch form (M <= 64, K <= 8192) workgroup m takes row m's rstd and
 * publishes it (with M = 1 every workgroup takes it itself), and every
 * router tile normalises its own columns of x (and the residual) with that
 * rstd instead of reading a written xn. Otherwise the norm's own launch comes
 * first and the route call reads its xn (rgt_last_launch_count tells which).
 * The one-launch form is taken at M = 1, where it is faster; the environment
 * variable RGT_NORM_IN_LAUNCH=1 takes it for every M it covers, =0 never.
 * Arguments: those of rgt_rmsnorm (x, residual, gamma, eps, xn,
 * residual_out, rstd; xn is required and must not overlap x or residual)
 * and of rgt_route_sort_quant (w, bias, sizes, outputs, workspace: the same
 * rgt_workspace_bytes); `x` is the raw input, not the router's. Coverage and
 * errors: the union of both calls' rules. The one-launch form waits on
 * device words like rgt_route_sort_quant; after an expired wait the route
 * outputs are the poison values and xn, residual_out and rstd are
 * unspecified. */
rgt_status rgt_rmsnorm_route_sort_quant(const void* x, int64_t ldx, const void* residual, int64_t ldr,
                                        const void* gamma, float eps, const void* w, int64_t ldw, const float* bias,
                                        int m, int n, int k, int topk, int block, void* xn, int64_t ldxn,
                                        void* residual_out, int64_t ldro, float* rstd, float* logits,
                                        int32_t* topk_ids, float* topk_w, int32_t* sorted_ids, int32_t* expert_ids,
                                        int32_t* offsets, uint8_t* a_q, uint8_t* a_scale, void* ws, size_t ws_bytes,
                                        hipStream_t stream);
rgt_status rgt_rmsnorm_route_sort_quant_mxfp4(const void* x, int64_t ldx, const void* residual, int64_t ldr,
                                              const void* gamma, float eps, const void* w, int64_t ldw,
                                              const float* bias, int m, int n, int k, int topk, int block, void* xn,
                                              int64_t ldxn, void* residual_out, int64_t ldro, float* rstd,
                                              float* logits, int32_t* topk_ids, float* topk_w, int32_t* sorted_ids,
                                              int32_t* expert_ids, int32_t* offsets, uint8_t* a_q, uint8_t* a_scale,
                                              void* ws, size_t ws_bytes, hipStream_t stream);

/* Settings are read from the environment at the first call of the process
 * and again by this call, never on the call path (so a call costs no
 * getenv); call it after changing them, with no call of the library in
 * flight on any thread:
 *   RGT_WAIT_BUDGET_US  deadline of each device-side wait, in us (100000)
 *   RGT_NO_FUSE=1       never the one-launch form of the route calls
 *   RGT_NORM_IN_LAUNCH  1: the norm joins the route's launch whenever it
 *                       fits, 0: never (default: at M = 1)
 *   RGT_FORCE_BUCKET    comma-separated, for experiments and tests: valu or
 *                       mfma (the router tile; valu only up to M = 8), small
 *                       or large (the one-launch form's mode); a workspace
 *                       must be sized under the same setting
 *   RGT_LOG=1           one line on stderr per new shape with the plan taken
 *   RGT_FAULT_INJECT=1  host-forced fault for tests: no tagged word is
 *                       published, so every device-side wait runs into its
 *                       deadline
 * Settings apply to every device. */
void rgt_reload_env(void);

/* Number of kernel launches the last successful call of each entry point made
 * on this thread (diagnostics for launch-count checks). */
int rgt_last_launch_count(void);

/* Measurement helpers (not part of the routing path).
 * rgt_diag_read: one launch of `grid` workgroups that streams `bytes` (a
 *   multiple of 16) from device memory `src` with 16-byte loads; `sink` is a
 *   device uint32 array of `grid` words that receives one word per workgroup.
 *   It is the floor of any kernel that must read the same bytes.
 * rgt_diag_copy: one launch copying `bytes` (a multiple of 16) from `src` to
 *   `dst` (device, 16-byte aligned, not overlapping): a kernel of known
 *   traffic for calibrating hardware byte counters. */
rgt_status rgt_diag_read(const void* src, size_t bytes, uint32_t* sink, int grid, hipStream_t stream);
rgt_status rgt_diag_copy(const void* src, void* dst, size_t bytes, int grid, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* RGT_H */
