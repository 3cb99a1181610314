"""CPU oracle for the MoE routing front-end (test infrastructure only).

This module is test infrastructure. Only the tests, the smoke check and the
CPU-baseline leg of the benchmark may import it. The product path (the HIP
library and its Python binding) never calls it, and it shares no code with
that path: no kernels, helpers, tables or constant generators. Both sides are
fed from the seeded generators in ``router_gemv_top_amd.inputs``, which hold
none of the method's arithmetic.

It is deliberately plain and slow: fp64 arithmetic, library primitives
(matmul, argmax, stable argsort) used as whole steps, no blocking or fusion.

Sources (titles of the pages this follows):
  [GEMV]  "MiniMax-M3: Triton split-K router GEMV with in-kernel split-K fixup"
          (sglang PR #36557), opening summary: logits[M,N] fp32 =
          x[M,K] bf16 . W[N,K]^T bf16.
  [M31K]  MiniMax-M3.1-Flash MoE/GEMM kernels (sglang PR #46691), Summary
          (router, MoE sorting + quant) and "Changes to existing kernels"
          (fp64 accuracy and determinism test of the router).
  [K3]    "Kimi-K3: fused MoE routing, sort, quant and epilogue"
          (sglang PR #46652), Modifications and the review snippet on the
          stable rank (a pair's rank counts earlier tokens on the same expert).
  [MONO]  "minimax_m31: Run MiniMax-M3.1-Flash's decode FFN as one monokernel
          launch a layer" (sgl-amd-mono PR #56), the MXFP8 shared-expert
          commit (group-32 scales).
  [M3R]   sglang PR #46691 (MiniMax-M3.1-Flash MoE/GEMM kernels), Summary:
          fp8 producers (the Gemma RMSNorm (+ residual) producers in front of
          the next GEMM) and the measured gain of those producers.
  [FUSE]  sglang PR #46691 (MiniMax-M3.1-Flash MoE/GEMM kernels), Summary:
          Router (the split-K partials exposed and fused with the shared
          expert's fp8 SwiGLU in one launch) and GEMM (the M3.1 shared
          expert's 1536 x 6144 gate_up); [MONO] MXFP8 shared-expert commit
          (fp8 values with one scale per 32 elements along K).
  [K3S1]  "Kimi-K3: fused MoE routing, sort, quant and epilogue" (sglang PR
          #46652), Modifications: the sorted, quantised activations feed the
          routed experts' stage-1 GEMM of AITER's fused MoE, A8W4 (8-bit
          activations, 4-bit weights); MiniMax-M3.1-Flash MoE/GEMM kernels
          (sglang PR #46691), Summary: MoE sorting + quant (the stage-1
          activations).
  [OCP]   OCP Microscaling Formats (MX) v1.0: e4m3 element format (bias 7,
          max normal 448, no infinities), e8m0 shared scale (bias 127), shared
          exponent = floor(log2(amax)) - emax_elem with emax_elem = 8 for e4m3;
          e2m1 element format (1 sign bit, 2 exponent bits with bias 1, 1
          mantissa bit: 0, 0.5, 1, 1.5, 2, 3, 4, 6; no infinities or NaN) with
          emax_elem = 2.

Readings taken where the pages are silent (each is listed in the design
notes):
  * Gate scores: s = fp32(L + bias) when a bias is given, else s = L.
  * Top-k order: score descending, expert index ascending on ties; -0 == +0.
  * Weights: w_j = exp(s_j - s_0) / sum_{i<k} exp(s_i - s_0), i.e. full
    softmax then renormalisation over the selected k, evaluated by one written
    fp64 recipe (``exp64`` below) so that a second implementation can match it
    bit for bit.
  * Sort: pair id p = m*k + j; segments by ascending expert, pairs inside a
    segment in ascending p, each segment padded up to a multiple of the block
    size with the sentinel P = M*k; empty experts get no block.
  * MXFP8: OCP floor rule for the shared exponent, round to nearest even,
    saturation to +-448, sign kept (so -0 encodes as 0x80).
  * RMSNorm producer ([M3R]; [MONO] "route on the norm's scale": the norm
    publishes each token's rstd): h = bf16(x + residual) with one fp32 add,
    rstd = 1/sqrt(mean(h^2) + eps), xn = bf16((h * rstd) * (1 + gamma)) with
    fp32 steps (Gemma weights). rstd is compared within its rounding; xn is
    exact given the rstd used.
  * MXFP4 (the stage-1 activation quant of [M31K], Summary: MoE sorting +
    quant): the same floor rule with emax_elem = 2 for e2m1, round to nearest
    even, saturation to +-6, sign kept (-0 -> 0x8); two codes a byte, the
    even element in the low nibble.

  * Shared expert ([FUSE]): gate_up is [2I][K] MXFP8, the I gate rows first,
    then the I up rows; element (r, i) = e4m3(code) * 2^(scale[r][i/32] - 127).
    g = x . Wg^T, u = x . Wu^T (exact products, fp64 sums); SwiGLU
    h = silu(g) * u with silu(g) = g / (1 + exp(-g)), no clamp; the kernel
    rounds h once to bf16.
  * Router partials: k-slice s covers K/S consecutive elements
    [s*K/S, (s+1)*K/S); part[s] = fp32(sum over the slice), summed in fp64.
  * Stage-1 grouped MoE GEMM ([K3S1]): every valid padded row p (a real
    pair) of the sort, with expert e = expert_ids[p // B], takes its MXFP8 row
    a = dequant(a_q[p], a_scale[p]) against expert e's MXFP4 gate_up weights
    W_e [2I][K] (e2m1 codes two a byte, low nibble first, e8m0 scale per 32
    along K; the I gate rows first): g = a . W_e[:I], u = a . W_e[I:] (exact
    products, fp64 sums), h = silu(g) * u (the shared expert's SwiGLU
    reading). Pad rows have no output.

Parity pins: every function here is checked by the ``-m "not gpu"`` tests
against brute force, exact rationals, closed forms or invariants.
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# bf16 helpers
# ---------------------------------------------------------------------------


def bf16_bits_to_f64(h: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns as fp64."""
    u = np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# Router logits [GEMV]
# ---------------------------------------------------------------------------


def router_logits(x_bits: np.ndarray, w_bits: np.ndarray) -> np.ndarray:
    """logits[m][n] = fp32( sum_i x[m][i] * W[n][i] ), summed in fp64.

    [GEMV] opening summary: the router gate is [M,K] bf16 x [N,K] bf16 ->
    [M,N] fp32. Products of two bf16 values are exact in fp64; the fp64 sum
    (a library matmul) is then rounded once, to nearest even, to fp32. The
    fp64 accumulation error is far below one fp32 ulp of any logit that
    matters for the tolerance used against the GPU. [M31K] names an fp64
    accuracy test for the router; this is that reference.
    """
    x = bf16_bits_to_f64(x_bits)
    w = bf16_bits_to_f64(w_bits)
    assert np.all(np.isfinite(x)) and np.all(np.isfinite(w))
    return (x @ w.T).astype(np.float32)


# ---------------------------------------------------------------------------
# Softmax top-k gate (reading: softmax, top-k, renormalise)
# ---------------------------------------------------------------------------


def gate_scores(logits: np.ndarray, bias: np.ndarray | None) -> np.ndarray:
    """s = fp32(L + bias) (one IEEE fp32 add per element) or s = L."""
    s = np.asarray(logits, dtype=np.float32)
    if bias is not None:
        s = (s + np.asarray(bias, dtype=np.float32)[None, :]).astype(np.float32)
    assert np.all(np.isfinite(s)), "scores must be finite"
    return s


def topk_ids(scores: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest scores per row, largest first.

    Order key: score descending, then expert index ascending; -0 and +0 are
    equal (IEEE compare). Selection by k rounds of "first index of the
    maximum" over the experts not yet chosen.
    """
    s = np.asarray(scores, dtype=np.float32)
    s = np.where(s == 0, np.float32(0), s)  # -0 -> +0, so they tie
    m, n = s.shape
    assert 1 <= k <= n
    taken = np.zeros((m, n), dtype=bool)
    out = np.empty((m, k), dtype=np.int32)
    rows = np.arange(m)
    for j in range(k):
        masked = np.where(taken, -np.inf, s.astype(np.float64))
        idx = np.argmax(masked, axis=1)  # first occurrence -> lowest index on ties
        out[:, j] = idx
        taken[rows, idx] = True
    return out


# exp64 recipe constants. Each is the fp64 number nearest to the stated
# mathematical value, except LN2_HI, which is ln 2 cut to 24 significant bits
# so that n * LN2_HI is exact for |n| < 2**29 (Cody & Waite range reduction).
LOG2E = float.fromhex("0x1.71547652b82fep+0")      # 1/ln 2
LN2_HI = float.fromhex("0x1.62e42e0000000p-1")     # ln 2, 24 bits
LN2_LO = float.fromhex("0x1.efa39ef35793cp-25")    # ln 2 - LN2_HI
INV_FACT = [float.fromhex(h) for h in (             # 1/j!, j = 0..13
    "0x1.0000000000000p+0", "0x1.0000000000000p+0", "0x1.0000000000000p-1",
    "0x1.5555555555555p-3", "0x1.5555555555555p-5", "0x1.1111111111111p-7",
    "0x1.6c16c16c16c17p-10", "0x1.a01a01a01a01ap-13", "0x1.a01a01a01a01ap-16",
    "0x1.71de3a556c734p-19", "0x1.27e4fb7789f5cp-22", "0x1.ae64567f544e4p-26",
    "0x1.1eed8eff8d898p-29", "0x1.6124613a86d09p-33")]
EXP64_CUTOFF = -200.0  # exp(d) for d < -200 is returned as 0 (w rounds to 0 in fp32 anyway)


def exp64(d: np.ndarray) -> np.ndarray:
    """exp(d) for d <= 0 in fp64 by a fixed sequence of IEEE operations.

    1. n = rint(d * LOG2E)                    (round half to even)
    2. r = (d - n * LN2_HI) - n * LN2_LO      (Cody-Waite reduction, |r| <= ln2/2)
    3. p = sum_{j=0}^{13} r^j / j!            (Horner; each step one multiply,
                                               then one add, no fused multiply-add)
    4. e = p * 2^n                            (exact scaling)
    d < -200 gives 0. Truncation error of the degree-13 polynomial is below
    2^-57 relative on |r| <= ln2/2; the whole recipe is within a few fp64 ulp
    of exp(d).
    """
    d = np.asarray(d, dtype=np.float64)
    n = np.rint(d * LOG2E)
    r = (d - n * LN2_HI) - n * LN2_LO
    p = np.full_like(d, INV_FACT[13])
    for j in range(12, -1, -1):
        p = p * r
        p = p + INV_FACT[j]
    n_int = np.where(d < EXP64_CUTOFF, 0, n).astype(np.int64)
    e = np.ldexp(p, n_int)
    return np.where(d < EXP64_CUTOFF, 0.0, e)


def topk_weights(sel_scores: np.ndarray) -> np.ndarray:
    """Renormalised softmax weights of the selected scores (slot 0 = largest).

    w_j = exp(s_j - s_0) / sum_{i<k} exp(s_i - s_0). Equal to taking the full
    softmax over all N experts and dividing the k selected probabilities by
    their sum, since the common factor cancels. fp64 throughout: the
    differences, exp64, the sum in slot order, the division; one RNE rounding
    to fp32 at the end.
    """
    s = np.asarray(sel_scores, dtype=np.float32).astype(np.float64)
    d = s - s[:, :1]
    e = exp64(d)
    total = e[:, 0].copy()
    for j in range(1, e.shape[1]):
        total = total + e[:, j]
    return (e / total[:, None]).astype(np.float32)


def topk_gate(logits: np.ndarray, bias: np.ndarray | None, k: int):
    """(ids int32 [M][k], w fp32 [M][k]) of the softmax top-k gate."""
    s = gate_scores(logits, bias)
    ids = topk_ids(s, k)
    sel = np.take_along_axis(s, ids.astype(np.int64), axis=1)
    return ids, topk_weights(sel)


def sum_partials(part: np.ndarray) -> np.ndarray:
    """logits [M][N] fp32 from split-K partials part [S][M][N] fp32, added in
    k-slice order: ((p_0 + p_1) + p_2) + ... , each add one IEEE fp32 add.

    [GEMV] opening summary: the split-K reduction sums the partials of every
    k-slice; [M31K] Summary: Router, the gate can take the partials and sum
    them itself. The slice order is the fixed, deterministic reduction order
    (our reading: ascending slice index, as the last arriver sums them).
    """
    p = np.asarray(part, dtype=np.float32)
    assert p.ndim == 3 and np.all(np.isfinite(p))
    acc = p[0].copy()
    for s in range(1, p.shape[0]):
        acc = (acc + p[s]).astype(np.float32)   # float32 + float32: one rounding per add
    return acc


def topk_gate_partials(part: np.ndarray, bias: np.ndarray | None, k: int):
    """(logits, ids, w) of the softmax top-k gate fed the split-K partials:
    the logits are sum_partials(part), then the gate as topk_gate."""
    logits = sum_partials(part)
    ids, w = topk_gate(logits, bias, k)
    return logits, ids, w


# ---------------------------------------------------------------------------
# RMSNorm producer in front of the router [M3R], [MONO]
# ---------------------------------------------------------------------------


def bf16_round(v: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of finite fp32 values, rounded to nearest, ties to
    even: 8 significant bits (spacing 2^-133 below the normal range), from the
    exact fp64 value."""
    a = np.asarray(v, dtype=np.float32).astype(np.float64)
    _, ex = np.frexp(a)                        # |a| = f * 2^ex, f in [0.5, 1)
    qexp = np.maximum(ex - 8, -133)            # spacing of bf16 values near a
    q = np.rint(np.ldexp(a, -qexp))            # RNE to a multiple of the spacing
    r = np.ldexp(q, qexp).astype(np.float32)   # exact: a bf16 value
    return (r.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def residual_add(x_bits: np.ndarray, r_bits: np.ndarray) -> np.ndarray:
    """h = bf16(fp32(x) + fp32(r)): one fp32 add, then rounded to bf16 (the
    producer's residual stream)."""
    x = bf16_bits_to_f64(x_bits).astype(np.float32)
    r = bf16_bits_to_f64(r_bits).astype(np.float32)
    return bf16_round((x + r).astype(np.float32))


def rmsnorm_rstd(h_bits: np.ndarray, eps: float) -> np.ndarray:
    """rstd[m] = 1 / sqrt(mean_i h[m][i]^2 + eps), in fp64, rounded once to
    fp32 (the per-token scale the norm publishes)."""
    h = bf16_bits_to_f64(h_bits)
    ms = (h * h).sum(axis=1) / h.shape[1]
    return (1.0 / np.sqrt(ms + float(np.float32(eps)))).astype(np.float32)


def rmsnorm_apply(h_bits: np.ndarray, rstd: np.ndarray, gamma_bits: np.ndarray) -> np.ndarray:
    """xn = bf16( fp32( fp32(h * rstd) * fp32(1 + gamma) ) ): the Gemma form
    (weight 1 + gamma), each step one IEEE fp32 operation, then rounded to
    bf16. rstd is fp32 [M]; the result is bf16 bits [M][K]."""
    h = bf16_bits_to_f64(h_bits).astype(np.float32)
    g = (np.float32(1.0) + bf16_bits_to_f64(gamma_bits).astype(np.float32)).astype(np.float32)
    t = (h * np.asarray(rstd, np.float32)[:, None]).astype(np.float32)
    return bf16_round((t * g[None, :]).astype(np.float32))


def rmsnorm(x_bits, r_bits, gamma_bits, eps: float):
    """(xn bits, rstd fp32, h bits): h = residual_add(x, r) (or x without a
    residual), rstd = rmsnorm_rstd(h), xn = rmsnorm_apply(h, rstd, gamma)."""
    h = x_bits if r_bits is None else residual_add(x_bits, r_bits)
    rstd = rmsnorm_rstd(h, eps)
    return rmsnorm_apply(h, rstd, gamma_bits), rstd, h


# ---------------------------------------------------------------------------
# Token -> expert sort [M31K, K3]
# ---------------------------------------------------------------------------


def sort_capacity(m: int, n: int, k: int, block: int) -> int:
    """Upper bound on the padded total: P + min(N, P)*(B-1), rounded up to B."""
    p = m * k
    cap = p + min(n, p) * (block - 1)
    return (cap + block - 1) // block * block


def moe_sort(ids: np.ndarray, n: int, block: int):
    """Counting sort of (token, slot) pairs into block-padded expert segments.

    Returns (sorted_ids int32 [total], expert_ids int32 [total/B],
    offsets int32 [N+1], total). Pair p = m*k + j goes to expert ids[m][j].
    Segment e starts at offsets[e] and holds cnt[e] pair ids in ascending p
    (the stable rank of [K3]: earlier tokens on the same expert come first),
    then the sentinel P = M*k up to the next multiple of B.
    """
    ids = np.asarray(ids, dtype=np.int64)
    m, k = ids.shape
    p_total = m * k
    e_of_pair = ids.reshape(-1)
    assert np.all((e_of_pair >= 0) & (e_of_pair < n))
    cnt = np.bincount(e_of_pair, minlength=n)
    padded = (cnt + block - 1) // block * block
    offsets = np.zeros(n + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(padded)
    total = int(offsets[n])
    sorted_ids = np.full(total, p_total, dtype=np.int32)
    order = np.argsort(e_of_pair, kind="stable")  # by expert, ascending p inside
    start = 0
    for e in range(n):
        c = int(cnt[e])
        sorted_ids[offsets[e]:offsets[e] + c] = order[start:start + c]
        start += c
    expert_ids = np.repeat(np.arange(n, dtype=np.int32), padded // block)
    return sorted_ids, expert_ids, offsets.astype(np.int32), total


# ---------------------------------------------------------------------------
# MXFP8 quantisation [OCP], [MONO] group-32 scales
# ---------------------------------------------------------------------------

E4M3_MAX = 448.0
E4M3_EMAX = 8          # floor(log2(448))
MX_BLOCK = 32


def e4m3_code(y: np.ndarray, neg: np.ndarray) -> np.ndarray:
    """e4m3fn code of |y| (fp64, >= 0, exact) with the given sign.

    Round to nearest, ties to even, over normals (3 mantissa bits, exponent
    >= -6) and subnormals (step 2^-9); magnitudes above 448 saturate to 448.
    """
    a = np.asarray(y, dtype=np.float64)
    _, ex = np.frexp(a)                        # a = f * 2^ex, f in [0.5, 1)
    binade = np.maximum(ex - 1, -6)            # floor(log2 a), at least -6
    qexp = binade - 3                          # spacing of representable values
    units = np.rint(np.ldexp(a, -qexp))        # RNE to a multiple of the spacing
    val = np.ldexp(units, qexp)
    val = np.where(a > E4M3_MAX, E4M3_MAX, val)
    val = np.minimum(val, E4M3_MAX)
    # encode the (now representable) magnitude
    _, vex = np.frexp(val)
    vb = vex - 1
    is_norm = (val > 0) & (vb >= -6)
    mant_norm = np.ldexp(val, -(vb - 3)) - 8.0          # 0..7
    code_norm = ((vb + 7) << 3) + mant_norm.astype(np.int64)
    code_sub = np.ldexp(val, 9).astype(np.int64)        # 0..7 (0 for zero)
    code = np.where(is_norm, code_norm, code_sub).astype(np.int64)
    code = code | (np.asarray(neg, dtype=np.int64) << 7)
    return code.astype(np.uint8)


def mxfp8_quant_rows(x_bits: np.ndarray):
    """MXFP8 of bf16 rows: (codes u8 [R][K], scales u8 [R][K/32]).

    Per 32-element block: amax = max |v|; E = floor(log2 amax) (exact, from the
    binary exponent); shared exponent se = clamp(E - 8, -127, 127) (0 scale
    byte when amax = 0); scale byte = se + 127 (e8m0); element code =
    e4m3(v / 2^se).
    """
    h = np.asarray(x_bits, dtype=np.uint16)
    r, k = h.shape
    assert k % MX_BLOCK == 0
    v = bf16_bits_to_f64(h).reshape(r, k // MX_BLOCK, MX_BLOCK)
    neg = ((h >> np.uint16(15)) & np.uint16(1)).reshape(v.shape).astype(bool)
    av = np.abs(v)
    amax = av.max(axis=2)
    _, ex = np.frexp(amax)
    e_floor = ex - 1
    se = np.where(amax > 0, np.clip(e_floor - E4M3_EMAX, -127, 127), -127).astype(np.int64)
    scale = (se + 127).astype(np.uint8)
    y = np.ldexp(av, -se[:, :, None])          # exact: power-of-two scaling
    codes = e4m3_code(y, neg)
    return codes.reshape(r, k), scale


# ---------------------------------------------------------------------------
# MXFP4 quantisation [OCP] e2m1 elements, [M31K] stage-1 activation quant
# ---------------------------------------------------------------------------

E2M1_MAX = 6.0
E2M1_EMAX = 2          # floor(log2(6))


def e2m1_code(y: np.ndarray, neg: np.ndarray) -> np.ndarray:
    """e2m1 code (4 bits) of |y| (fp64, >= 0, exact) with the given sign.

    Round to nearest, ties to even, over normals (1 mantissa bit, exponent
    >= 0) and the subnormal 0.5 (step 2^-1); magnitudes above 6 saturate to 6.
    """
    a = np.asarray(y, dtype=np.float64)
    _, ex = np.frexp(a)                        # a = f * 2^ex, f in [0.5, 1)
    binade = np.maximum(ex - 1, 0)             # floor(log2 a), at least 0
    qexp = binade - 1                          # spacing of representable values
    units = np.rint(np.ldexp(a, -qexp))        # RNE to a multiple of the spacing
    val = np.minimum(np.ldexp(units, qexp), E2M1_MAX)
    # encode the (now representable) magnitude
    _, vex = np.frexp(val)
    vb = vex - 1
    is_norm = val >= 1.0
    mant_norm = np.ldexp(val, -(vb - 1)) - 2.0          # 0 or 1
    code_norm = ((vb + 1) << 1) + mant_norm.astype(np.int64)
    code_sub = np.ldexp(val, 1).astype(np.int64)        # 0 or 1
    code = np.where(is_norm, code_norm, code_sub).astype(np.int64)
    code = code | (np.asarray(neg, dtype=np.int64) << 3)
    return code.astype(np.uint8)


def mxfp4_quant_rows(x_bits: np.ndarray):
    """MXFP4 of bf16 rows: (packed codes u8 [R][K/2], scales u8 [R][K/32]).

    Per 32-element block: amax = max |v|; E = floor(log2 amax); shared
    exponent se = clamp(E - 2, -127, 127) (0 scale byte when amax = 0); scale
    byte = se + 127 (e8m0); element code = e2m1(v / 2^se). Byte j of a row
    holds element 2j in its low nibble and element 2j+1 in its high nibble.
    """
    h = np.asarray(x_bits, dtype=np.uint16)
    r, k = h.shape
    assert k % MX_BLOCK == 0
    v = bf16_bits_to_f64(h).reshape(r, k // MX_BLOCK, MX_BLOCK)
    neg = ((h >> np.uint16(15)) & np.uint16(1)).reshape(v.shape).astype(bool)
    av = np.abs(v)
    amax = av.max(axis=2)
    _, ex = np.frexp(amax)
    e_floor = ex - 1
    se = np.where(amax > 0, np.clip(e_floor - E2M1_EMAX, -127, 127), -127).astype(np.int64)
    scale = (se + 127).astype(np.uint8)
    y = np.ldexp(av, -se[:, :, None])          # exact: power-of-two scaling
    codes = e2m1_code(y, neg).reshape(r, k)
    packed = codes[:, 0::2] | (codes[:, 1::2] << np.uint8(4))
    return packed.astype(np.uint8), scale


def moe_sort_quant(ids: np.ndarray, x_bits: np.ndarray, n: int, block: int,
                   rows_per_chunk: int = 2048, fmt: str = "mxfp8"):
    """Sort pairs into padded expert segments and quantise the gathered rows
    (fmt "mxfp8": e4m3 codes, a_q [total][K]; fmt "mxfp4": packed e2m1
    codes, a_q [total][K/2]).

    Returns dict with sorted_ids, expert_ids, offsets, total, a_q (pad rows
    zero and marked invalid), a_scale [total][K/32], valid [total]. Row p
    (valid) holds the quantised activations of token sorted_ids[p] // k.
    """
    quant = {"mxfp8": mxfp8_quant_rows, "mxfp4": mxfp4_quant_rows}[fmt]
    ids = np.asarray(ids)
    m, k = ids.shape
    sorted_ids, expert_ids, offsets, total = moe_sort(ids, n, block)
    kdim = x_bits.shape[1]
    valid = sorted_ids != m * k
    a_q = np.zeros((total, kdim if fmt == "mxfp8" else kdim // 2), dtype=np.uint8)
    a_scale = np.zeros((total, kdim // MX_BLOCK), dtype=np.uint8)
    pos = np.nonzero(valid)[0]
    for c in range(0, len(pos), rows_per_chunk):
        pc = pos[c:c + rows_per_chunk]
        tok = sorted_ids[pc] // k
        q, s = quant(x_bits[tok])
        a_q[pc] = q
        a_scale[pc] = s
    return dict(sorted_ids=sorted_ids, expert_ids=expert_ids, offsets=offsets,
                total=total, a_q=a_q, a_scale=a_scale, valid=valid)


def route_sort_quant(x_bits, w_bits, bias, k: int, block: int, fmt: str = "mxfp8"):
    """The whole front-end chained: logits -> gate -> sort -> MX quant."""
    logits = router_logits(x_bits, w_bits)
    ids, w = topk_gate(logits, bias, k)
    out = moe_sort_quant(ids, x_bits, w_bits.shape[0], block, fmt=fmt)
    out.update(logits=logits, topk_ids=ids, topk_w=w)
    return out


# ---------------------------------------------------------------------------
# Router split-K partials and the shared expert's SwiGLU [FUSE], [MONO], [OCP]
# ---------------------------------------------------------------------------


def router_partials(x_bits: np.ndarray, w_bits: np.ndarray, s: int) -> np.ndarray:
    """part [S][M][N] fp32: part[s] = fp32( sum over k-slice s of x * W ), the
    slice being K/S consecutive elements (fp64 sums of exact products, rounded
    once). Summed over s they give the logits ([GEMV] opening summary)."""
    x = bf16_bits_to_f64(x_bits)
    w = bf16_bits_to_f64(w_bits)
    k = x.shape[1]
    assert k % s == 0
    ks = k // s
    return np.stack([(x[:, i * ks:(i + 1) * ks] @ w[:, i * ks:(i + 1) * ks].T).astype(np.float32)
                     for i in range(s)])


def e4m3_value(codes: np.ndarray) -> np.ndarray:
    """Exact fp64 value of e4m3fn codes [OCP]: bit 7 the sign, bits 6..3 the
    exponent (bias 7), bits 2..0 the mantissa; exponent field 0 holds the
    subnormals mant * 2^-9; 0x7F and 0xFF are NaN (no infinities)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    e = (c >> 3) & 0xF
    mant = (c & 7).astype(np.float64)
    mag = np.where(e == 0, np.ldexp(mant, -9), np.ldexp(8.0 + mant, e - 10))
    val = np.where(c & 0x80, -mag, mag)
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


def e8m0_value(scales: np.ndarray) -> np.ndarray:
    """2^(b - 127) for the e8m0 scale byte b [OCP]; 255 is NaN."""
    b = np.asarray(scales, dtype=np.uint8).astype(np.int64)
    return np.where(b == 255, np.nan, np.ldexp(1.0, b - 127))


def mxfp8_dequant(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """fp64 [R][K] values of MXFP8 rows: code [R][K] e4m3fn, scale [R][K/32]
    e8m0, element (r, i) = e4m3(code[r][i]) * 2^(scale[r][i // 32] - 127)."""
    c = np.asarray(codes, dtype=np.uint8)
    sc = np.asarray(scales, dtype=np.uint8)
    assert c.ndim == 2 and sc.shape == (c.shape[0], c.shape[1] // MX_BLOCK) and c.shape[1] % MX_BLOCK == 0
    return e4m3_value(c) * np.repeat(e8m0_value(sc), MX_BLOCK, axis=1)


def shared_gate_up(x_bits: np.ndarray, wq: np.ndarray, ws: np.ndarray) -> np.ndarray:
    """gu [M][2I] fp64 = x . W^T with W the dequantised MXFP8 gate_up
    weights (bf16 x e4m3 * 2^e products are exact in fp64)."""
    x = bf16_bits_to_f64(x_bits)
    w = mxfp8_dequant(wq, ws)
    assert np.all(np.isfinite(x)) and np.all(np.isfinite(w))
    return x @ w.T


def silu(g: np.ndarray) -> np.ndarray:
    """silu(g) = g / (1 + exp(-g)) in fp64 (g * sigmoid(g))."""
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def swiglu(gu: np.ndarray, inter: int) -> np.ndarray:
    """h [M][I] = silu(g) * u with g = gu[:, :I] (gate rows first) and
    u = gu[:, I:2I] (up rows), in fp64."""
    gu = np.asarray(gu, dtype=np.float64)
    assert gu.shape[1] == 2 * inter
    return silu(gu[:, :inter]) * gu[:, inter:]


def shared_swiglu(x_bits: np.ndarray, wq: np.ndarray, ws: np.ndarray):
    """(h fp64 [M][I], g [M][I], u [M][I]) of the shared expert's gate/up and
    SwiGLU on MXFP8 gate_up weights wq [2I][K], ws [2I][K/32]."""
    gu = shared_gate_up(x_bits, wq, ws)
    inter = gu.shape[1] // 2
    return swiglu(gu, inter), gu[:, :inter], gu[:, inter:]


# ---------------------------------------------------------------------------
# Stage-1 grouped MoE GEMM on the sorted segments [K3S1], [OCP]
# ---------------------------------------------------------------------------


def e2m1_value(codes: np.ndarray) -> np.ndarray:
    """Exact fp64 value of 4-bit e2m1 codes [OCP]: bit 3 the sign, bits 2..1
    the exponent (bias 1), bit 0 the mantissa; exponent field 0 holds the
    subnormals 0 and 0.5. No infinities or NaN."""
    c = np.asarray(codes, dtype=np.int64) & 0xF
    e = (c >> 1) & 3
    f = (c & 1).astype(np.float64)
    mag = np.where(e == 0, 0.5 * f, np.ldexp(1.0 + 0.5 * f, e - 1))
    return np.where(c & 8, -mag, mag)


def mxfp4_dequant(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """fp64 [R][K] values of MXFP4 rows: packed [R][K/2] (byte j holds
    element 2j in its low nibble and 2j+1 in its high nibble), scales
    [R][K/32] e8m0; element (r, i) = e2m1(code) * 2^(scale[r][i // 32] - 127)."""
    pk = np.asarray(packed, dtype=np.uint8)
    sc = np.asarray(scales, dtype=np.uint8)
    r, half = pk.shape
    k = 2 * half
    assert sc.shape == (r, k // MX_BLOCK) and k % MX_BLOCK == 0
    codes = np.empty((r, k), dtype=np.uint8)
    codes[:, 0::2] = pk & 0xF
    codes[:, 1::2] = pk >> 4
    return e2m1_value(codes) * np.repeat(e8m0_value(sc), MX_BLOCK, axis=1)


def moe_stage1_swiglu(a_q, a_scale, sorted_ids, expert_ids, total: int, n_pairs: int, block: int,
                      w_q, w_scale, rows=None):
    """Stage-1 of the routed experts on the sorted, padded MXFP8 rows.

    For each padded row p < total whose sorted_ids entry is a pair (not the
    sentinel n_pairs): e = expert_ids[p // block], a = the row's MXFP8 values,
    W = expert e's MXFP4 gate_up weights [2I][K]; g = a . W[:I], u = a . W[I:]
    in fp64 (exact products), h = silu(g) * u. Returns (h, g, u) fp64
    [total][I], NaN in pad rows. `rows`: only these padded rows (others NaN).
    """
    w_q = np.asarray(w_q, np.uint8)
    inter = w_q.shape[1] // 2
    h = np.full((total, inter), np.nan)
    g = np.full((total, inter), np.nan)
    u = np.full((total, inter), np.nan)
    sid = np.asarray(sorted_ids)[:total]
    eid = np.asarray(expert_ids)
    want = np.arange(total) if rows is None else np.asarray(rows)
    valid = [p for p in want if sid[p] != n_pairs]
    by_expert = {}
    for p in valid:
        by_expert.setdefault(int(eid[p // block]), []).append(p)
    for e, ps in by_expert.items():
        w = mxfp4_dequant(w_q[e], w_scale[e])
        a = mxfp8_dequant(a_q[ps], a_scale[ps])
        assert np.all(np.isfinite(a)) and np.all(np.isfinite(w))
        gu = a @ w.T
        g[ps] = gu[:, :inter]
        u[ps] = gu[:, inter:]
        h[ps] = silu(g[ps]) * u[ps]
    return h, g, u


# ---------------------------------------------------------------------------
# Routing on the norm's scale [MONO] "route on the norm's scale", [M3R]
# ---------------------------------------------------------------------------


def rmsnorm_route_sort_quant(x_bits, r_bits, gamma_bits, eps: float, w_bits, bias, k: int, block: int,
                             rstd=None, fmt: str = "mxfp8"):
    """The front end fed by the RMSNorm producer: h = x (+ residual), rstd,
    xn = bf16((h * rstd) * (1 + gamma)), then route_sort_quant on xn (router
    logits, gate, sort and the MX quant of the gathered xn rows). The router
    routes on the norm's published scale: its activations are exactly the
    norm's xn. `rstd`: the per-token scale to use (a kernel's own, whose fp32
    sum order is its own); None takes the oracle's fp64 value. Returns the
    route_sort_quant dict plus xn, rstd and h."""
    h = x_bits if r_bits is None else residual_add(x_bits, r_bits)
    if rstd is None:
        rstd = rmsnorm_rstd(h, eps)
    xn = rmsnorm_apply(h, rstd, gamma_bits)
    out = route_sort_quant(xn, w_bits, bias, k, block, fmt=fmt)
    out.update(xn=xn, rstd=np.asarray(rstd, np.float32), h=h)
    return out
