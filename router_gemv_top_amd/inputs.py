"""Seeded synthetic inputs for the routing front-end.

This module only draws random numbers and packs them as bf16 bit patterns.
It holds none of the routing arithmetic, so both the CPU oracle and the HIP
path can be fed from it without sharing any of the method's code.

Shapes and distributions follow the MoE router shapes named on the pages:
MiniMax-M3 (128 experts, hidden 6144; "MiniMax-M3: Triton split-K router GEMV
with in-kernel split-K fixup", summary paragraph) and Kimi-K3 (896 experts,
top-k 16, hidden 3584; "Kimi-K3: fused MoE routing, sort, quant and epilogue",
Modifications).

Random streams: ``numpy.random.default_rng([seed, stream])`` with one
independent stream per tensor, so W does not change when M changes:
stream 0 = x, 1 = W, 2 = bias, 3 = the duplicated-row choice, 4 = W-row ties,
5 = skew bias, 6 = the shared expert's MXFP8 gate_up weights, 7 = the routed
experts' MXFP4 gate_up weights.

The shared expert's shape is MiniMax-M3.1's 1536 x 6144 gate_up (768 gate
rows, then 768 up rows; "MiniMax-M3.1-Flash MoE/GEMM kernels", Summary: GEMM).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

STREAM_X, STREAM_W, STREAM_BIAS, STREAM_DUP, STREAM_WTIE, STREAM_SKEW, STREAM_SHARED, STREAM_EXPERTS = range(8)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even) and return uint16 bits.

    Inputs must be finite; the generators below never produce NaN or Inf.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 values (exact)."""
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([seed, stream])


def gen_x(m: int, k: int, seed: int = 0, dup_frac: float = 0.0) -> np.ndarray:
    """Activations x[M][K] as bf16 bits, drawn ~N(0, 1).

    With ``dup_frac > 0`` a share of rows (round(dup_frac*M) destination rows,
    drawn without replacement) is overwritten with copies of source rows drawn
    from the remaining rows, so that identical tokens produce identical logits
    and many equal sort keys.
    """
    x = _rng(seed, STREAM_X).standard_normal((m, k), dtype=np.float32)
    xb = f32_to_bf16_bits(x)
    ndup = int(round(dup_frac * m))
    if ndup > 0:
        r = _rng(seed, STREAM_DUP)
        dst = r.choice(m, size=ndup, replace=False)
        rest = np.setdiff1d(np.arange(m), dst)
        src = r.choice(rest, size=ndup, replace=True)
        xb[dst] = xb[src]
    return xb


def gen_w(n: int, k: int, seed: int = 0, std: float = 0.02, tie_rows: int = 0) -> np.ndarray:
    """Router weight W[N][K] as bf16 bits, drawn ~N(0, std^2).

    ``tie_rows > 0`` copies that many rows onto other rows, so some experts
    score exactly alike in every token and the index tie-break is exercised.
    """
    w = std * _rng(seed, STREAM_W).standard_normal((n, k), dtype=np.float32)
    wb = f32_to_bf16_bits(w)
    if tie_rows > 0:
        r = _rng(seed, STREAM_WTIE)
        dst = r.choice(n, size=tie_rows, replace=False)
        rest = np.setdiff1d(np.arange(n), dst)
        src = r.choice(rest, size=tie_rows, replace=True)
        wb[dst] = wb[src]
    return wb


def gen_bias(n: int, seed: int = 0, std: float = 0.1) -> np.ndarray:
    """Per-expert fp32 router bias ~N(0, std^2)."""
    return (std * _rng(seed, STREAM_BIAS).standard_normal(n)).astype(np.float32)


def gen_skew_bias(n: int, hot: int, seed: int = 0, lift: float = 8.0) -> np.ndarray:
    """A bias that lifts ``hot`` chosen experts far above the rest, so that
    almost every token routes to the same few experts (skewed routing)."""
    b = np.zeros(n, dtype=np.float32)
    b[_rng(seed, STREAM_SKEW).choice(n, size=hot, replace=False)] = lift
    return b


@dataclass(frozen=True)
class Workload:
    """One routing configuration: sizes, top-k, block size and input recipe."""
    name: str
    m: int
    n: int
    k: int
    topk: int
    block: int
    bias: bool = False
    dup_frac: float = 0.0
    seed: int = 0

    def make(self):
        """Return (x_bits[M][K] u16, w_bits[N][K] u16, bias f32[N] or None)."""
        x = gen_x(self.m, self.k, self.seed, self.dup_frac)
        w = gen_w(self.n, self.k, self.seed)
        b = gen_bias(self.n, self.seed) if self.bias else None
        return x, w, b


def gen_mxfp8_weights(rows: int, k: int, seed: int = 0, scale_lo: int = 110, scale_hi: int = 116):
    """(codes uint8 [rows][K], scales uint8 [rows][K/32]) of random MXFP8
    weights: element codes uniform over the 254 non-NaN e4m3fn bytes (the NaN
    bytes 0x7F and 0xFF are redrawn as 0x00), scale bytes uniform in
    [scale_lo, scale_hi), so elements are at most 448 * 2^(scale_hi - 128)."""
    rng = _rng(seed, STREAM_SHARED)
    codes = rng.integers(0, 256, size=(rows, k), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0
    scales = rng.integers(scale_lo, scale_hi, size=(rows, k // 32), dtype=np.uint8)
    return codes, scales


def gen_mxfp4_expert_weights(n: int, rows: int, k: int, seed: int = 0, scale_lo: int = 118, scale_hi: int = 122):
    """(codes uint8 [n][rows][k/2], scales uint8 [n][rows][k/32]) of random
    MXFP4 expert weights: every byte holds two e2m1 codes drawn uniformly over
    all 16 (the format has no NaN), scale bytes uniform in [scale_lo,
    scale_hi), so elements are at most 6 * 2^(scale_hi - 128)."""
    rng = _rng(seed, STREAM_EXPERTS)
    codes = rng.integers(0, 256, size=(n, rows, k // 2), dtype=np.uint8)
    scales = rng.integers(scale_lo, scale_hi, size=(n, rows, k // 32), dtype=np.uint8)
    return codes, scales


def workloads_decode_128(ms=(1, 2, 4, 8, 16, 32, 64)):
    """MiniMax-M3-shaped decode sweep: N=128 experts, K=6144, top-8, block 16."""
    return [Workload(f"m3_decode_M{m}", m, 128, 6144, 8, 16) for m in ms]


def workload_tiny():
    """Tiny case: one token, K=6144, N=128, top-8, block 16, seed 0."""
    return Workload("tiny_M1", 1, 128, 6144, 8, 16)


def workloads_wide_128(ms=(128, 256, 512)):
    """Wide-batch router: N=128, K=6144, top-8, block 32."""
    return [Workload(f"m3_wide_M{m}", m, 128, 6144, 8, 32) for m in ms]


def workloads_decode_896(ms=(1, 4, 8, 16, 32)):
    """Many-expert decode: N=896, K=3584, fp32 bias, top-16, block 16."""
    return [Workload(f"k3_decode_M{m}", m, 896, 3584, 16, 16, bias=True) for m in ms]


def workload_prefill_896(m: int = 8192):
    """Prefill-sized routing: N=896, K=3584, top-16, block 64, 5% duplicate tokens."""
    return Workload(f"k3_prefill_M{m}", m, 896, 3584, 16, 64, dup_frac=0.05)


def workloads_decode_128_top4(ms=(1, 2, 4, 8, 16, 32, 64)):
    """The 128-expert, top-4, hidden-6144 decode point whose sort carries the
    stage-1 MXFP4 activation quant (MiniMax-M3.1-Flash MoE/GEMM kernels,
    "Changes to existing kernels"); same input recipe as the top-8 sweep."""
    return [Workload(f"decode_top4_M{m}", m, 128, 6144, 4, 16) for m in ms]
