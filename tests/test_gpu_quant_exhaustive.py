"""MXFP8 and MXFP4 encoders over their whole input space: every finite bf16
value, placed in blocks whose largest element sets the shared exponent 0 to 17
binades above the value's own (saturation, every normal and subnormal element
binade, and rounding to zero), quantised on the GPU through
rgt_moe_sort_quant / rgt_moe_sort_quant_mxfp4 and compared bit for bit with
the oracle."""
import numpy as np
import pytest

from _helpers import say, to_dev, to_dev_bf16
from oracle import rgt_oracle as O

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

K = 6144
BLOCK = 32
GAPS = tuple(range(18))


def bf16_binade(h):
    """floor(log2 |v|) of nonzero finite bf16 bit patterns."""
    e = (h >> 7) & 0xFF
    m = h & 0x7F
    sub = np.floor(np.log2(np.maximum(m, 1))).astype(np.int64) - 133
    return np.where(e > 0, e.astype(np.int64) - 127, sub)


def pow2_bf16(E):
    """bf16 bits of 2^E, E in [-133, 127]."""
    E = np.asarray(E, dtype=np.int64)
    normal = ((E + 127) << 7).astype(np.uint16)
    sub = (np.uint16(1) << np.clip(E + 133, 0, 6).astype(np.uint16)).astype(np.uint16)
    return np.where(E >= -126, normal, sub).astype(np.uint16)


def exhaustive_rows(seed=0):
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    finite_nonzero = (((h >> 7) & 0xFF) != 0xFF) & ((h & 0x7FFF) != 0)
    vals = h[finite_nonzero]
    b = bf16_binade(vals)
    blocks = []
    rng = np.random.default_rng(seed)
    for gap in GAPS:
        top = np.minimum(b + gap, 127)
        for E in np.unique(top):
            members = vals[top == E]
            members = members[rng.permutation(members.size)]
            for i in range(0, members.size, BLOCK - 1):
                chunk = members[i:i + BLOCK - 1]
                blk = np.zeros(BLOCK, dtype=np.uint16)          # +0 fills short blocks
                blk[0] = pow2_bf16(E)
                blk[1:1 + chunk.size] = chunk
                blocks.append(blk)
    # signed zeros and the block maxima themselves with a negative sign
    zb = np.zeros(BLOCK, dtype=np.uint16)
    zb[1::2] = 0x8000
    blocks.append(zb)
    blocks = np.stack(blocks)
    per_row = K // BLOCK
    pad = (-len(blocks)) % per_row
    if pad:
        blocks = np.concatenate([blocks, np.zeros((pad, BLOCK), dtype=np.uint16)])
    return blocks.reshape(-1, K)


def test_mxfp8_encoder_every_bf16():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import router_gemv_top_amd as R
    x = exhaustive_rows()
    m = x.shape[0]
    say(f"exhaustive MXFP8: {m} rows x {K}")
    n, topk, block = 16, 1, 16
    ids = np.zeros((m, topk), dtype=np.int32)       # every token to expert 0: a_q row p = token p
    ws = R.Workspace(m, n, K, topk, block)
    out = R.moe_sort_quant(to_dev(ids), to_dev_bf16(x), n, block, ws)
    torch.cuda.synchronize()
    codes, scales = O.mxfp8_quant_rows(x)
    got_q = out["a_q"][:m].cpu().numpy()
    got_s = out["a_scale"][:m].cpu().numpy()
    bad = np.argwhere(got_q != codes)
    if bad.size:
        r, c = bad[0]
        raise AssertionError(f"{len(bad)} codes differ; first row {r} col {c}: bf16 0x{x[r, c]:04x} "
                             f"block max 0x{x[r, c - c % BLOCK]:04x} got 0x{got_q[r, c]:02x} "
                             f"want 0x{codes[r, c]:02x}")
    np.testing.assert_array_equal(got_s, scales)


def test_mxfp4_encoder_every_bf16():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import router_gemv_top_amd as R
    x = exhaustive_rows(seed=1)
    m = x.shape[0]
    say(f"exhaustive MXFP4: {m} rows x {K}")
    n, topk, block = 16, 1, 16
    ids = np.zeros((m, topk), dtype=np.int32)       # every token to expert 0: a_q row p = token p
    ws = R.Workspace(m, n, K, topk, block)
    out = R.moe_sort_quant_mxfp4(to_dev(ids), to_dev_bf16(x), n, block, ws)
    torch.cuda.synchronize()
    packed, scales = O.mxfp4_quant_rows(x)
    got_q = out["a_q"][:m].cpu().numpy()
    got_s = out["a_scale"][:m].cpu().numpy()
    assert got_q.shape == packed.shape
    bad = np.argwhere(got_q != packed)
    if bad.size:
        r, c = bad[0]
        raise AssertionError(f"{len(bad)} bytes differ; first row {r} byte {c}: bf16 0x{x[r, 2 * c]:04x} "
                             f"0x{x[r, 2 * c + 1]:04x} block max 0x{x[r, 2 * c - 2 * c % BLOCK]:04x} "
                             f"got 0x{got_q[r, c]:02x} want 0x{packed[r, c]:02x}")
    np.testing.assert_array_equal(got_s, scales)
