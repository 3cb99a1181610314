"""GPU parity of the expert sort + MX quant (rgt_moe_sort_quant for MXFP8,
rgt_moe_sort_quant_mxfp4 for MXFP4): bit-exact against the oracle fed the same
top-k ids; nothing written past the padded total or into pad rows."""
import numpy as np
import pytest

from _helpers import CANARY, check_sort_quant, say, to_dev, to_dev_bf16
from router_gemv_top_amd.inputs import gen_x

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def R():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import router_gemv_top_amd as R
    R.lib()
    return R


def random_ids(m, n, k, seed, hot=None):
    rng = np.random.default_rng(seed)
    pool = np.arange(n) if hot is None else rng.choice(n, size=hot, replace=False)
    return np.stack([rng.choice(pool, size=k, replace=False) for _ in range(m)]).astype(np.int32)


def run(R, ids, x, n, block, fmt="mxfp8"):
    m, kdim = x.shape
    k = ids.shape[1]
    ws = R.Workspace(m, n, kdim, k, block)
    out = R.alloc_sort_outputs(m, n, kdim, k, block, fill=CANARY, fmt=fmt)
    fn = R.moe_sort_quant if fmt == "mxfp8" else R.moe_sort_quant_mxfp4
    fn(to_dev(ids), to_dev_bf16(x), n, block, ws, out=out)
    torch.cuda.synchronize()
    return out


CASES = [
    (1, 128, 6144, 8, 16, None), (2, 128, 6144, 8, 16, None), (64, 128, 6144, 8, 16, None),
    (64, 128, 6144, 8, 16, 8), (17, 128, 6144, 8, 32, None), (512, 128, 6144, 8, 32, None),
    (32, 896, 3584, 16, 16, None), (1, 896, 3584, 16, 16, None), (3, 16, 512, 4, 64, None),
    (1025, 896, 512, 8, 16, None),      # P = 8200: first size above the one-workgroup sort
    (2048, 128, 1024, 8, 64, 8),        # large path, heavily skewed
]


@pytest.mark.parametrize("m,n,kdim,k,block,hot", CASES)
def test_sort_quant_parity(R, m, n, kdim, k, block, hot):
    say(f"sort_quant M={m} N={n} K={kdim} k={k} B={block} hot={hot}")
    ids = random_ids(m, n, k, seed=m + n, hot=hot)
    x = gen_x(m, kdim, seed=m)
    out = run(R, ids, x, n, block)
    rng = np.random.default_rng(0)
    sample = None if m * k <= 4096 else (lambda nv: rng.choice(nv, size=min(nv, 600), replace=False))
    check_sort_quant(out, ids, x, n, block, sample_rows=sample)


def test_sort_quant_special_values(R):
    say("sort_quant with zero, tiny, huge and negative-zero blocks")
    m, n, kdim, k, block = 4, 16, 512, 2, 16
    x = gen_x(m, kdim, seed=4)
    x[0, :32] = 0x0000
    x[0, 32:64] = 0x8000                      # -0 block
    x[1, :32] = 0x0001                        # smallest subnormal
    x[1, 40] = 0x7F7F                         # largest finite bf16
    x[2, 64:96] = 0x3F80                      # all 1.0
    x[3, 96:128] = np.array([0x3FF8] * 32)    # 1.9375: saturating block
    ids = random_ids(m, n, k, seed=3)
    out = run(R, ids, x, n, block)
    check_sort_quant(out, ids, x, n, block)


def test_sort_quant_prefill_size(R):
    say("sort_quant prefill size M=8192 N=896 K=3584 k=16 B=64")
    m, n, kdim, k, block = 8192, 896, 3584, 16, 64
    ids = random_ids(m, n, k, seed=11)
    x = gen_x(m, kdim, seed=11, dup_frac=0.05)
    out = run(R, ids, x, n, block)
    rng = np.random.default_rng(1)
    check_sort_quant(out, ids, x, n, block, sample_rows=lambda nv: rng.choice(nv, size=800, replace=False))


# MXFP4: the M3.1 point (128 experts, top-4, hidden 6144) over decode and
# wide batches, the many-expert shape, the multi-workgroup sort, and a ragged
# small shape.
CASES_FP4 = [
    (1, 128, 6144, 4, 16, None), (8, 128, 6144, 4, 16, None), (64, 128, 6144, 4, 16, None),
    (1024, 128, 6144, 4, 32, None), (3, 16, 512, 4, 64, None), (32, 896, 3584, 16, 16, None),
    (2048, 128, 1024, 8, 64, 8),
]


@pytest.mark.parametrize("m,n,kdim,k,block,hot", CASES_FP4)
def test_sort_quant_mxfp4_parity(R, m, n, kdim, k, block, hot):
    say(f"sort_quant_mxfp4 M={m} N={n} K={kdim} k={k} B={block} hot={hot}")
    ids = random_ids(m, n, k, seed=m + n + 7, hot=hot)
    x = gen_x(m, kdim, seed=m + 7)
    out = run(R, ids, x, n, block, fmt="mxfp4")
    rng = np.random.default_rng(2)
    sample = None if m * k <= 4096 else (lambda nv: rng.choice(nv, size=min(nv, 600), replace=False))
    check_sort_quant(out, ids, x, n, block, sample_rows=sample, fmt="mxfp4")


def test_sort_quant_mxfp4_special_values(R):
    say("sort_quant_mxfp4 with zero, tiny, huge, negative-zero and tie blocks")
    m, n, kdim, k, block = 4, 16, 512, 2, 16
    x = gen_x(m, kdim, seed=5)
    x[0, :32] = 0x0000
    x[0, 32:64] = 0x8000                      # -0 block
    x[1, :32] = 0x0001                        # smallest subnormal
    x[1, 40] = 0x7F7F                         # largest finite bf16
    x[2, 64:96] = 0x3F80                      # all 1.0
    x[3, 96:128] = np.array([0x40E0] * 32)    # 7.0: ties past 6, saturating
    x[3, 128:160] = np.array([0x4080, 0x3E80, 0x3F40, 0x3FA0, 0x3FE0, 0x4020, 0x4060, 0x40A0] * 4)  # midpoints
    ids = random_ids(m, n, k, seed=6)
    out = run(R, ids, x, n, block, fmt="mxfp4")
    check_sort_quant(out, ids, x, n, block, fmt="mxfp4")
