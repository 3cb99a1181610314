"""C-ABI checks that need no GPU: the library loads, exports every function
include/rgt.h declares, and rejects bad arguments with the documented status
codes before any HIP call."""
import ctypes
import os
import re

import pytest

from oracle import rgt_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rgt.h")

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def L():
    import router_gemv_top_amd as R
    return R.lib()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(rgt_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_function(L):
    names = declared_functions()
    assert len(names) >= 12
    assert {"rgt_moe_sort_quant_mxfp4", "rgt_route_sort_quant_mxfp4"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    import router_gemv_top_amd as R
    for s in range(6):
        assert R.status_string(s)
    assert R.version() >= 100


def test_sort_capacity_matches_oracle(L):
    import router_gemv_top_amd as R
    for (m, n, k, b) in [(1, 128, 8, 16), (64, 128, 8, 16), (512, 128, 8, 32), (32, 896, 16, 16),
                         (8192, 896, 16, 64), (0, 128, 8, 16), (3, 16, 4, 64)]:
        assert R.sort_capacity(m, n, k, b) == O.sort_capacity(m, n, k, b)
    assert R.sort_capacity(1, 128, 8, 8) == -1          # block not covered
    assert R.sort_capacity(1, 128, 33, 16) == -1        # topk > 32


def test_coverage(L):
    import router_gemv_top_amd as R
    assert R.router_supported(64, 128, 6144)
    assert R.router_supported(8192, 896, 3584)
    assert not R.router_supported(8193, 128, 6144)
    assert not R.router_supported(4, 130, 6144)        # N % 16
    assert not R.router_supported(4, 128, 6000)        # K % 512
    assert not R.router_supported(4, 2048, 6144)       # N > 1024
    assert R.workspace_bytes(64, 128, 6144, 8, 16) > 0
    assert R.workspace_bytes(64, 128, 6000, 8, 16) == 0
    sizes = [R.workspace_bytes(m, 896, 3584, 16, 16) for m in (1, 8, 9, 64, 65, 512)]
    assert sizes == sorted(sizes)


FAKE = 1 << 20   # an aligned, never dereferenced address


def call_router(L, x=FAKE, ldx=6144, w=FAKE, ldw=6144, out=FAKE, m=4, n=128, k=6144, ws=FAKE, wsb=1 << 30):
    return L.rgt_router_logits(x, ldx, w, ldw, out, m, n, k, ws, wsb, None)


def test_router_argument_errors(L):
    assert call_router(L, m=0, x=None) == 0            # M == 0: no-op
    assert call_router(L, n=130) == 1                  # unsupported
    assert call_router(L, x=None) == 2                 # null x
    assert call_router(L, x=FAKE + 2) == 2             # misaligned x
    assert call_router(L, ldx=6000) == 2               # ld < K
    assert call_router(L, ldx=6148) == 2               # ld % 8
    assert call_router(L, out=FAKE + 2) == 2           # misaligned logits
    assert call_router(L, ws=None) == 3                # no workspace
    assert call_router(L, ws=FAKE + 64) == 3           # misaligned workspace
    assert call_router(L, wsb=1024) == 3               # too small


def test_gate_argument_errors(L):
    f = L.rgt_topk_gate
    assert f(FAKE, None, 0, 128, 8, FAKE, FAKE, None) == 0
    assert f(FAKE, None, 4, 128, 0, FAKE, FAKE, None) == 1
    assert f(FAKE, None, 4, 128, 33, FAKE, FAKE, None) == 1
    assert f(FAKE, None, 4, 16, 17, FAKE, FAKE, None) == 1
    assert f(None, None, 4, 128, 8, FAKE, FAKE, None) == 2
    assert f(FAKE, FAKE + 1, 4, 128, 8, FAKE, FAKE, None) == 2


@pytest.mark.parametrize("entry", ["rgt_moe_sort_quant", "rgt_moe_sort_quant_mxfp4"])
def test_sort_quant_argument_errors(L, entry):
    f = getattr(L, entry)
    ok = dict(ids=FAKE, x=FAKE, ldx=6144, m=4, n=128, k=6144, topk=8, block=16, s=FAKE, e=FAKE, o=FAKE,
              q=FAKE, sc=FAKE, ws=FAKE, wsb=1 << 30)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["ids"], a["x"], a["ldx"], a["m"], a["n"], a["k"], a["topk"], a["block"], a["s"], a["e"],
                 a["o"], a["q"], a["sc"], a["ws"], a["wsb"], None)

    assert call(block=8) == 1
    assert call(topk=0) == 1
    assert call(ids=None) == 2
    assert call(q=FAKE + 4) == 2
    assert call(sc=FAKE + 2) == 2
    assert call(s=None) == 2
    assert call(wsb=100) == 3


@pytest.mark.parametrize("entry", ["rgt_route_sort_quant", "rgt_route_sort_quant_mxfp4"])
def test_route_sort_quant_argument_errors(L, entry):
    f = getattr(L, entry)

    def call(x=FAKE, w=FAKE, bias=None, m=4, n=128, k=6144, topk=8, block=16, logits=None, ids=FAKE,
             tw=FAKE, ws=FAKE, wsb=1 << 30):
        return f(x, k, w, k, bias, m, n, k, topk, block, logits, ids, tw, FAKE, FAKE, FAKE, FAKE, FAKE,
                 ws, wsb, None)

    assert call(m=0) == 0
    assert call(n=100) == 1
    assert call(block=128) == 1
    assert call(tw=None) == 2
    assert call(bias=FAKE + 2) == 2
    assert call(logits=FAKE + 1) == 2
    assert call(wsb=256) == 3


def test_workspace_helpers_reject_bad_buffers(L):
    assert L.rgt_reset_workspace(None, 1024, None) == 3
    assert L.rgt_check_workspace(FAKE + 8, 1024, None) == 3
    assert L.rgt_check_workspace(FAKE, 16, None) == 3


def test_gate_partials_argument_errors(L):
    f = L.rgt_topk_gate_partials

    def call(part=FAKE, s=4, bias=None, m=4, n=128, topk=8, logits=None, ids=FAKE, w=FAKE):
        return f(part, s, bias, m, n, topk, logits, ids, w, None)

    assert call(m=0) == 0
    assert call(s=0) == 1
    assert call(s=1025) == 1
    assert call(n=100) == 1
    assert call(topk=33) == 1
    assert call(part=None) == 2
    assert call(part=FAKE + 2) == 2
    assert call(logits=FAKE + 1) == 2
    assert call(w=None) == 2


def test_rmsnorm_argument_errors(L):
    f = L.rgt_rmsnorm

    def call(x=FAKE, ldx=6144, r=None, ldr=0, g=FAKE, eps=1e-6, m=4, k=6144, xn=FAKE, ldxn=6144, ro=None, ldro=0,
             rstd=None):
        return f(x, ldx, r, ldr, g, eps, m, k, xn, ldxn, ro, ldro, rstd, None)

    assert call(m=0) == 0
    assert call(k=6) == 1 and call(k=16392) == 1 and call(k=100) == 1
    assert call(x=None) == 2 and call(g=FAKE + 2) == 2 and call(xn=FAKE + 8) == 2
    assert call(ldx=100) == 2 and call(ldxn=6146) == 2
    assert call(eps=-1.0) == 2
    assert call(ro=FAKE, ldro=6144) == 2          # residual_out without a residual
    assert call(r=FAKE, ldr=6100) == 2
    assert call(rstd=FAKE + 1) == 2


@pytest.mark.parametrize("entry", ["rgt_rmsnorm_route_sort_quant", "rgt_rmsnorm_route_sort_quant_mxfp4"])
def test_rmsnorm_route_sort_quant_argument_errors(L, entry):
    """Both calls' argument rules apply, checked before any launch."""
    f = getattr(L, entry)

    def call(x=FAKE, r=None, ldr=0, g=FAKE, eps=1e-6, m=4, n=128, k=6144, topk=8, block=16, xn=FAKE, ldxn=6144,
             ro=None, ldro=0, rstd=None, tw=FAKE, wsb=1 << 30):
        return f(x, k, r, ldr, g, eps, FAKE, k, None, m, n, k, topk, block, xn, ldxn, ro, ldro, rstd, None, FAKE,
                 tw, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, wsb, None)

    assert call(m=0) == 0
    assert call(n=100) == 1 and call(block=128) == 1
    assert call(tw=None) == 2
    assert call(g=None) == 2 and call(g=FAKE + 2) == 2
    assert call(xn=None) == 2 and call(xn=FAKE + 8) == 2 and call(ldxn=6146) == 2
    assert call(eps=-1.0) == 2
    assert call(ro=FAKE, ldro=6144) == 2          # residual_out without a residual
    assert call(r=FAKE, ldr=6100) == 2
    assert call(rstd=FAKE + 1) == 2
    assert call(wsb=256) == 3


def test_router_shared_swiglu_argument_errors(L):
    S = L.rgt_router_partial_slices
    # VALU plan at M = 4 (three slices of 2048), MFMA plan at M = 16 (twelve of 512)
    assert S(4, 128, 6144) == 3 and S(16, 128, 6144) == 12
    assert S(0, 128, 6144) == 0 and S(17, 128, 6144) == 0 and S(4, 100, 6144) == 0
    assert S(4, 128, 8704) == 0 and S(4, 128, 6000) == 0
    f = L.rgt_router_shared_swiglu

    def call(x=FAKE, ldx=6144, w=FAKE, ldw=6144, m=4, n=128, k=6144, part=FAKE, s=3, q=FAKE, sc=FAKE, inter=768,
             h=FAKE, ldh=768):
        return f(x, ldx, w, ldw, m, n, k, part, s, q, sc, inter, h, ldh, None)

    assert call(m=0) == 0
    assert call(m=17) == 1 and call(n=100) == 1 and call(k=8704) == 1 and call(inter=0) == 1
    assert call(s=4) == 2 and call(part=None) == 2 and call(part=FAKE + 4) == 2
    assert call(q=None) == 2 and call(q=FAKE + 8) == 2 and call(sc=None) == 2
    assert call(h=None) == 2 and call(h=FAKE + 1) == 2 and call(ldh=767) == 2
    assert call(x=FAKE + 2) == 2 and call(ldx=6000) == 2


def test_route_sort_quant_noalloc_argument_errors(L):
    f = L.rgt_route_sort_quant_noalloc

    def call(x=FAKE, w=FAKE, bias=None, m=4, n=128, k=6144, topk=8, block=16, logits=None, ids=FAKE, tw=FAKE):
        return f(x, k, w, k, bias, m, n, k, topk, block, logits, ids, tw, FAKE, FAKE, FAKE, FAKE, FAKE, None)

    assert call(m=0) == 0
    assert call(n=100) == 1
    assert call(block=128) == 1
    assert call(tw=None) == 2
    assert call(x=FAKE + 2) == 2
    assert call(bias=FAKE + 2) == 2
    # a workspace beyond the library's 8 MiB scratch array: unsupported, nothing launched
    assert call(m=1024, n=1024, k=8192, topk=32, block=64) == 1
    assert L.rgt_last_launch_count() == 0
