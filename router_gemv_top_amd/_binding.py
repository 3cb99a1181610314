"""ctypes binding of ``librgt.so`` (the C ABI declared in include/rgt.h).

Argument marshalling only: every step of the routing path runs in the HIP
kernels of the library. torch is used for device memory and the current
stream. The library must be built (``python -m router_gemv_top_amd.build``);
without it every call raises, there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# RGT_LIBRARY selects another build of the same ABI (e.g. librgt_trace.so).
LIB_PATH = os.environ.get("RGT_LIBRARY") or os.path.join(_HERE, "librgt.so")

RGT_OK, RGT_ERR_UNSUPPORTED, RGT_ERR_INVALID, RGT_ERR_WORKSPACE, RGT_ERR_HIP, RGT_ERR_TIMEOUT = range(6)

_lib = None
_lock = threading.Lock()


class RgtError(RuntimeError):
    """A non-OK status from the library."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


class RgtUnsupported(RgtError):
    """Shape outside coverage: the caller may fall back to another path."""


def _hip_runtimes_loaded():
    with open("/proc/self/maps") as f:
        return sorted({ln.split()[-1] for ln in f if "libamdhip64" in ln})


def lib() -> ctypes.CDLL:
    """Load the library once (after torch, so torch's HIP runtime is the one
    it binds to) and declare the signatures."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m router_gemv_top_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
        sigs = {
            "rgt_status_string": ([i32], ctypes.c_char_p),
            "rgt_version": ([], i32),
            "rgt_workspace_bytes": ([i32, i32, i32, i32, i32], sz),
            "rgt_sort_capacity": ([i32, i32, i32, i32], i64),
            "rgt_router_supported": ([i32, i32, i32], i32),
            "rgt_reset_workspace": ([vp, sz, vp], i32),
            "rgt_check_workspace": ([vp, sz, vp], i32),
            "rgt_router_logits": ([vp, i64, vp, i64, vp, i32, i32, i32, vp, sz, vp], i32),
            "rgt_topk_gate": ([vp, vp, i32, i32, i32, vp, vp, vp], i32),
            "rgt_topk_gate_partials": ([vp, i32, vp, i32, i32, i32, vp, vp, vp, vp], i32),
            "rgt_moe_sort_quant": ([vp, vp, i64, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp], i32),
            "rgt_route_sort_quant": ([vp, i64, vp, i64, vp, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp,
                                      vp, vp, vp, sz, vp], i32),
            "rgt_route_sort_quant_noalloc": ([vp, i64, vp, i64, vp, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp,
                                              vp, vp, vp, vp], i32),
            "rgt_moe_sort_quant_mxfp4": ([vp, vp, i64, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp],
                                         i32),
            "rgt_route_sort_quant_mxfp4": ([vp, i64, vp, i64, vp, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp,
                                            vp, vp, vp, sz, vp], i32),
            "rgt_router_partial_slices": ([i32, i32, i32], i32),
            "rgt_moe_stage1_swiglu": ([vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp, vp, i32, vp, i64, vp], i32),
            "rgt_router_shared_swiglu": ([vp, i64, vp, i64, i32, i32, i32, vp, i32, vp, vp, i32, vp, i64, vp], i32),
            "rgt_rmsnorm": ([vp, i64, vp, i64, vp, ctypes.c_float, i32, i32, vp, i64, vp, i64, vp, vp], i32),
            "rgt_reload_env": ([], None),
            "rgt_rmsnorm_route_sort_quant": ([vp, i64, vp, i64, vp, ctypes.c_float, vp, i64, vp, i32, i32, i32, i32,
                                              i32, vp, i64, vp, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                              ctypes.c_size_t, vp], i32),
            "rgt_rmsnorm_route_sort_quant_mxfp4": ([vp, i64, vp, i64, vp, ctypes.c_float, vp, i64, vp, i32, i32, i32,
                                                    i32, i32, vp, i64, vp, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                                    vp, ctypes.c_size_t, vp], i32),
            "rgt_last_launch_count": ([], i32),
            "rgt_diag_read": ([vp, sz, vp, i32, vp], i32),
            "rgt_diag_copy": ([vp, vp, sz, i32, vp], i32),
        }
        for name, (args, res) in sigs.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        runtimes = _hip_runtimes_loaded()
        if len(runtimes) > 1:
            raise RuntimeError(f"more than one HIP runtime loaded in this process: {runtimes}")
        _lib = L
    return _lib


def exported_symbols():
    return [n for n in dir(lib()) if n.startswith("rgt_")]


def status_string(status: int) -> str:
    return lib().rgt_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status == RGT_OK:
        return
    if status == RGT_ERR_UNSUPPORTED:
        raise RgtUnsupported(status, where)
    raise RgtError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def version() -> int:
    return lib().rgt_version()


def workspace_bytes(max_m: int, n: int, k: int, topk: int, block: int) -> int:
    return lib().rgt_workspace_bytes(max_m, n, k, topk, block)


def sort_capacity(m: int, n: int, topk: int, block: int) -> int:
    return lib().rgt_sort_capacity(m, n, topk, block)


def router_supported(m: int, n: int, k: int) -> bool:
    return lib().rgt_router_supported(m, n, k) == RGT_OK


def last_launch_count() -> int:
    return lib().rgt_last_launch_count()


class Workspace:
    """Caller-owned, zero-initialised device workspace for one stream."""

    def __init__(self, max_m: int, n: int, k: int, topk: int, block: int, device="cuda"):
        nbytes = workspace_bytes(max_m, n, k, topk, block)
        if nbytes == 0:
            raise RgtUnsupported(RGT_ERR_UNSUPPORTED, "workspace_bytes")
        self.nbytes = nbytes
        self.buf = torch.zeros(nbytes, dtype=torch.uint8, device=device)  # zero-filled once

    def reset(self, stream=None):
        _check(lib().rgt_reset_workspace(_ptr(self.buf), self.nbytes, _stream(stream)), "reset_workspace")

    def check(self, stream=None) -> int:
        return lib().rgt_check_workspace(_ptr(self.buf), self.nbytes, _stream(stream))


def reset_workspace(ws: Workspace, stream=None):
    ws.reset(stream)


def check_workspace(ws: Workspace, stream=None) -> int:
    return ws.check(stream)


def _bf16_2d(t, name):
    if t.dtype != torch.bfloat16 or t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D bfloat16 tensor with a contiguous last dimension")
    return t


def router_logits(x, w, ws: Workspace, logits=None, stream=None):
    """logits[M][N] fp32 = x[M][K] . W[N][K]^T (bf16 in, fp32 out)."""
    _bf16_2d(x, "x"), _bf16_2d(w, "w")
    m, k = x.shape
    n = w.shape[0]
    if logits is None:
        logits = torch.empty((m, n), dtype=torch.float32, device=x.device)
    _check(lib().rgt_router_logits(_ptr(x), x.stride(0), _ptr(w), w.stride(0), _ptr(logits), m, n, k,
                                   _ptr(ws.buf), ws.nbytes, _stream(stream)), "router_logits")
    return logits


def router_partial_slices(m: int, n: int, k: int) -> int:
    """S of the router partials router_shared_swiglu writes (0: not covered)."""
    return int(lib().rgt_router_partial_slices(m, n, k))


def router_shared_swiglu(x, w, wsh_q, wsh_scale, part=None, h=None, stream=None):
    """(part fp32 [S][M][N], h bf16 [M][I]) from one launch: the router's
    k-slice partials of x . W^T and the shared expert's SwiGLU
    h = silu(x . Wg^T) * (x . Wu^T) on MXFP8 gate_up weights wsh_q uint8
    [2I][K] (gate rows first) with e8m0 scales wsh_scale uint8 [2I][K/32]."""
    _bf16_2d(x, "x"), _bf16_2d(w, "w")
    m, k = x.shape
    n = w.shape[0]
    if wsh_q.dtype != torch.uint8 or wsh_q.dim() != 2 or not wsh_q.is_contiguous() or wsh_q.shape[1] != k:
        raise ValueError("wsh_q must be a contiguous [2I][K] uint8 tensor")
    if (wsh_scale.dtype != torch.uint8 or not wsh_scale.is_contiguous()
            or tuple(wsh_scale.shape) != (wsh_q.shape[0], k // 32)):
        raise ValueError("wsh_scale must be a contiguous [2I][K/32] uint8 tensor")
    inter = wsh_q.shape[0] // 2
    s = router_partial_slices(m, n, k) if m > 0 else 1
    if s <= 0:
        raise RgtUnsupported(RGT_ERR_UNSUPPORTED, "router_partial_slices")
    if part is None:
        part = torch.empty((s, m, n), dtype=torch.float32, device=x.device)
    if h is None:
        h = torch.empty((m, inter), dtype=torch.bfloat16, device=x.device)
    if part.dtype != torch.float32 or not part.is_contiguous() or tuple(part.shape) != (s, m, n):
        raise ValueError(f"part must be a contiguous [{s}][{m}][{n}] float32 tensor")
    if h.dtype != torch.bfloat16 or h.dim() != 2 or h.stride(1) != 1 or h.shape[0] != m or h.shape[1] < inter:
        raise ValueError("h must be a [M][>= I] bfloat16 tensor with unit column stride")
    _check(lib().rgt_router_shared_swiglu(_ptr(x), x.stride(0), _ptr(w), w.stride(0), m, n, k, _ptr(part), s,
                                          _ptr(wsh_q), _ptr(wsh_scale), inter, _ptr(h), h.stride(0),
                                          _stream(stream)), "router_shared_swiglu")
    return part, h


def topk_gate(logits, topk: int, bias=None, ids=None, weights=None, stream=None):
    """(topk_ids int32 [M][topk], topk_w fp32 [M][topk]) of the softmax top-k gate."""
    m, n = logits.shape
    if ids is None:
        ids = torch.empty((m, topk), dtype=torch.int32, device=logits.device)
    if weights is None:
        weights = torch.empty((m, topk), dtype=torch.float32, device=logits.device)
    _check(lib().rgt_topk_gate(_ptr(logits), _ptr(bias), m, n, topk, _ptr(ids), _ptr(weights), _stream(stream)),
           "topk_gate")
    return ids, weights


def topk_gate_partials(part, topk: int, bias=None, logits=None, ids=None, weights=None, stream=None):
    """(topk_ids, topk_w) of the gate fed split-K partials part [S][M][N] fp32,
    summed in slice order; logits (if given, [M][N] fp32) receives the sum."""
    if part.dtype != torch.float32 or part.dim() != 3 or not part.is_contiguous():
        raise ValueError("part must be a contiguous [S][M][N] float32 tensor")
    s, m, n = part.shape
    if ids is None:
        ids = torch.empty((m, topk), dtype=torch.int32, device=part.device)
    if weights is None:
        weights = torch.empty((m, topk), dtype=torch.float32, device=part.device)
    _check(lib().rgt_topk_gate_partials(_ptr(part), s, _ptr(bias), m, n, topk, _ptr(logits), _ptr(ids),
                                        _ptr(weights), _stream(stream)), "topk_gate_partials")
    return ids, weights


def alloc_sort_outputs(m: int, n: int, k: int, topk: int, block: int, device="cuda", fill: int | None = None,
                       fmt: str = "mxfp8"):
    """Device buffers sized to the sort capacity (optionally pre-filled with a
    canary byte so that writes past the padded total can be detected). a_q
    has K bytes a row for MXFP8, K/2 for MXFP4."""
    if fmt not in ("mxfp8", "mxfp4"):
        raise ValueError(f"unknown activation format {fmt!r}")
    cap = sort_capacity(m, n, topk, block)
    if cap < 0:
        raise RgtUnsupported(RGT_ERR_UNSUPPORTED, "sort_capacity")
    cap = max(cap, block)

    def mk(shape, dt):
        if fill is None:
            return torch.empty(shape, dtype=dt, device=device)
        nbytes = torch.tensor([], dtype=dt).element_size()
        numel = 1
        for d in shape:
            numel *= d
        # every byte set to `fill`, whatever the element type
        return torch.full((numel * nbytes,), fill, dtype=torch.uint8, device=device).view(dt).view(shape)
    return dict(
        sorted_ids=mk((cap,), torch.int32),
        expert_ids=mk((cap // block,), torch.int32),
        offsets=mk((n + 1,), torch.int32),
        a_q=mk((cap, k if fmt == "mxfp8" else k // 2), torch.uint8),
        a_scale=mk((cap, k // 32), torch.uint8),
    )


def moe_sort_quant(topk_ids, x, n: int, block: int, ws: Workspace, out=None, stream=None):
    """Sort pairs into block-padded expert segments and MXFP8-quantise the
    gathered rows of x. Returns the dict of output buffers."""
    return _moe_sort_quant(lib().rgt_moe_sort_quant, "mxfp8", topk_ids, x, n, block, ws, out, stream)


def moe_sort_quant_mxfp4(topk_ids, x, n: int, block: int, ws: Workspace, out=None, stream=None):
    """As moe_sort_quant, with MXFP4 rows (K/2 bytes of packed e2m1 codes)."""
    return _moe_sort_quant(lib().rgt_moe_sort_quant_mxfp4, "mxfp4", topk_ids, x, n, block, ws, out, stream)


def _moe_sort_quant(fn, fmt, topk_ids, x, n, block, ws, out, stream):
    _bf16_2d(x, "x")
    m, k = x.shape
    topk = topk_ids.shape[1]
    if out is None:
        out = alloc_sort_outputs(m, n, k, topk, block, x.device, fmt=fmt)
    _check(fn(_ptr(topk_ids), _ptr(x), x.stride(0), m, n, k, topk, block,
              _ptr(out["sorted_ids"]), _ptr(out["expert_ids"]), _ptr(out["offsets"]),
              _ptr(out["a_q"]), _ptr(out["a_scale"]), _ptr(ws.buf), ws.nbytes,
              _stream(stream)), fn.__name__[4:])
    return out


def route_sort_quant(x, w, topk: int, block: int, ws: Workspace, bias=None, out=None, want_logits=True,
                     stream=None):
    """The whole front end (one launch for M <= 64). Returns a dict with
    logits (if requested), topk_ids, topk_w and the sort/quant buffers."""
    return _route_sort_quant(lib().rgt_route_sort_quant, "mxfp8", x, w, topk, block, ws, bias, out, want_logits,
                             stream)


def route_sort_quant_mxfp4(x, w, topk: int, block: int, ws: Workspace, bias=None, out=None, want_logits=True,
                           stream=None):
    """As route_sort_quant, with MXFP4 rows (K/2 bytes of packed e2m1 codes)."""
    return _route_sort_quant(lib().rgt_route_sort_quant_mxfp4, "mxfp4", x, w, topk, block, ws, bias, out,
                             want_logits, stream)


def route_sort_quant_noalloc(x, w, topk: int, block: int, bias=None, out=None, want_logits=True, stream=None):
    """As route_sort_quant, on the library's own per-GPU scratch array (no
    workspace argument; the call allocates no device memory)."""
    return _route_sort_quant(lib().rgt_route_sort_quant_noalloc, "mxfp8", x, w, topk, block, None, bias, out,
                             want_logits, stream)


def _route_sort_quant(fn, fmt, x, w, topk, block, ws, bias, out, want_logits, stream):
    _bf16_2d(x, "x"), _bf16_2d(w, "w")
    m, k = x.shape
    n = w.shape[0]
    if out is None:
        out = alloc_sort_outputs(m, n, k, topk, block, x.device, fmt=fmt)
        out["topk_ids"] = torch.empty((m, topk), dtype=torch.int32, device=x.device)
        out["topk_w"] = torch.empty((m, topk), dtype=torch.float32, device=x.device)
        out["logits"] = torch.empty((m, n), dtype=torch.float32, device=x.device) if want_logits else None
    args = [_ptr(x), x.stride(0), _ptr(w), w.stride(0), _ptr(bias), m, n, k, topk, block,
            _ptr(out.get("logits")), _ptr(out["topk_ids"]), _ptr(out["topk_w"]),
            _ptr(out["sorted_ids"]), _ptr(out["expert_ids"]), _ptr(out["offsets"]),
            _ptr(out["a_q"]), _ptr(out["a_scale"])]
    if ws is not None:
        args += [_ptr(ws.buf), ws.nbytes]
    _check(fn(*args, _stream(stream)), fn.__name__[4:])
    return out


def moe_stage1_swiglu(sort_out, m: int, n: int, topk: int, block: int, w_q, w_scale, h=None, stream=None):
    """Stage-1 GEMM of the routed experts on the sorted MXFP8 rows of
    sort_out (a dict with a_q, a_scale, sorted_ids, expert_ids, offsets, as
    moe_sort_quant / route_sort_quant fill it): h bf16 [cap][I] with
    h[p] = silu(a . W_e[:I]) * (a . W_e[I:]) for the pair rows p. w_q uint8
    [N][2I][K/2] (e2m1 codes, low nibble first), w_scale uint8 [N][2I][K/32]."""
    a_q = sort_out["a_q"]
    k = a_q.shape[1]
    if w_q.dtype != torch.uint8 or w_q.dim() != 3 or not w_q.is_contiguous() or w_q.shape[2] * 2 != k:
        raise ValueError("w_q must be a contiguous uint8 [N][2I][K/2] tensor")
    inter = w_q.shape[1] // 2
    if w_scale.dtype != torch.uint8 or tuple(w_scale.shape) != (w_q.shape[0], 2 * inter, k // 32) or \
            not w_scale.is_contiguous():
        raise ValueError("w_scale must be a contiguous uint8 [N][2I][K/32] tensor")
    if h is None:
        h = torch.zeros((a_q.shape[0], inter), dtype=torch.bfloat16, device=a_q.device)
    _check(lib().rgt_moe_stage1_swiglu(_ptr(a_q), _ptr(sort_out["a_scale"]), _ptr(sort_out["sorted_ids"]),
                                       _ptr(sort_out["expert_ids"]), _ptr(sort_out["offsets"]), m, n, k, topk, block,
                                       _ptr(w_q), _ptr(w_scale), inter, _ptr(h), h.stride(0), _stream(stream)),
           "moe_stage1_swiglu")
    return h


def rmsnorm(x, gamma, eps: float, residual=None, xn=None, residual_out=None, rstd=None, stream=None):
    """Gemma RMSNorm producer: (xn bf16 [M][K], rstd fp32 [M], residual_out or
    None). residual_out (bf16, h = x + residual) is allocated when a residual
    is given and none is passed."""
    _bf16_2d(x, "x")
    m, k = x.shape
    if gamma.dtype != torch.bfloat16 or gamma.dim() != 1 or not gamma.is_contiguous():
        raise ValueError("gamma must be a contiguous 1-D bfloat16 tensor")
    if residual is not None:
        _bf16_2d(residual, "residual")
        if residual_out is None:
            residual_out = torch.empty((m, k), dtype=torch.bfloat16, device=x.device)
    if xn is None:
        xn = torch.empty((m, k), dtype=torch.bfloat16, device=x.device)
    if rstd is None:
        rstd = torch.empty((m,), dtype=torch.float32, device=x.device)
    _check(lib().rgt_rmsnorm(_ptr(x), x.stride(0), _ptr(residual), 0 if residual is None else residual.stride(0),
                             _ptr(gamma), float(eps), m, k, _ptr(xn), xn.stride(0), _ptr(residual_out),
                             0 if residual_out is None else residual_out.stride(0), _ptr(rstd), _stream(stream)),
           "rmsnorm")
    return xn, rstd, residual_out


def rmsnorm_route_sort_quant(x, gamma, eps: float, w, topk: int, block: int, ws: Workspace, residual=None,
                             bias=None, out=None, want_logits=True, fmt: str = "mxfp8", stream=None):
    """The front end behind its RMSNorm producer (one launch for M <= 64 and
    K <= 8192): x and residual are the raw inputs; returns the route dict of
    route_sort_quant plus xn, rstd and residual_out (h, with a residual)."""
    _bf16_2d(x, "x"), _bf16_2d(w, "w")
    m, k = x.shape
    n = w.shape[0]
    if gamma.dtype != torch.bfloat16 or gamma.dim() != 1 or not gamma.is_contiguous():
        raise ValueError("gamma must be a contiguous 1-D bfloat16 tensor")
    if residual is not None:
        _bf16_2d(residual, "residual")
    if fmt not in ("mxfp8", "mxfp4"):
        raise ValueError("fmt must be 'mxfp8' or 'mxfp4'")
    if out is None:
        out = alloc_sort_outputs(m, n, k, topk, block, x.device, fmt=fmt)
        out["topk_ids"] = torch.empty((m, topk), dtype=torch.int32, device=x.device)
        out["topk_w"] = torch.empty((m, topk), dtype=torch.float32, device=x.device)
        out["logits"] = torch.empty((m, n), dtype=torch.float32, device=x.device) if want_logits else None
        out["xn"] = torch.empty((m, k), dtype=torch.bfloat16, device=x.device)
        out["rstd"] = torch.empty((m,), dtype=torch.float32, device=x.device)
        out["residual_out"] = None if residual is None else torch.empty((m, k), dtype=torch.bfloat16,
                                                                        device=x.device)
    ro = out.get("residual_out")
    fn = lib().rgt_rmsnorm_route_sort_quant if fmt == "mxfp8" else lib().rgt_rmsnorm_route_sort_quant_mxfp4
    _check(fn(_ptr(x), x.stride(0), _ptr(residual), 0 if residual is None else residual.stride(0), _ptr(gamma),
              float(eps), _ptr(w), w.stride(0), _ptr(bias), m, n, k, topk, block, _ptr(out["xn"]), out["xn"].stride(0),
              _ptr(ro), 0 if ro is None else ro.stride(0), _ptr(out.get("rstd")), _ptr(out.get("logits")),
              _ptr(out["topk_ids"]), _ptr(out["topk_w"]), _ptr(out["sorted_ids"]), _ptr(out["expert_ids"]),
              _ptr(out["offsets"]), _ptr(out["a_q"]), _ptr(out["a_scale"]), _ptr(ws.buf), ws.nbytes,
              _stream(stream)), fn.__name__[4:])
    return out


def reload_env():
    """Re-read the RGT_* environment settings (the library reads them at its
    first call and here only)."""
    lib().rgt_reload_env()


def diag_read(src, sink, grid: int, nbytes: int | None = None, stream=None):
    """Stream-read `nbytes` of `src` (default: all of it) in one launch."""
    nbytes = src.numel() * src.element_size() if nbytes is None else nbytes
    _check(lib().rgt_diag_read(_ptr(src), nbytes, _ptr(sink), grid, _stream(stream)), "diag_read")


def diag_copy(src, dst, grid: int, nbytes: int | None = None, stream=None):
    """Copy `nbytes` of `src` to `dst` in one launch."""
    nbytes = src.numel() * src.element_size() if nbytes is None else nbytes
    _check(lib().rgt_diag_copy(_ptr(src), _ptr(dst), nbytes, grid, _stream(stream)), "diag_copy")
