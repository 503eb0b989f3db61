"""MI355X-native IndexCache / DeepSeek-Sparse-Attention hot path.

Thin Python binding over libdsa_indexcache.so (C ABI in include/dsa_indexcache.h):
argument marshalling only - every step runs in the gfx950 HIP kernels.  Tensors
must be contiguous device tensors; work is enqueued on torch's current stream.

    indexer_scores(q, w, k, ctx_len, q_scale=None, k_scale=None) -> scores [B,T,Lmax]
    topk(scores, ctx_len, k)                                     -> idx [B,T,k] int32
    indexer_topk(q, w, k, ctx_len, k_sel, q_scale, k_scale)      -> idx (decode; no scores)
    sparse_attn(q, kv, idx, ctx_len, scale)                      -> (out, lse)
    kv_append(ctx_len, kv_new, kv_cache, k_new, k_cache, k_scale) -> None (caches in place)
    run_stack(pattern, layers, ...)                              -> stats dict
    reuse_costs(layers, ctx_len, proxy, ...)                     -> cost [n,n] fp64 (device)
    pattern_cost(cost, pattern) / greedy_search(cost, n_shared)  -> host-side search
"""
from __future__ import annotations

import ctypes
from typing import Dict, List, Optional, Sequence

from . import _lib
from ._lib import DSAError, Layer, StackShape, StackStats  # noqa: F401

__all__ = ["probe_stream_read", "indexer_scores", "topk", "topk_workspace_size", "indexer_topk",
           "indexer_topk_workspace_size", "sparse_attn",
           "sparse_attn_workspace_size", "kv_append", "run_stack",
           "reuse_costs", "reuse_costs_workspace_size", "pattern_cost", "greedy_search",
           "Stack", "DSAError", "library", "ld_for"]


def library():
    return _lib.load()


def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream=None) -> int:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _need(t, name, dtypes, ndim=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise TypeError(f"{name} must be contiguous")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if ndim is not None and t.dim() != ndim:
        raise TypeError(f"{name} must have {ndim} dims, got {t.dim()}")


def _shape(t, name, shape):
    if tuple(t.shape) != tuple(shape):
        raise TypeError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _same_device(ref, *named):
    for name, t in named:
        if t is not None and t.device != ref.device:
            raise TypeError(f"{name} is on {t.device}, expected {ref.device}")


def _ctx(ctx_len, B):
    _need(ctx_len, "ctx_len", (_torch().int32,), 1)
    if ctx_len.shape[0] != B:
        raise TypeError(f"ctx_len has {ctx_len.shape[0]} entries, expected B = {B}")


def _workspace(ws, need: int, device, zero: bool):
    """The caller's workspace (checked: contiguous uint8 on `device`; its real
    size goes to the C ABI, which rejects one that is too small), or a fresh
    one of `need` bytes."""
    torch = _torch()
    if ws is None:
        alloc = torch.zeros if zero else torch.empty
        return alloc(max(need, 1), dtype=torch.uint8, device=device)
    _need(ws, "workspace", (torch.uint8,))
    if ws.device != torch.device(device):
        raise TypeError(f"workspace is on {ws.device}, expected {device}")
    return ws


def _indexer_inputs(q, w, k, ctx_len, q_scale, k_scale):
    """Shapes of the indexer operands: q [B,T,H,D], w [B,T,H] fp32, k
    [B,Lmax,D] of q's dtype, and for fp8 q_scale [B,T,H] and k_scale [B,Lmax]
    fp32; ctx_len [B] int32."""
    torch = _torch()
    _need(q, "q", (torch.bfloat16, torch.float8_e4m3fn), 4)
    _need(k, "k", (q.dtype,), 3)
    _need(w, "w", (torch.float32,), 3)
    B, T, H, D = q.shape
    Lmax = k.shape[1]
    _shape(k, "k", (B, Lmax, D))
    _shape(w, "w", (B, T, H))
    _ctx(ctx_len, B)
    if q.dtype == torch.float8_e4m3fn:
        if q_scale is None or k_scale is None:
            raise TypeError("fp8 indexer inputs need q_scale and k_scale")
        _need(q_scale, "q_scale", (torch.float32,), 3)
        _need(k_scale, "k_scale", (torch.float32,), 2)
        _shape(q_scale, "q_scale", (B, T, H))
        _shape(k_scale, "k_scale", (B, Lmax))
    elif q_scale is not None or k_scale is not None:
        raise TypeError("bf16 indexer inputs take no scales")
    _same_device(q, ("w", w), ("k", k), ("ctx_len", ctx_len), ("q_scale", q_scale),
                 ("k_scale", k_scale))
    return B, T, H, D, Lmax


def ld_for(Lmax: int) -> int:
    return (Lmax + 3) // 4 * 4


def _idx_dtype(q):
    torch = _torch()
    if q.dtype == torch.bfloat16:
        return _lib.DSA_BF16
    if q.dtype == torch.float8_e4m3fn:
        return _lib.DSA_FP8_E4M3
    raise TypeError(f"indexer inputs must be bf16 or float8_e4m3fn, got {q.dtype}")


def indexer_scores(q, w, k, ctx_len, q_scale=None, k_scale=None, out=None, stream=None):
    """Lightning-indexer scores [B,T,Lmax] fp32 (a view of a [B,T,ld] buffer)."""
    torch = _torch()
    B, T, H, D, Lmax = _indexer_inputs(q, w, k, ctx_len, q_scale, k_scale)
    ld = ld_for(Lmax)
    if out is None:
        out = torch.empty((B, T, ld), dtype=torch.float32, device=q.device)
    _need(out, "out", (torch.float32,), 3)
    if out.shape[0] != B or out.shape[1] != T or out.shape[2] < Lmax or out.shape[2] % 4:
        raise TypeError(f"out has shape {tuple(out.shape)}, expected ({B}, {T}, ld) with "
                        f"ld >= {Lmax} a multiple of 4")
    _same_device(q, ("out", out))
    lib = library()
    _lib.check(lib.dsa_indexer_scores(_ptr(q), _idx_dtype(q), _ptr(q_scale), _ptr(w), _ptr(k),
                                      _ptr(k_scale), _ptr(ctx_len), B, T, H, D, Lmax,
                                      _ptr(out), out.shape[-1], _stream(stream)))
    return out[..., :Lmax]


def topk(scores, ctx_len, k: int, out=None, workspace=None, stream=None):
    """Per-row top-k positions, ascending, -1 padded: [B,T,k] int32.

    `scores` may be the [B,T,Lmax] view returned by indexer_scores (its row
    stride is then the padded buffer's).  A reused `workspace` (uint8 device
    tensor of topk_workspace_size bytes) must start zero-filled; calls leave
    it zero-filled."""
    torch = _torch()
    if scores.dim() != 3 or scores.dtype != torch.float32 or not scores.is_cuda:
        raise TypeError("scores must be a [B,T,L] float32 device tensor")
    if scores.stride(2) != 1 or scores.stride(0) != scores.shape[1] * scores.stride(1):
        raise TypeError("scores rows must be contiguous with a uniform row stride")
    B, T, Lmax = scores.shape
    _ctx(ctx_len, B)
    ld = scores.stride(1)
    if out is None:
        out = torch.empty((B, T, k), dtype=torch.int32, device=scores.device)
    _need(out, "out", (torch.int32,), 3)
    _shape(out, "out", (B, T, k))
    _same_device(scores, ("ctx_len", ctx_len), ("out", out))
    lib = library()
    need = ctypes.c_size_t(0)
    _lib.check(lib.dsa_topk_workspace_size(B, T, Lmax, k, ctypes.byref(need)))
    ws = _workspace(workspace, need.value, scores.device, zero=True)
    _lib.check(lib.dsa_topk(_ptr(scores), ld, _ptr(ctx_len), B, T, Lmax, k, _ptr(out),
                            _ptr(ws), ws.numel(), _stream(stream)))
    return out


def indexer_topk_workspace_size(B: int, T: int, H: int, D: int, Lmax: int, k: int,
                                idx_dtype: str = "bf16") -> int:
    """Workspace bytes of indexer_topk; raises DSAError for shapes it does not take."""
    need = ctypes.c_size_t(0)
    dt = _lib.DSA_FP8_E4M3 if idx_dtype == "fp8" else _lib.DSA_BF16
    _lib.check(library().dsa_indexer_topk_workspace_size(B, T, H, D, dt, Lmax, k,
                                                         ctypes.byref(need)))
    return need.value


def indexer_topk(q, w, k_cache, ctx_len, k: int, q_scale=None, k_scale=None, out=None,
                 workspace=None, stream=None):
    """Indexer scores and top-k in one pass: [B,T,k] int32.

    The same set as topk(indexer_scores(q, w, k_cache, ...), ctx_len, k), with
    the scores kept on chip.  A reused `workspace` (uint8 device tensor of
    indexer_topk_workspace_size bytes) must start zero-filled; calls leave the
    part that must start at zero as they found it."""
    torch = _torch()
    B, T, H, D, Lmax = _indexer_inputs(q, w, k_cache, ctx_len, q_scale, k_scale)
    if out is None:
        out = torch.empty((B, T, k), dtype=torch.int32, device=q.device)
    _need(out, "out", (torch.int32,), 3)
    _shape(out, "out", (B, T, k))
    _same_device(q, ("out", out))
    lib = library()
    dt = _idx_dtype(q)
    need = ctypes.c_size_t(0)
    _lib.check(lib.dsa_indexer_topk_workspace_size(B, T, H, D, dt, Lmax, k, ctypes.byref(need)))
    ws = _workspace(workspace, need.value, q.device, zero=True)
    _lib.check(lib.dsa_indexer_topk(_ptr(q), dt, _ptr(q_scale), _ptr(w), _ptr(k_cache),
                                    _ptr(k_scale), _ptr(ctx_len), B, T, H, D, Lmax, k, _ptr(out),
                                    _ptr(ws), ws.numel(), _stream(stream)))
    return out


def topk_workspace_size(B: int, T: int, Lmax: int, k: int) -> int:
    need = ctypes.c_size_t(0)
    _lib.check(library().dsa_topk_workspace_size(B, T, Lmax, k, ctypes.byref(need)))
    return need.value


def sparse_attn_workspace_size(B: int, T: int, Hq: int, k: int) -> int:
    need = ctypes.c_size_t(0)
    _lib.check(library().dsa_sparse_attn_workspace_size(B, T, Hq, k, 512, ctypes.byref(need)))
    return need.value


def sparse_attn(q, kv, idx, ctx_len, scale: float, out=None, lse=None, want_lse=True,
                workspace=None, stream=None):
    """Sparse MLA attention: (out [B,T,Hq,512] bf16, lse [B,T,Hq] fp32 or None).

    `workspace`: optional uint8 device tensor of sparse_attn_workspace_size bytes."""
    torch = _torch()
    _need(q, "q", (torch.bfloat16,), 4)
    _need(kv, "kv", (torch.bfloat16,), 3)
    _need(idx, "idx", (torch.int32,), 3)
    B, T, Hq, d_qk = q.shape
    Lmax = kv.shape[1]
    k = idx.shape[2]
    d_v = 512
    _shape(kv, "kv", (B, Lmax, d_qk))
    _shape(idx, "idx", (B, T, k))
    _ctx(ctx_len, B)
    if out is None:
        out = torch.empty((B, T, Hq, d_v), dtype=torch.bfloat16, device=q.device)
    _need(out, "out", (torch.bfloat16,), 4)
    _shape(out, "out", (B, T, Hq, d_v))
    if lse is None and want_lse:
        lse = torch.empty((B, T, Hq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", (torch.float32,), 3)
        _shape(lse, "lse", (B, T, Hq))
    _same_device(q, ("kv", kv), ("idx", idx), ("ctx_len", ctx_len), ("out", out), ("lse", lse))
    lib = library()
    need = ctypes.c_size_t(0)
    _lib.check(lib.dsa_sparse_attn_workspace_size(B, T, Hq, k, d_v, ctypes.byref(need)))
    ws = _workspace(workspace, need.value, q.device, zero=False)
    _lib.check(lib.dsa_sparse_attn(_ptr(q), _ptr(kv), _ptr(idx), _ptr(ctx_len), B, T, Hq, Lmax,
                                   k, d_qk, d_v, float(scale), _ptr(out), _ptr(lse), _ptr(ws),
                                   ws.numel(), _stream(stream)))
    return out, lse


def kv_append(ctx_len, kv_new=None, kv_cache=None, k_new=None, k_cache=None, k_scale=None,
              stream=None) -> None:
    """Write T new token rows per sequence into the caches, in place.

    kv_new [B,T,d_qk] fp32 -> kv_cache [B,Lmax,d_qk] bf16; k_new [B,T,D] fp32 ->
    k_cache [B,Lmax,D] bf16, or float8_e4m3fn with k_scale [B,Lmax] fp32.  Row t
    of sequence b lands at position ctx_len[b] - T + t.  Either pair may be
    omitted."""
    torch = _torch()
    _need(ctx_len, "ctx_len", (torch.int32,), 1)
    B = T = Lmax = None
    d_qk = D = 0
    dt = _lib.DSA_BF16
    if kv_new is not None or kv_cache is not None:
        _need(kv_new, "kv_new", (torch.float32,), 3)
        _need(kv_cache, "kv_cache", (torch.bfloat16,), 3)
        B, T, d_qk = kv_new.shape
        Lmax = kv_cache.shape[1]
        if kv_cache.shape[0] != B or kv_cache.shape[2] != d_qk:
            raise TypeError("kv_cache must be [B, Lmax, d_qk] matching kv_new")
    if k_new is not None or k_cache is not None:
        _need(k_new, "k_new", (torch.float32,), 3)
        _need(k_cache, "k_cache", (torch.bfloat16, torch.float8_e4m3fn), 3)
        Bk, Tk, D = k_new.shape
        if B is not None and (Bk, Tk, k_cache.shape[1]) != (B, T, Lmax):
            raise TypeError("k_new / k_cache disagree with kv_new / kv_cache on B, T or Lmax")
        B, T, Lmax = Bk, Tk, k_cache.shape[1]
        if k_cache.shape[0] != B or k_cache.shape[2] != D:
            raise TypeError("k_cache must be [B, Lmax, D] matching k_new")
        dt = _idx_dtype(k_cache)
        if dt == _lib.DSA_FP8_E4M3:
            _need(k_scale, "k_scale", (torch.float32,), 2)
            if tuple(k_scale.shape) != (B, Lmax):
                raise TypeError("k_scale must be [B, Lmax]")
    if B is None:
        raise TypeError("kv_append needs kv_new/kv_cache, k_new/k_cache or both")
    if ctx_len.shape[0] != B:
        raise TypeError("ctx_len must have B entries")
    _lib.check(library().dsa_kv_append(_ptr(kv_new), _ptr(k_new), _ptr(ctx_len), B, T, Lmax,
                                       d_qk, D, dt, _ptr(kv_cache), _ptr(k_cache), _ptr(k_scale),
                                       _stream(stream)))



def probe_stream_read(src, sink, workgroups: int = 256, form: str = "tiles", stream=None):
    """Read every byte of the contiguous device tensor `src` once (a streaming-read
    ceiling for the decode indexer's key sweep; no step of the method).

    form "tiles": the indexer's load pattern, `workgroups` workgroups each sweeping
    a contiguous run of 8 KB tiles; "stride": a grid-stride sweep. `sink` is a
    device int32 tensor the kernel almost never writes. src.nbytes must be a
    multiple of 8192."""
    if not src.is_cuda or not src.is_contiguous():
        raise TypeError("src must be a contiguous device tensor")
    _need(sink, "sink", (_torch().int32,))
    if sink.numel() < 1:
        raise TypeError("sink must hold at least one int32")
    _same_device(src, ("sink", sink))
    forms = {"tiles": _lib.DSA_PROBE_TILES, "stride": _lib.DSA_PROBE_STRIDE}
    if form not in forms:
        raise ValueError(f"form must be one of {sorted(forms)}")
    nbytes = src.numel() * src.element_size()
    _lib.check(library().dsa_probe_stream_read(_ptr(src), nbytes, workgroups, forms[form],
                                               _ptr(sink), _stream(stream)))

def _layer_array(layers):
    arr = (Layer * len(layers))()
    for i, L in enumerate(layers):
        arr[i] = Layer(_ptr(L.get("q_idx")), _ptr(L.get("q_idx_scale")), _ptr(L.get("w")),
                       _ptr(L.get("k_idx")), _ptr(L.get("k_idx_scale")), _ptr(L.get("q")),
                       _ptr(L.get("kv")), _ptr(L.get("out")), _ptr(L.get("lse")))
    return arr


def _check_layers(layers, indexer_layers, ctx_len, *, B, T, H, D, Lmax, Hq, idx_dtype,
                  d_qk=576, d_v=512):
    """Every tensor a layer entry hands to the C ABI has the stack's shape,
    dtype and device (the ABI sees only pointers): indexer operands on the
    layers in `indexer_layers`, attention operands on every layer when Hq > 0."""
    torch = _torch()
    _ctx(ctx_len, B)
    kdt = torch.float8_e4m3fn if idx_dtype == "fp8" else torch.bfloat16
    for l, L in enumerate(layers):
        if l in indexer_layers:
            q_idx, k_idx = L.get("q_idx"), L.get("k_idx")
            _need(q_idx, f"layer {l} q_idx", (kdt,), 4)
            _shape(q_idx, f"layer {l} q_idx", (B, T, H, D))
            got = _indexer_inputs(q_idx, L.get("w"), k_idx, ctx_len, L.get("q_idx_scale"),
                                  L.get("k_idx_scale"))
            if got[4] != Lmax:
                raise TypeError(f"layer {l} k_idx holds {got[4]} rows, expected Lmax = {Lmax}")
        if Hq > 0:
            q, kv, out, lse = L.get("q"), L.get("kv"), L.get("out"), L.get("lse")
            for name, t, dt, shp in (("q", q, torch.bfloat16, (B, T, Hq, d_qk)),
                                     ("kv", kv, torch.bfloat16, (B, Lmax, d_qk)),
                                     ("out", out, torch.bfloat16, (B, T, Hq, d_v))):
                _need(t, f"layer {l} {name}", (dt,), len(shp))
                _shape(t, f"layer {l} {name}", shp)
                _same_device(ctx_len, (f"layer {l} {name}", t))
            if lse is not None:
                _need(lse, f"layer {l} lse", (torch.float32,), 3)
                _shape(lse, f"layer {l} lse", (B, T, Hq))
                _same_device(ctx_len, (f"layer {l} lse", lse))


_PROXIES = {"output": _lib.DSA_PROXY_OUTPUT, "miss": _lib.DSA_PROXY_MISS}


def reuse_costs_workspace_size(n_layers: int, *, B, T, H, D, Lmax, k, Hq=0, idx_dtype="bf16",
                               scale=1.0, proxy="output", d_qk=576, d_v=512) -> int:
    dt = _lib.DSA_FP8_E4M3 if idx_dtype == "fp8" else _lib.DSA_BF16
    shape = StackShape(B, T, H, D, Lmax, k, Hq, d_qk, d_v, dt, float(scale))
    need = ctypes.c_size_t(0)
    _lib.check(library().indexcache_reuse_costs_workspace_size(
        ctypes.byref(shape), n_layers, _PROXIES[proxy], ctypes.byref(need)))
    return need.value


def reuse_costs(layers: Sequence[Dict], ctx_len, *, B, T, H, D, Lmax, k, Hq=0,
                idx_dtype="bf16", scale=1.0, proxy="output", d_qk=576, d_v=512, workspace=None,
                stream=None):
    """Proxy cost matrix [n, n] fp64 (device) of the training-free pattern
    search: entry (l, j), j < l, is what layer l loses with layer j's index
    set.  With proxy "output" every layer's `out` receives its all-F output.
    `workspace`: optional zero-filled uint8 device tensor, reusable."""
    torch = _torch()
    if proxy not in _PROXIES:
        raise ValueError(f"proxy must be one of {sorted(_PROXIES)}")
    n = len(layers)
    dt = _lib.DSA_FP8_E4M3 if idx_dtype == "fp8" else _lib.DSA_BF16
    shape = StackShape(B, T, H, D, Lmax, k, Hq, d_qk, d_v, dt, float(scale))
    dev = ctx_len.device
    _check_layers(layers, set(range(n)), ctx_len, B=B, T=T, H=H, D=D, Lmax=Lmax,
                  Hq=Hq if proxy == "output" else 0, idx_dtype=idx_dtype, d_qk=d_qk, d_v=d_v)
    need = ctypes.c_size_t(0)
    lib = library()
    _lib.check(lib.indexcache_reuse_costs_workspace_size(ctypes.byref(shape), n, _PROXIES[proxy],
                                                         ctypes.byref(need)))
    ws = _workspace(workspace, need.value, dev, zero=True)
    ld = ld_for(Lmax)
    score = torch.empty((B, T, ld), dtype=torch.float32, device=dev)
    cost = torch.empty((n, n), dtype=torch.float64, device=dev)
    arr = _layer_array(layers)
    _lib.check(lib.indexcache_reuse_costs(n, arr, ctypes.byref(shape), _ptr(ctx_len),
                                          _PROXIES[proxy], _ptr(cost), _ptr(score), ld, _ptr(ws),
                                          ws.numel(), _stream(stream)))
    return cost


def _host_cost(cost):
    import numpy as np
    c = cost.detach().cpu().numpy() if hasattr(cost, "detach") else np.asarray(cost)
    c = np.ascontiguousarray(c, dtype=np.float64)
    if c.ndim != 2 or c.shape[0] != c.shape[1]:
        raise TypeError("cost must be a square [n, n] matrix")
    return c


def pattern_cost(cost, pattern: str) -> float:
    """Proxy loss of one pattern under a cost matrix (host computation)."""
    c = _host_cost(cost)
    out = ctypes.c_double(0.0)
    _lib.check(library().indexcache_pattern_cost(c.ctypes.data, c.shape[0], pattern.encode(),
                                                 ctypes.byref(out)))
    return out.value


def greedy_search(cost, n_shared: int):
    """Greedy F -> S conversion: [(pattern, cost)] after each of n_shared steps."""
    c = _host_cost(cost)
    n = c.shape[0]
    pats = ctypes.create_string_buffer(max(1, n_shared * (n + 1)))
    totals = (ctypes.c_double * max(1, n_shared))()
    _lib.check(library().indexcache_greedy_search(c.ctypes.data, n, n_shared,
                                                  ctypes.addressof(pats), ctypes.addressof(totals)))
    raw = pats.raw
    return [(raw[m * (n + 1): m * (n + 1) + n].decode(), totals[m]) for m in range(n_shared)]


class Stack:
    """Pre-marshalled arguments of indexcache_run_stack for repeated calls."""

    def __init__(self, pattern: str, layers: Sequence[Dict], ctx_len, *, B, T, H, D, Lmax, k,
                 Hq=0, idx_dtype="bf16", scale=1.0, d_qk=576, d_v=512, device=None,
                 fused_topk=True):
        """fused_topk: F layers run indexer_topk (scores kept on chip) where
        it takes the shape; False: scores through score_buf, then topk."""
        torch = _torch()
        self.pattern = pattern.encode()
        self.n_layers = len(layers)
        self._keep = [layers, ctx_len]
        _check_layers(layers, {l for l, c in enumerate(pattern) if c == "F"}, ctx_len, B=B, T=T,
                      H=H, D=D, Lmax=Lmax, Hq=Hq, idx_dtype=idx_dtype, d_qk=d_qk, d_v=d_v)
        self.layers = _layer_array(layers)
        dt = _lib.DSA_FP8_E4M3 if idx_dtype == "fp8" else _lib.DSA_BF16
        flags = 0 if fused_topk else _lib.DSA_STACK_UNFUSED_TOPK
        self.shape = StackShape(B, T, H, D, Lmax, k, Hq, d_qk, d_v, dt, float(scale), flags)
        self.ctx_len = ctx_len
        dev = device if device is not None else ctx_len.device
        self.ld = ld_for(Lmax)
        self.idx_buf = torch.empty((B, T, k), dtype=torch.int32, device=dev)
        fz = ctypes.c_int(0)
        _lib.check(library().indexcache_stack_fuses_topk(ctypes.byref(self.shape),
                                                         ctypes.byref(fz)))
        self.fused = bool(fz.value)
        # the fused path never writes scores, so it needs no score buffer
        self.score_buf = None if self.fused else torch.empty((B, T, self.ld),
                                                             dtype=torch.float32, device=dev)
        need = ctypes.c_size_t(0)
        _lib.check(library().indexcache_stack_workspace_size(ctypes.byref(self.shape),
                                                             ctypes.byref(need)))
        self.ws_bytes = need.value
        self.ws = torch.zeros(max(need.value, 1), dtype=torch.uint8, device=dev)
        self.stats = StackStats()

    def run(self, stream=None) -> Dict[str, int]:
        _lib.check(library().indexcache_run_stack(
            self.pattern, self.n_layers, self.layers, ctypes.byref(self.shape),
            _ptr(self.ctx_len), _ptr(self.idx_buf), _ptr(self.score_buf), self.ld, _ptr(self.ws),
            self.ws_bytes, ctypes.byref(self.stats), _stream(stream)))
        return dict(n_indexer_calls=self.stats.n_indexer_calls,
                    n_topk_calls=self.stats.n_topk_calls, n_attn_calls=self.stats.n_attn_calls)


    def run_noalloc(self, stream=None) -> Dict[str, int]:
        """The same call through indexcache_run_stack_noalloc: the library's
        static scratch instead of this object's workspace (shapes up to
        DSA_NOALLOC_SCRATCH_BYTES of workspace)."""
        _lib.check(library().indexcache_run_stack_noalloc(
            self.pattern, self.n_layers, self.layers, ctypes.byref(self.shape),
            _ptr(self.ctx_len), _ptr(self.idx_buf), _ptr(self.score_buf), self.ld,
            ctypes.byref(self.stats), _stream(stream)))
        return dict(n_indexer_calls=self.stats.n_indexer_calls,
                    n_topk_calls=self.stats.n_topk_calls, n_attn_calls=self.stats.n_attn_calls)


def run_stack(pattern: str, layers: List[Dict], ctx_len, **shape) -> Dict:
    """One pass of the IndexCache layer loop; returns stats plus idx_buf."""
    st = Stack(pattern, layers, ctx_len, **shape)
    stats = st.run()
    stats["idx_buf"] = st.idx_buf
    return stats
