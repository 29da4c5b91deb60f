"""MI355X-native SparsePR attention call (gfx950 HIP kernels behind a C ABI).

The functions here carry the names of the C entry points declared in
``include/sparsepr.h`` and only marshal torch tensors (device memory and the
current stream) into the library.  Inputs are [B, H, N, d] bf16 or fp32 CUDA
(ROCm) tensors whose last dimension is contiguous.
"""

from __future__ import annotations

import ctypes
from typing import Optional

from ._lib import (  # noqa: F401
    PART_INDEPENDENT,
    PART_RESPONSE_COUPLED,
    ROUTER_ALPHA,
    ROUTER_BUDGET,
    SPARSEPR_BF16,
    SPARSEPR_FP32,
    SparsePRError,
    SparseprConfig,
    SparseprHeadStats,
    SparseprTensors,
    check,
    lib,
)

__all__ = [
    "sparsepr_config_default", "sparsepr_workspace_size", "sparsepr_validate", "sparsepr_attention",
    "sparsepr_attention_with_partition", "sparsepr_key_metric", "sparsepr_partition", "sparsepr_route",
    "sparsepr_sparse_attention", "sparsepr_probe_fit", "sparsepr_dense_attention", "make_config",
    "stats_to_dicts", "SparseprConfig", "SparsePRError", "sparsepr_attention_profile", "Workspace",
    "sparsepr_mfma_rounding_check", "sparsepr_attention_noalloc", "noalloc_scratch_bytes",
]


def _torch():
    import torch
    return torch


def sparsepr_config_default(n: int, d: int) -> SparseprConfig:
    cfg = SparseprConfig()
    check(lib().sparsepr_config_default(n, d, ctypes.byref(cfg)), "sparsepr_config_default")
    return cfg


def make_config(n: int, d: int, **kw) -> SparseprConfig:
    """Defaults for (N, d) with fields overridden by keyword."""
    cfg = sparsepr_config_default(n, d)
    for k, v in kw.items():
        if k == "partition_mode" and isinstance(v, str):
            v = {"response_coupled": PART_RESPONSE_COUPLED, "independent": PART_INDEPENDENT}[v]
        if k == "ridge_mode" and isinstance(v, str):
            v = {"relative": 0, "absolute": 1}[v]
        if k == "router" and isinstance(v, str):
            v = {"budget": ROUTER_BUDGET, "alpha": ROUTER_ALPHA}[v]
        if not hasattr(cfg, k):
            raise KeyError(k)
        setattr(cfg, k, v)
    return cfg


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return SPARSEPR_BF16
    if t.dtype == torch.float32:
        return SPARSEPR_FP32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _tensors(q, k, v, o) -> SparseprTensors:
    for t in (q, k, v, o):
        if t.dim() != 4 or not t.is_cuda:
            raise ValueError("q, k, v, o must be 4-D [B, H, N, d] device tensors")
        if t.dtype != q.dtype or t.shape != q.shape:
            raise ValueError("q, k, v, o must share dtype and shape")
    io = SparseprTensors()
    io.q, io.k, io.v, io.o = q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr()
    for name, t in (("q_strides", q), ("k_strides", k), ("v_strides", v), ("o_strides", o)):
        arr = getattr(io, name)
        for i, s in enumerate(t.stride()):
            arr[i] = s
    io.B, io.H, io.N, io.d = (int(x) for x in q.shape)
    io.dtype = _dtype_code(q)
    return io


def _stream(stream=None) -> int:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def sparsepr_validate(cfg: SparseprConfig, B: int, H: int, N: int, d: int, dtype: int) -> int:
    return lib().sparsepr_validate(ctypes.byref(cfg), B, H, N, d, dtype)


def sparsepr_workspace_size(cfg: SparseprConfig, B: int, H: int, N: int, d: int, dtype: int) -> int:
    n = ctypes.c_size_t(0)
    check(lib().sparsepr_workspace_size(ctypes.byref(cfg), B, H, N, d, dtype, ctypes.byref(n)),
          "sparsepr_workspace_size")
    return int(n.value)


class Workspace:
    """Reusable device workspaces, one per (device, stream).

    Calls that share a workspace must be ordered; keeping one buffer per
    stream means calls on different streams never share one.  A buffer is
    never released while the Workspace lives: when a call needs more, a larger
    buffer (at least twice the size) replaces it for later calls and the old
    one is kept, so a HIP graph captured with the old pointer stays valid.
    """

    def __init__(self):
        self.bufs = {}     # (device index, stream handle) -> current buffer
        self.retired = []  # superseded buffers, kept alive

    def get(self, nbytes: int, device, stream=None):
        torch = _torch()
        s = stream if stream is not None else torch.cuda.current_stream(device)
        key = (device.index if device.index is not None else torch.cuda.current_device(), s.cuda_stream)
        buf = self.bufs.get(key)
        if buf is None or buf.numel() < nbytes:
            if buf is not None:
                self.retired.append(buf)
                nbytes = max(nbytes, 2 * buf.numel())
            with torch.cuda.stream(s):
                buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
            self.bufs[key] = buf
        return buf


_default_ws = Workspace()


def _ws(cfg, q, workspace, stream=None):
    nbytes = sparsepr_workspace_size(cfg, *q.shape, _dtype_code(q))
    buf = (workspace or _default_ws).get(nbytes, q.device, stream)
    return buf, nbytes


def _on_stream(stream, *tensors) -> None:
    """Tell the caching allocator that a call on an explicit stream uses these
    tensors, so their memory is not reused before that stream's work ends."""
    if stream is None:
        return
    for t in tensors:
        if t is not None:
            t.record_stream(stream)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def stats_to_dicts(stats_tensor) -> list:
    raw = stats_tensor.cpu().numpy().tobytes()
    n = len(raw) // ctypes.sizeof(SparseprHeadStats)
    arr = (SparseprHeadStats * n).from_buffer_copy(raw)
    out = []
    for s in arr:
        d = {k: getattr(s, k) for k, _ in SparseprHeadStats._fields_ if k != "sigma"}
        d["sigma"] = list(s.sigma)
        out.append(d)
    return out


def _stats_buf(q):
    torch = _torch()
    n = q.shape[0] * q.shape[1] * ctypes.sizeof(SparseprHeadStats)
    return torch.empty(n, dtype=torch.uint8, device=q.device)


def sparsepr_attention(q, k, v, cfg: SparseprConfig, out=None, workspace: Optional[Workspace] = None,
                       stream=None, with_stats: bool = False):
    """Corrected SparsePR attention output (original token order)."""
    torch = _torch()
    out = torch.empty_like(q) if out is None else out
    io = _tensors(q, k, v, out)
    buf, nbytes = _ws(cfg, q, workspace, stream)
    st = _stats_buf(q) if with_stats else None
    check(lib().sparsepr_attention(ctypes.byref(cfg), ctypes.byref(io), buf.data_ptr(), nbytes,
                                   _stream(stream), _ptr(st)), "sparsepr_attention")
    _on_stream(stream, out, st)
    return (out, st) if with_stats else out


def sparsepr_attention_noalloc(q, k, v, cfg: SparseprConfig, out=None, stream=None, with_stats: bool = False):
    """The full call in the library's fixed per-GPU scratch (no workspace, no
    allocation by the library; `out` and the stats buffer are the caller's)."""
    torch = _torch()
    out = torch.empty_like(q) if out is None else out
    io = _tensors(q, k, v, out)
    st = _stats_buf(q) if with_stats else None
    check(lib().sparsepr_attention_noalloc(ctypes.byref(cfg), ctypes.byref(io), _stream(stream), _ptr(st)),
          "sparsepr_attention_noalloc")
    _on_stream(stream, out, st)
    return (out, st) if with_stats else out


def noalloc_scratch_bytes() -> int:
    return int(lib().sparsepr_noalloc_scratch_bytes())


def sparsepr_attention_profile(q, k, v, cfg, out=None, workspace: Optional[Workspace] = None, stream=None):
    """Run one call with per-stage HIP events; returns (out, {stage: ms}, stats tensor)."""
    from ._lib import STAGES
    torch = _torch()
    out = torch.empty_like(q) if out is None else out
    io = _tensors(q, k, v, out)
    buf, nbytes = _ws(cfg, q, workspace, stream)
    st = _stats_buf(q)
    ms = (ctypes.c_float * len(STAGES))()
    check(lib().sparsepr_attention_profile(ctypes.byref(cfg), ctypes.byref(io), buf.data_ptr(), nbytes,
                                           _stream(stream), st.data_ptr(), ms), "sparsepr_attention_profile")
    _on_stream(stream, out, st)
    return out, dict(zip(STAGES, list(ms))), st


def sparsepr_attention_with_partition(q, k, v, cfg, q_labels, kv_labels, out=None, workspace=None,
                                      stream=None, with_stats: bool = False):
    torch = _torch()
    out = torch.empty_like(q) if out is None else out
    io = _tensors(q, k, v, out)
    buf, nbytes = _ws(cfg, q, workspace, stream)
    st = _stats_buf(q) if with_stats else None
    ql = q_labels.to(torch.int32).contiguous()
    kl = kv_labels.to(torch.int32).contiguous()
    check(lib().sparsepr_attention_with_partition(ctypes.byref(cfg), ctypes.byref(io), ql.data_ptr(),
                                                  kl.data_ptr(), buf.data_ptr(), nbytes, _stream(stream),
                                                  _ptr(st)), "sparsepr_attention_with_partition")
    _on_stream(stream, out, st, ql, kl)
    return (out, st) if with_stats else out


def sparsepr_key_metric(q, k, v, cfg, workspace=None, stream=None):
    """Returns (sample [B*H, M_s] int32, M_K [B*H, d, d], eigenvalues [B*H, d],
    key coordinate map [B*H, d, r_K])."""
    torch = _torch()
    B, H, N, d = q.shape
    ms = min(cfg.n_sample_q, N)
    dummy_o = torch.empty_like(q)
    io = _tensors(q, k, v, dummy_o)
    buf, nbytes = _ws(cfg, q, workspace, stream)
    smp = torch.empty(B * H, ms, dtype=torch.int32, device=q.device)
    mk = torch.empty(B * H, d, d, dtype=torch.float64, device=q.device)
    ev = torch.empty(B * H, d, dtype=torch.float64, device=q.device)
    rk = min(cfg.key_coord_rank, d, ms)
    km = torch.empty(B * H, d, rk, dtype=torch.float64, device=q.device)
    check(lib().sparsepr_key_metric(ctypes.byref(cfg), ctypes.byref(io), buf.data_ptr(), nbytes,
                                    _stream(stream), smp.data_ptr(), mk.data_ptr(), ev.data_ptr(),
                                    km.data_ptr()),
          "sparsepr_key_metric")
    return smp, mk, ev, km


def sparsepr_partition(q, k, v, cfg, workspace=None, stream=None):
    """Returns (q_labels, kv_labels), int32 [B*H, N]."""
    torch = _torch()
    B, H, N, d = q.shape
    io = _tensors(q, k, v, torch.empty_like(q))
    buf, nbytes = _ws(cfg, q, workspace, stream)
    ql = torch.empty(B * H, N, dtype=torch.int32, device=q.device)
    kl = torch.empty(B * H, N, dtype=torch.int32, device=q.device)
    check(lib().sparsepr_partition(ctypes.byref(cfg), ctypes.byref(io), buf.data_ptr(), nbytes,
                                   _stream(stream), ql.data_ptr(), kl.data_ptr()), "sparsepr_partition")
    return ql, kl


def sparsepr_route(q, k, v, cfg, q_labels, kv_labels, workspace=None, stream=None):
    """Returns dict of perm_q, perm_k, off_q, off_k, csr_rowptr, csr_cols, stats."""
    torch = _torch()
    B, H, N, d = q.shape
    io = _tensors(q, k, v, torch.empty_like(q))
    buf, nbytes = _ws(cfg, q, workspace, stream)
    dev = q.device
    BH, GQ, GK = B * H, cfg.n_q_groups, cfg.n_kv_groups
    res = {
        "perm_q": torch.empty(BH, N, dtype=torch.int32, device=dev),
        "perm_k": torch.empty(BH, N, dtype=torch.int32, device=dev),
        "off_q": torch.empty(BH, GQ + 1, dtype=torch.int32, device=dev),
        "off_k": torch.empty(BH, GK + 1, dtype=torch.int32, device=dev),
        "csr_rowptr": torch.empty(BH, GQ + 1, dtype=torch.int32, device=dev),
        "csr_cols": torch.full((BH, GQ * GK), -1, dtype=torch.int32, device=dev),
    }
    st = _stats_buf(q)
    ql = q_labels.to(torch.int32).contiguous()
    kl = kv_labels.to(torch.int32).contiguous()
    check(lib().sparsepr_route(ctypes.byref(cfg), ctypes.byref(io), ql.data_ptr(), kl.data_ptr(), buf.data_ptr(),
                               nbytes, _stream(stream), res["perm_q"].data_ptr(), res["perm_k"].data_ptr(),
                               res["off_q"].data_ptr(), res["off_k"].data_ptr(), res["csr_rowptr"].data_ptr(),
                               res["csr_cols"].data_ptr(), st.data_ptr()), "sparsepr_route")
    res["stats"] = st
    return res


def sparsepr_sparse_attention(q, k, v, cfg, q_labels, kv_labels, out=None, workspace=None, stream=None):
    """Uncorrected (hard-drop) sparse output in token order."""
    torch = _torch()
    out = torch.empty_like(q) if out is None else out
    io = _tensors(q, k, v, out)
    buf, nbytes = _ws(cfg, q, workspace, stream)
    ql = q_labels.to(torch.int32).contiguous()
    kl = kv_labels.to(torch.int32).contiguous()
    check(lib().sparsepr_sparse_attention(ctypes.byref(cfg), ctypes.byref(io), ql.data_ptr(), kl.data_ptr(),
                                          buf.data_ptr(), nbytes, _stream(stream)), "sparsepr_sparse_attention")
    _on_stream(stream, out, ql, kl)
    return out


def sparsepr_probe_fit(q, k, v, cfg, q_labels, kv_labels, workspace=None, stream=None):
    """Probe positions, exact dense and sparse probe outputs, and the fitted map."""
    torch = _torch()
    B, H, N, d = q.shape
    BH, M, R = B * H, cfg.probe_rows, max(cfg.residual_rank, 1)
    io = _tensors(q, k, v, torch.empty_like(q))
    buf, nbytes = _ws(cfg, q, workspace, stream)
    dev = q.device
    res = {
        "probe_pos": torch.empty(BH, M, dtype=torch.int32, device=dev),
        "o_dense": torch.empty(BH, M, d, dtype=torch.float32, device=dev),
        "o_sparse": torch.empty(BH, M, d, dtype=torch.float32, device=dev),
        "W": torch.empty(BH, d, R, dtype=torch.float32, device=dev),
        "V": torch.empty(BH, d, R, dtype=torch.float32, device=dev),
        "b": torch.empty(BH, d, dtype=torch.float32, device=dev),
        "rank": torch.empty(BH, dtype=torch.int32, device=dev),
    }
    ql = q_labels.to(torch.int32).contiguous()
    kl = kv_labels.to(torch.int32).contiguous()
    check(lib().sparsepr_probe_fit(ctypes.byref(cfg), ctypes.byref(io), ql.data_ptr(), kl.data_ptr(),
                                   buf.data_ptr(), nbytes, _stream(stream), res["probe_pos"].data_ptr(),
                                   res["o_dense"].data_ptr(), res["o_sparse"].data_ptr(), res["W"].data_ptr(),
                                   res["V"].data_ptr(), res["b"].data_ptr(), res["rank"].data_ptr()),
          "sparsepr_probe_fit")
    _on_stream(stream, ql, kl, *res.values())
    return res


def sparsepr_dense_attention(q, k, v, out=None, scale: float = 0.0, stream=None):
    torch = _torch()
    out = torch.empty_like(q) if out is None else out
    io = _tensors(q, k, v, out)
    check(lib().sparsepr_dense_attention(ctypes.byref(io), float(scale), _stream(stream)),
          "sparsepr_dense_attention")
    _on_stream(stream, out)
    return out


def sparsepr_mfma_rounding_check(patterns, stream=None):
    """Element (0, 0) of one bf16 32x32x16 matrix-core product per pattern.

    patterns: device float32 [n, 33] (16 values of row 0 of A, 16 of column 0
    of B, exact in bf16, then the accumulator).  Returns device float32 [n]."""
    torch = _torch()
    pats = patterns.to(torch.float32).contiguous()
    out = torch.empty(pats.shape[0], dtype=torch.float32, device=pats.device)
    check(lib().sparsepr_mfma_rounding_check(pats.data_ptr(), int(pats.shape[0]), out.data_ptr(), _stream(stream)),
          "sparsepr_mfma_rounding_check")
    return out
