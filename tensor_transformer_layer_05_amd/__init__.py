"""Python binding of libtplayer: one tensor-parallel rank's share of a
Megatron-style decoder layer on MI355X (gfx950) HIP kernels.

This module only marshals arguments: it checks devices/dtypes/contiguity,
allocates outputs with torch (device memory plumbing) and calls the C ABI
declared in ``include/tplayer.h`` on torch's current HIP stream.  Every step of
the computation runs in the library's kernels; there is no CPU or torch
fallback -- if the library is missing the calls raise.

Entry points (same names as the C ABI, without the ``tp_`` prefix):
``column_linear``, ``column_linear_act``, ``row_linear_partial``,
``swiglu_local``, ``local_attention``, ``kv_append``, ``reduce_partials``,
``reduce_partials_rmsnorm``, ``rmsnorm``, ``paged_attention_decode``,
``paged_kv_append``, ``decode_attention_append``, ``decode_attention_append_noalloc``,
``paged_decode_attention_append``,
``vocab_argmax_local``, ``vocab_argmax_reduce``.
Weights use the nn.Linear layout ``[out_features, in_features]``.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "lib", "library_path", "TPError",
    "column_linear", "column_linear_act", "row_linear_partial", "swiglu_local",
    "local_attention", "local_attention_workspace", "kv_append", "reduce_partials",
    "reduce_partials_rmsnorm", "rmsnorm", "vocab_argmax_local", "vocab_argmax_reduce",
    "paged_attention_decode", "paged_attention_workspace", "paged_kv_append",
    "decode_attention_append", "decode_attention_append_noalloc", "paged_decode_attention_append",
    "shard_column", "shard_row", "shard_qkv", "kv_heads_of_rank", "kv_cache_bytes_per_rank",
    "F32", "BF16", "ACT_NONE", "ACT_SWIGLU", "ACT_GELU",
]

F32, BF16 = 0, 1
ACT_NONE, ACT_SWIGLU, ACT_GELU = 0, 1, 2
_ACTS = {"none": ACT_NONE, "swiglu": ACT_SWIGLU, "gelu": ACT_GELU}
_DT = {torch.float32: F32, torch.bfloat16: BF16}

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libtplayer.so")

_lib = None

_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
_i64p = ctypes.POINTER(ctypes.c_int64)

_SIGS = {
    "tp_column_linear": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i64, _i64, ctypes.c_int, _vp]),
    "tp_column_linear_act": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i64, _i64, ctypes.c_int,
                                            ctypes.c_int, _vp]),
    "tp_row_linear_partial": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i64, _i64, ctypes.c_int, _vp]),
    "tp_swiglu_local": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i64, _i64, ctypes.c_int, ctypes.c_int, _vp]),
    "tp_local_attention": (ctypes.c_int, [_vp, _i64p, _vp, _vp, _i64p, _vp, _i64p, _i64, _i64, _i64,
                                          _i64, _i64, _i64, ctypes.c_int, ctypes.c_float, ctypes.c_int,
                                          _vp, ctypes.c_size_t, _vp]),
    "tp_local_attention_workspace": (ctypes.c_size_t, [_i64, _i64, _i64, _i64, _i64, _i64]),
    "tp_kv_append": (ctypes.c_int, [_vp, _vp, _i64, _vp, _vp, _i64p, _i64, _i64, _i64, _i64, _i64,
                                    ctypes.c_int, _vp]),
    "tp_reduce_partials": (ctypes.c_int, [ctypes.POINTER(_vp), _i64, _vp, ctypes.c_int, _vp, _i64,
                                          _i64, ctypes.c_int, _vp]),
    "tp_reduce_partials_rmsnorm": (ctypes.c_int, [ctypes.POINTER(_vp), _i64, _vp, ctypes.c_int, _vp,
                                                  ctypes.c_int, _vp, _vp, _i64, _i64, ctypes.c_float,
                                                  ctypes.c_int, _vp]),
    "tp_rmsnorm": (ctypes.c_int, [_vp, ctypes.c_int, _vp, _vp, _i64, _i64, ctypes.c_float,
                                  ctypes.c_int, _vp]),
    "tp_paged_attention_decode": (ctypes.c_int, [_vp, _i64p, _vp, _vp, _i64p, _i64, _vp, _i64, _vp,
                                                 _i64, _i64, _vp, _i64p, _i64, _i64, _i64, _i64,
                                                 ctypes.c_float, ctypes.c_int, _vp, ctypes.c_size_t,
                                                 _vp]),
    "tp_paged_attention_workspace": (ctypes.c_size_t, [_i64, _i64, _i64, _i64, _i64]),
    "tp_paged_kv_append": (ctypes.c_int, [_vp, _vp, _i64, _vp, _vp, _i64p, _i64, _vp, _i64, _vp,
                                          _i64, _i64, _i64, _i64, ctypes.c_int, _vp]),
    "tp_decode_attention_append": (ctypes.c_int, [_vp, _i64p, _vp, _vp, _i64, _vp, _vp, _i64p, _i64,
                                                  _i64, _vp, _i64p, _i64, _i64, _i64, _i64,
                                                  ctypes.c_float, ctypes.c_int, _vp, ctypes.c_size_t,
                                                  _vp]),
    "tp_decode_attention_append_noalloc": (ctypes.c_int, [_vp, _i64p, _vp, _vp, _i64, _vp, _vp,
                                                          _i64p, _i64, _i64, _vp, _i64p, _i64, _i64,
                                                          _i64, _i64, ctypes.c_float, ctypes.c_int,
                                                          _vp]),
    "tp_paged_decode_attention_append": (ctypes.c_int, [_vp, _i64p, _vp, _vp, _i64, _vp, _vp, _i64p,
                                                        _i64, _vp, _i64, _vp, _i64, _i64, _vp, _i64p,
                                                        _i64, _i64, _i64, _i64, ctypes.c_float,
                                                        ctypes.c_int, _vp, ctypes.c_size_t, _vp]),
    "tp_vocab_argmax_local": (ctypes.c_int, [_vp, _i64, _i64, _i64, _vp, _vp, _vp]),
    "tp_vocab_argmax_reduce": (ctypes.c_int, [ctypes.POINTER(_vp), ctypes.POINTER(_vp), _i64, _i64,
                                              _vp, _vp, _vp]),
    "tp_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "tp_last_error": (ctypes.c_char_p, []),
    "tp_version": (ctypes.c_char_p, []),
}

EXPORTED = tuple(_SIGS)


class TPError(RuntimeError):
    def __init__(self, fn: str, status: int):
        l = lib()
        msg = l.tp_status_string(status).decode()
        if status == 6:
            msg += ": " + l.tp_last_error().decode()
        super().__init__(f"{fn} failed with status {status} ({msg})")
        self.status = status


def lib():
    """Load (once) and return the ctypes handle of libtplayer.so."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise RuntimeError(
                f"{library_path} is not built; run `python -c 'import __graft_entry__ as g; g.build()'` "
                "(there is no fallback path)")
        l = ctypes.CDLL(library_path)
        for name, (res, args) in _SIGS.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


def _check(fn: str, status: int):
    if status != 0:
        raise TPError(fn, status)


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dev(t: torch.Tensor, name: str, dtypes=_DT):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype not in dtypes:
        raise ValueError(f"{name}: unsupported dtype {t.dtype}")
    return t


def _contig(t: torch.Tensor, name: str, dtypes=_DT):
    _dev(t, name, dtypes)
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _arr3(strides):
    return (ctypes.c_int64 * 3)(*[int(s) for s in strides])


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------

def column_linear(x: torch.Tensor, w: torch.Tensor, out: torch.Tensor | None = None):
    """Rank's output slice ``y = x @ w.T`` (x ``[M,K]``, w ``[N,K]``)."""
    _contig(x, "x"); _contig(w, "w")
    M, K = x.shape
    N = w.shape[0]
    if w.shape[1] != K or w.dtype != x.dtype:
        raise ValueError("w must be [N, K] with the dtype of x")
    if out is None:
        out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    _contig(out, "out")
    _check("tp_column_linear", lib().tp_column_linear(x.data_ptr(), w.data_ptr(), out.data_ptr(),
                                                      M, K, N, _DT[x.dtype], _stream(x)))
    return out


def column_linear_act(x: torch.Tensor, w: torch.Tensor, act: str = "swiglu",
                      out: torch.Tensor | None = None):
    """Column-parallel linear with the rank-local activation in its epilogue.
    swiglu: w ``[2I, K]`` (gate rows then up rows) -> ``[M, I]``;
    gelu: w ``[I, K]`` -> ``[M, I]``.  Equals ``column_linear`` followed by
    ``swiglu_local`` bit for bit, without the ``[M, 2I]`` intermediate."""
    _contig(x, "x"); _contig(w, "w")
    M, K = x.shape
    a = _act(act)
    if w.dim() != 2 or w.shape[1] != K or w.dtype != x.dtype:
        raise ValueError("w must be [N, K] with the dtype of x")
    if a == ACT_SWIGLU:
        if w.shape[0] % 2:
            raise ValueError("swiglu needs a [2I, K] gate|up weight")
        I_ = w.shape[0] // 2
    else:
        I_ = w.shape[0]
    if out is None:
        out = torch.empty((M, I_), dtype=x.dtype, device=x.device)
    _contig(out, "out")
    if out.shape != (M, I_) or out.dtype != x.dtype:
        raise ValueError("out must be [M, I] with the dtype of x")
    _check("tp_column_linear_act", lib().tp_column_linear_act(
        x.data_ptr(), w.data_ptr(), out.data_ptr(), M, K, I_, a, _DT[x.dtype], _stream(x)))
    return out


def row_linear_partial(x: torch.Tensor, w: torch.Tensor, out: torch.Tensor | None = None):
    """Rank's float32 partial ``p = x_r @ w_r.T`` (x ``[M,K_r]``, w ``[N,K_r]``)."""
    _contig(x, "x"); _contig(w, "w")
    M, K = x.shape
    N = w.shape[0]
    if w.shape[1] != K or w.dtype != x.dtype:
        raise ValueError("w must be [N, K] with the dtype of x")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=x.device)
    _contig(out, "out")
    if out.dtype != torch.float32:
        raise ValueError("partials are float32")
    _check("tp_row_linear_partial", lib().tp_row_linear_partial(
        x.data_ptr(), w.data_ptr(), out.data_ptr(), M, K, N, _DT[x.dtype], _stream(x)))
    return out


def swiglu_local(gate: torch.Tensor, up: torch.Tensor | None = None, act: str = "swiglu",
                 out: torch.Tensor | None = None):
    """Rank-local activation.  ``gate``/``up`` are ``[M, I]`` views that may
    share a row stride (e.g. the two halves of a fused gate|up output)."""
    _dev(gate, "gate")
    if gate.dim() != 2 or gate.stride(1) != 1:
        raise ValueError("gate must be a 2-D row-major view")
    M, I = gate.shape
    ld = gate.stride(0)
    a = _act(act)
    if a == ACT_SWIGLU:
        if up is None:
            raise ValueError("swiglu needs up")
        _dev(up, "up")
        if up.shape != gate.shape or up.stride() != gate.stride() or up.dtype != gate.dtype:
            raise ValueError("up must match gate's shape, strides and dtype")
    if out is None:
        out = torch.empty((M, I), dtype=gate.dtype, device=gate.device)
    _contig(out, "out")
    _check("tp_swiglu_local", lib().tp_swiglu_local(
        gate.data_ptr(), up.data_ptr() if (up is not None and a == ACT_SWIGLU) else None,
        out.data_ptr(), M, I, ld, a, _DT[gate.dtype], _stream(gate)))
    return out


def _act(act):
    if isinstance(act, int):
        return act
    return _ACTS[act]


def local_attention_workspace(B, Sq, Skv, Hq, Hkv, D) -> int:
    return int(lib().tp_local_attention_workspace(B, Sq, Skv, Hq, Hkv, D))


def local_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = True,
                    scale: float | None = None, out: torch.Tensor | None = None,
                    workspace: torch.Tensor | None = None):
    """Attention over local heads.  q ``[B,Sq,Hq,D]``, k/v ``[B,Skv,Hkv,D]``
    (any strides with a contiguous last dim; k and v share strides).
    Returns o ``[B,Sq,Hq,D]`` (or writes the given ``out`` view)."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _dev(t, n)
        if t.dim() != 4 or t.stride(3) != 1:
            raise ValueError(f"{n} must be 4-D with a contiguous last dimension")
    if k.stride() != v.stride() or k.shape != v.shape:
        raise ValueError("k and v must have the same shape and strides")
    B, Sq, Hq, D = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    if out is None:
        out = torch.empty((B, Sq, Hq, D), dtype=q.dtype, device=q.device)
    if out.dim() != 4 or out.stride(3) != 1:
        raise ValueError("out must be 4-D with a contiguous last dimension")
    if scale is None:
        scale = 1.0 / (D ** 0.5)
    need = local_attention_workspace(B, Sq, Skv, Hq, Hkv, D)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    qs = _arr3([q.stride(0), q.stride(1), q.stride(2)])
    kvs = _arr3([k.stride(0), k.stride(1), k.stride(2)])
    os_ = _arr3([out.stride(0), out.stride(1), out.stride(2)])
    _check("tp_local_attention", lib().tp_local_attention(
        q.data_ptr(), qs, k.data_ptr(), v.data_ptr(), kvs, out.data_ptr(), os_,
        B, Sq, Skv, Hq, Hkv, D, int(bool(causal)), float(scale), _DT[q.dtype],
        workspace.data_ptr() if need else None, need, _stream(q)))
    return out


def kv_append(k_new: torch.Tensor, v_new: torch.Tensor, k_cache: torch.Tensor,
              v_cache: torch.Tensor, pos: int):
    """Write the current token's k/v (``[B, Hkv, D]`` views with a shared row
    stride) into the caches ``[B, T, Hkv, D]`` (any strides, last dim
    contiguous) at key position ``pos``."""
    for t, n in ((k_new, "k_new"), (v_new, "v_new"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _dev(t, n)
    B, H, D = k_new.shape
    if k_new.stride(2) != 1 or k_new.stride(1) != D or v_new.stride() != k_new.stride():
        raise ValueError("k_new/v_new must be [B, Hkv, D] rows of one stride")
    if k_cache.stride() != v_cache.stride() or k_cache.stride(3) != 1:
        raise ValueError("caches must share strides with a contiguous last dim")
    if not (0 <= pos < k_cache.shape[1]):
        raise ValueError("pos outside the cache")
    cs = _arr3([k_cache.stride(0), k_cache.stride(1), k_cache.stride(2)])
    _check("tp_kv_append", lib().tp_kv_append(
        k_new.data_ptr(), v_new.data_ptr(), k_new.stride(0), k_cache.data_ptr(), v_cache.data_ptr(),
        cs, B, H, D, k_cache.shape[1], pos, _DT[k_new.dtype], _stream(k_new)))


def _new_rows(k_new, v_new):
    for t, n in ((k_new, "k_new"), (v_new, "v_new")):
        _dev(t, n)
    B, H, D = k_new.shape
    if k_new.stride(2) != 1 or k_new.stride(1) != D or v_new.stride() != k_new.stride():
        raise ValueError("k_new/v_new must be [B, Hkv, D] rows of one stride")
    return B, H, D


def _decode_append_args(q, k_new, v_new, k_cache, v_cache, pos, scale, out):
    _dev(q, "q")
    if q.dim() != 3 or q.stride(2) != 1:
        raise ValueError("q must be [B, Hq, D] with a contiguous last dimension")
    B, H, D = _new_rows(k_new, v_new)
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        _dev(t, n)
    if k_cache.stride() != v_cache.stride() or k_cache.shape != v_cache.shape or k_cache.stride(3) != 1:
        raise ValueError("caches must share shape and strides with a contiguous last dim")
    if not (0 <= pos < k_cache.shape[1]):
        raise ValueError("pos outside the cache")
    Hq = q.shape[1]
    if out is None:
        out = torch.empty((B, Hq, D), dtype=q.dtype, device=q.device)
    if out.dim() != 3 or out.stride(2) != 1:
        raise ValueError("out must be [B, Hq, D] with a contiguous last dimension")
    if scale is None:
        scale = 1.0 / (D ** 0.5)
    qs = (ctypes.c_int64 * 2)(q.stride(0), q.stride(1))
    os_ = (ctypes.c_int64 * 2)(out.stride(0), out.stride(1))
    cs = _arr3([k_cache.stride(0), k_cache.stride(1), k_cache.stride(2)])
    args = (q.data_ptr(), qs, k_new.data_ptr(), v_new.data_ptr(), k_new.stride(0), k_cache.data_ptr(),
            v_cache.data_ptr(), cs, k_cache.shape[1], pos, out.data_ptr(), os_, B, Hq, H, D,
            float(scale), _DT[q.dtype])
    return out, args, (B, Hq, H, D)


def decode_attention_append(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                            k_cache: torch.Tensor, v_cache: torch.Tensor, pos: int,
                            scale: float | None = None, out: torch.Tensor | None = None,
                            workspace: torch.Tensor | None = None):
    """One decode step in one launch: store k_new/v_new (``[B, Hkv, D]``
    views with a shared row stride) at key position ``pos`` of the caches
    (``[B, T, Hkv, D]``, any strides, last dim contiguous) and attend q
    (``[B, Hq, D]``) over keys ``0..pos``.  The same bits as ``kv_append``
    followed by ``local_attention`` with ``Skv = pos + 1``.  Returns o
    ``[B, Hq, D]``."""
    out, args, (B, Hq, H, D) = _decode_append_args(q, k_new, v_new, k_cache, v_cache, pos, scale, out)
    need = local_attention_workspace(B, 1, pos + 1, Hq, H, D)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _check("tp_decode_attention_append", lib().tp_decode_attention_append(
        *args, workspace.data_ptr() if need else None, need, _stream(q)))
    return out


def decode_attention_append_noalloc(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                                    k_cache: torch.Tensor, v_cache: torch.Tensor, pos: int,
                                    out: torch.Tensor, scale: float | None = None):
    """``decode_attention_append`` with no workspace: the library keeps the
    split-key partials in its own static device buffer, so the call allocates
    nothing (``out`` must be given).  Calls overlapping in time on one GPU
    share that buffer and must not be issued."""
    if out is None:
        raise ValueError("out must be given (the call allocates nothing)")
    out, args, _ = _decode_append_args(q, k_new, v_new, k_cache, v_cache, pos, scale, out)
    _check("tp_decode_attention_append_noalloc",
           lib().tp_decode_attention_append_noalloc(*args, _stream(q)))
    return out


def _partials(partials):
    parts = list(partials)
    if not parts:
        raise ValueError("need at least one partial")
    for i, p in enumerate(parts):
        _contig(p, f"partials[{i}]")
        if p.dtype != torch.float32 or p.shape != parts[0].shape:
            raise ValueError("partials must be float32 tensors of one shape")
    return parts


def reduce_partials(partials, residual: torch.Tensor | None = None, out: torch.Tensor | None = None,
                    out_dtype: torch.dtype | None = None):
    """``y = sum_r partials[r] + residual`` in rank order (float32 sums, the
    residual added last).  The residual may be bf16 or float32 whatever the
    output dtype; ``out`` may be the residual tensor itself when the two share
    a dtype."""
    parts = _partials(partials)
    M, N = parts[0].shape
    if out is None:
        dt = out_dtype or (residual.dtype if residual is not None else torch.float32)
        out = torch.empty((M, N), dtype=dt, device=parts[0].device)
    _contig(out, "out")
    if out.shape != (M, N):
        raise ValueError("out must be [M, N]")
    if residual is not None:
        _contig(residual, "residual")
        if residual.shape != (M, N):
            raise ValueError("residual must be [M, N]")
    arr = (ctypes.c_void_p * len(parts))(*[p.data_ptr() for p in parts])
    _check("tp_reduce_partials", lib().tp_reduce_partials(
        arr, len(parts), residual.data_ptr() if residual is not None else None,
        _DT[residual.dtype] if residual is not None else F32, out.data_ptr(), M, N,
        _DT[out.dtype], _stream(parts[0])))
    return out


def reduce_partials_rmsnorm(partials, gamma: torch.Tensor, residual: torch.Tensor | None = None,
                            eps: float = 1e-5, out: torch.Tensor | None = None,
                            out_norm: torch.Tensor | None = None,
                            out_dtype: torch.dtype | None = None):
    """``y = sum_r partials[r] + residual`` (as ``reduce_partials``) and
    ``yn = rmsnorm(y) * gamma`` (as ``rmsnorm`` on the stored y) in one pass.
    ``yn`` has gamma's dtype; ``y`` has ``out``'s dtype, else ``out_dtype``,
    else gamma's (float32 keeps the residual stream unrounded).  Returns
    ``(y, yn)``."""
    parts = _partials(partials)
    M, N = parts[0].shape
    _contig(gamma, "gamma")
    dt = gamma.dtype
    if gamma.shape != (N,):
        raise ValueError("gamma must be [N]")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype or dt, device=parts[0].device)
    if out_norm is None:
        out_norm = torch.empty((M, N), dtype=dt, device=parts[0].device)
    _contig(out, "out")
    _contig(out_norm, "out_norm")
    if out.shape != (M, N):
        raise ValueError("out must be [M, N]")
    if out_norm.dtype != dt or out_norm.shape != (M, N):
        raise ValueError("out_norm must be [M, N] with gamma's dtype")
    if residual is not None:
        _contig(residual, "residual")
        if residual.shape != (M, N):
            raise ValueError("residual must be [M, N]")
    arr = (ctypes.c_void_p * len(parts))(*[p.data_ptr() for p in parts])
    _check("tp_reduce_partials_rmsnorm", lib().tp_reduce_partials_rmsnorm(
        arr, len(parts), residual.data_ptr() if residual is not None else None,
        _DT[residual.dtype] if residual is not None else F32, out.data_ptr(), _DT[out.dtype],
        gamma.data_ptr(), out_norm.data_ptr(), M, N, float(eps), _DT[dt], _stream(parts[0])))
    return out, out_norm


def rmsnorm(x: torch.Tensor, gamma: torch.Tensor, eps: float = 1e-5, out: torch.Tensor | None = None):
    """``y = x * rsqrt(mean(x^2) + eps) * gamma`` per row; y has gamma's dtype
    (x may be a float32 residual stream with bf16 gamma)."""
    _contig(x, "x"); _contig(gamma, "gamma")
    M, N = x.shape
    if gamma.shape != (N,):
        raise ValueError("gamma must be [N]")
    if out is None:
        out = torch.empty((M, N), dtype=gamma.dtype, device=x.device)
    _contig(out, "out")
    if out.dtype != gamma.dtype or out.shape != (M, N):
        raise ValueError("out must be [M, N] with gamma's dtype")
    _check("tp_rmsnorm", lib().tp_rmsnorm(x.data_ptr(), _DT[x.dtype], gamma.data_ptr(), out.data_ptr(),
                                          M, N, float(eps), _DT[gamma.dtype], _stream(x)))
    return out


def _paged_common(block_table, context_lens, k_pool, v_pool):
    _contig(block_table, "block_table", (torch.int32,))
    _contig(context_lens, "context_lens", (torch.int32,))
    for t, n in ((k_pool, "k_pool"), (v_pool, "v_pool")):
        _dev(t, n)
        if t.dim() != 4 or t.stride(3) != 1:
            raise ValueError(f"{n} must be [num_blocks, block_size, Hkv, D] with a contiguous last dim")
    if k_pool.shape != v_pool.shape or k_pool.stride() != v_pool.stride():
        raise ValueError("k_pool and v_pool must have the same shape and strides")
    if block_table.dim() != 2 or context_lens.shape != (block_table.shape[0],):
        raise ValueError("block_table must be [B, max_blocks] and context_lens [B]")
    return _arr3([k_pool.stride(0), k_pool.stride(1), k_pool.stride(2)])


def paged_attention_workspace(B, Hq, Hkv, max_context_len, block_size) -> int:
    return int(lib().tp_paged_attention_workspace(B, Hq, Hkv, max_context_len, block_size))


def paged_attention_decode(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                           block_table: torch.Tensor, context_lens: torch.Tensor,
                           max_context_len: int, scale: float | None = None,
                           out: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """Decode attention over a paged KV cache.  q ``[B, Hq, D]`` (last dim
    contiguous); pools ``[num_blocks, block_size, Hkv, D]``; block_table
    ``[B, max_blocks]`` int32; context_lens ``[B]`` int32 (keys per sequence,
    the current token included).  Returns o ``[B, Hq, D]``."""
    _dev(q, "q")
    if q.dim() != 3 or q.stride(2) != 1:
        raise ValueError("q must be [B, Hq, D] with a contiguous last dimension")
    ps = _paged_common(block_table, context_lens, k_pool, v_pool)
    B, Hq, D = q.shape
    nb, bs, Hkv = k_pool.shape[0], k_pool.shape[1], k_pool.shape[2]
    if block_table.shape[0] != B:
        raise ValueError("block_table must have one row per sequence")
    if out is None:
        out = torch.empty((B, Hq, D), dtype=q.dtype, device=q.device)
    if out.dim() != 3 or out.stride(2) != 1:
        raise ValueError("out must be [B, Hq, D] with a contiguous last dimension")
    if scale is None:
        scale = 1.0 / (D ** 0.5)
    need = paged_attention_workspace(B, Hq, Hkv, max_context_len, bs)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    qs = (ctypes.c_int64 * 2)(q.stride(0), q.stride(1))
    os_ = (ctypes.c_int64 * 2)(out.stride(0), out.stride(1))
    _check("tp_paged_attention_decode", lib().tp_paged_attention_decode(
        q.data_ptr(), qs, k_pool.data_ptr(), v_pool.data_ptr(), ps, nb, block_table.data_ptr(),
        block_table.stride(0), context_lens.data_ptr(), int(max_context_len), bs, out.data_ptr(), os_,
        B, Hq, Hkv, D, float(scale), _DT[q.dtype], workspace.data_ptr() if need else None, need,
        _stream(q)))
    return out


def paged_kv_append(k_new: torch.Tensor, v_new: torch.Tensor, k_pool: torch.Tensor,
                    v_pool: torch.Tensor, block_table: torch.Tensor, context_lens: torch.Tensor):
    """Store each sequence's current k/v (``[B, Hkv, D]`` views with a shared
    row stride) at position ``context_lens[b] - 1`` of the paged pools."""
    for t, n in ((k_new, "k_new"), (v_new, "v_new")):
        _dev(t, n)
    ps = _paged_common(block_table, context_lens, k_pool, v_pool)
    B, H, D = k_new.shape
    if k_new.stride(2) != 1 or k_new.stride(1) != D or v_new.stride() != k_new.stride():
        raise ValueError("k_new/v_new must be [B, Hkv, D] rows of one stride")
    _check("tp_paged_kv_append", lib().tp_paged_kv_append(
        k_new.data_ptr(), v_new.data_ptr(), k_new.stride(0), k_pool.data_ptr(), v_pool.data_ptr(), ps,
        k_pool.shape[0], block_table.data_ptr(), block_table.stride(0), context_lens.data_ptr(), B, H,
        D, k_pool.shape[1], _DT[k_new.dtype], _stream(k_new)))


def paged_decode_attention_append(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                                  k_pool: torch.Tensor, v_pool: torch.Tensor,
                                  block_table: torch.Tensor, context_lens: torch.Tensor,
                                  max_context_len: int, scale: float | None = None,
                                  out: torch.Tensor | None = None,
                                  workspace: torch.Tensor | None = None):
    """``paged_kv_append`` followed by ``paged_attention_decode`` in one
    launch, with the same bits (no slot the append writes may be read by
    another sequence or through a second table entry).  Returns o
    ``[B, Hq, D]``."""
    _dev(q, "q")
    if q.dim() != 3 or q.stride(2) != 1:
        raise ValueError("q must be [B, Hq, D] with a contiguous last dimension")
    B, H, D = _new_rows(k_new, v_new)
    ps = _paged_common(block_table, context_lens, k_pool, v_pool)
    Hq = q.shape[1]
    nb, bs, Hkv = k_pool.shape[0], k_pool.shape[1], k_pool.shape[2]
    if block_table.shape[0] != B or q.shape[0] != B or Hkv != H:
        raise ValueError("q, k_new, block_table and the pools must agree on sequences and KV heads")
    if out is None:
        out = torch.empty((B, Hq, D), dtype=q.dtype, device=q.device)
    if out.dim() != 3 or out.stride(2) != 1:
        raise ValueError("out must be [B, Hq, D] with a contiguous last dimension")
    if scale is None:
        scale = 1.0 / (D ** 0.5)
    need = paged_attention_workspace(B, Hq, Hkv, max_context_len, bs)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    qs = (ctypes.c_int64 * 2)(q.stride(0), q.stride(1))
    os_ = (ctypes.c_int64 * 2)(out.stride(0), out.stride(1))
    _check("tp_paged_decode_attention_append", lib().tp_paged_decode_attention_append(
        q.data_ptr(), qs, k_new.data_ptr(), v_new.data_ptr(), k_new.stride(0), k_pool.data_ptr(),
        v_pool.data_ptr(), ps, nb, block_table.data_ptr(), block_table.stride(0),
        context_lens.data_ptr(), int(max_context_len), bs, out.data_ptr(), os_, B, Hq, Hkv, D,
        float(scale), _DT[q.dtype], workspace.data_ptr() if need else None, need, _stream(q)))
    return out


def vocab_argmax_local(logits: torch.Tensor, vocab_offset: int = 0):
    """Per row of a rank's fp32 logits ``[M, V_r]``: the largest logit and its
    global vocab id (NaN counts as -inf; ties go to the lower id).
    Returns ``(values [M] float32, ids [M] int64)``."""
    _contig(logits, "logits")
    if logits.dtype != torch.float32 or logits.dim() != 2:
        raise ValueError("logits must be a 2-D float32 tensor")
    M, V = logits.shape
    mv = torch.empty(M, dtype=torch.float32, device=logits.device)
    mi = torch.empty(M, dtype=torch.int64, device=logits.device)
    _check("tp_vocab_argmax_local", lib().tp_vocab_argmax_local(
        logits.data_ptr(), M, V, int(vocab_offset), mv.data_ptr(), mi.data_ptr(), _stream(logits)))
    return mv, mi


def vocab_argmax_reduce(vals, idxs):
    """Combine the ranks' ``(values, ids)`` in rank order: the argmax over the
    full vocab.  Returns ``(values [M], ids [M])``."""
    vals, idxs = list(vals), list(idxs)
    if not vals or len(vals) != len(idxs):
        raise ValueError("need one (values, ids) pair per rank")
    M = vals[0].shape[0]
    for v, i in zip(vals, idxs):
        _contig(v, "values"); _contig(i, "ids", (torch.int64,))
        if v.dtype != torch.float32 or i.dtype != torch.int64 or v.shape != (M,) or i.shape != (M,):
            raise ValueError("values must be [M] float32 and ids [M] int64")
    ov = torch.empty(M, dtype=torch.float32, device=vals[0].device)
    oi = torch.empty(M, dtype=torch.int64, device=vals[0].device)
    va = (ctypes.c_void_p * len(vals))(*[v.data_ptr() for v in vals])
    ia = (ctypes.c_void_p * len(idxs))(*[i.data_ptr() for i in idxs])
    _check("tp_vocab_argmax_reduce", lib().tp_vocab_argmax_reduce(
        va, ia, len(vals), M, ov.data_ptr(), oi.data_ptr(), _stream(vals[0])))
    return ov, oi


# ---------------------------------------------------------------------------
# host-side shard slicing (contiguous blocks in rank order)
# ---------------------------------------------------------------------------

def _block(n: int, r: int, R: int):
    if R <= 0 or not (0 <= r < R):
        raise ValueError(f"rank {r} out of range for TP size {R}")
    if n % R:
        raise ValueError(f"dimension {n} is not divisible by TP size {R}")
    b = n // R
    return r * b, b


def shard_column(w: torch.Tensor, r: int, R: int) -> torch.Tensor:
    """Rank r's output-feature block (rows) of an ``[N, K]`` weight."""
    s, b = _block(w.shape[0], r, R)
    return w.narrow(0, s, b).contiguous()


def shard_row(w: torch.Tensor, r: int, R: int) -> torch.Tensor:
    """Rank r's input-feature block (columns) of an ``[N, K]`` weight."""
    s, b = _block(w.shape[1], r, R)
    return w.narrow(1, s, b).contiguous()


def kv_heads_of_rank(n_q: int, n_kv: int, r: int, R: int) -> list:
    """Global ids of the KV heads rank r holds.  KV heads are split in
    contiguous blocks when they divide by R; with fewer KV heads than ranks
    (GQA at a large TP size) each rank holds the single KV head its q heads
    read, replicated on R / n_kv ranks (requires R % n_kv == 0)."""
    if R <= 0 or not (0 <= r < R):
        raise ValueError(f"rank {r} out of range for TP size {R}")
    if n_q % R or n_q % n_kv:
        raise ValueError("q heads must divide by the TP size and by the KV heads")
    if n_kv % R == 0:
        c = n_kv // R
        return list(range(r * c, (r + 1) * c))
    if R % n_kv:
        raise ValueError("KV heads must divide by the TP size or the TP size by the KV heads")
    return [(r * (n_q // R)) // (n_q // n_kv)]


def kv_cache_bytes_per_rank(n_q: int, n_kv: int, R: int, batch: int, kv_len: int,
                            head_dim: int, elem_bytes: int = 2) -> int:
    """K and V cache bytes one rank keeps (replicated KV heads count on every
    rank that holds them)."""
    return 2 * batch * kv_len * len(kv_heads_of_rank(n_q, n_kv, 0, R)) * head_dim * elem_bytes


def shard_qkv(wq: torch.Tensor, wk: torch.Tensor, wv: torch.Tensor, r: int, R: int,
              head_dim: int) -> torch.Tensor:
    """Rank r's fused ``[q heads | k heads | v heads]`` weight (its KV heads
    per ``kv_heads_of_rank``)."""
    for t in (wq, wk, wv):
        if t.shape[0] % head_dim:
            raise ValueError("projection rows must be whole heads")
    heads = kv_heads_of_rank(wq.shape[0] // head_dim, wk.shape[0] // head_dim, r, R)
    j0, c = heads[0], len(heads)
    return torch.cat([shard_column(wq, r, R), wk.narrow(0, j0 * head_dim, c * head_dim),
                      wv.narrow(0, j0 * head_dim, c * head_dim)], 0).contiguous()
