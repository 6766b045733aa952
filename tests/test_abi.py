"""C-ABI checks that need no GPU: the library loads, exports every function
declared in include/tplayer.h, and rejects invalid arguments with the
documented status before launching anything.

The invalid-argument cases pass made-up non-NULL addresses; each is built so
that validation must reject it.  They are skipped where a GPU is visible, so
that a validation bug can never turn one into a launch on a bogus address.
"""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

import tensor_transformer_layer_05_amd as tpl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tplayer.h")

OK, NULL, SHAPE, DTYPE, ALIGN, WORKSPACE, HIP, UNSUPPORTED = range(8)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(tpl.library_path):
        from tensor_transformer_layer_05_amd.csrc import build
        build.build(force=False)
    return tpl.lib()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tp_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("tp_column_linear", "tp_swiglu_local", "tp_local_attention", "tp_row_linear_partial",
              "tp_reduce_partials", "tp_rmsnorm", "tp_kv_append", "tp_status_string",
              "tp_column_linear_act", "tp_reduce_partials_rmsnorm"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for n in _declared():
        assert hasattr(lib, n), f"{n} declared in tplayer.h but not exported"
    assert set(_declared()) == set(tpl.EXPORTED)


def test_reference_library_exports_its_header():
    """libtpref.so (the measurement reference stream, not part of the layer)
    exports what include/tpref.h declares."""
    import ctypes as C
    from tensor_transformer_layer_05_amd import ref
    if not os.path.exists(ref.library_path):
        from tensor_transformer_layer_05_amd.csrc import build
        build.build(force=False)
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "tpref.h")).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(tpref_[a-z_0-9]+)\s*\(", text)))
    assert names == ["tpref_stream_read"]
    l = C.CDLL(ref.library_path)
    for n in names:
        assert hasattr(l, n)


def test_status_strings(lib):
    for s in range(8):
        assert lib.tp_status_string(s)
    assert lib.tp_status_string(99) == b"unknown status"
    assert b"gfx950" in lib.tp_version()


no_gpu = pytest.mark.skipif(torch.cuda.device_count() > 0,
                            reason="fake-address validation cases run only where no GPU is visible")

P = 0x10000          # a made-up, 64 KiB aligned address (never dereferenced)
S = None             # default stream


@no_gpu
def test_linear_validation(lib):
    for fn in (lib.tp_column_linear, lib.tp_row_linear_partial):
        assert fn(None, P, P, 4, 8, 8, 1, S) == NULL
        assert fn(P, None, P, 4, 8, 8, 1, S) == NULL
        assert fn(P, P, None, 4, 8, 8, 1, S) == NULL
        assert fn(P, P, P, 0, 8, 8, 1, S) == SHAPE
        assert fn(P, P, P, 4, -1, 8, 1, S) == SHAPE
        assert fn(P, P, P, 4, 8, 0, 1, S) == SHAPE
        assert fn(P, P, P, 4, 8, 8, 7, S) == DTYPE
        assert fn(P + 1, P, P, 4, 8, 8, 1, S) == ALIGN
        assert fn(P, P + 2, P, 4, 8, 8, 0, S) == ALIGN       # fp32 needs 4-byte alignment
        assert fn(P, P, P, 1 << 31, 8, 8, 1, S) == UNSUPPORTED
    assert lib.tp_row_linear_partial(P, P, P + 2, 4, 8, 8, 1, S) == ALIGN   # fp32 partial


@no_gpu
def test_activation_validation(lib):
    f = lib.tp_swiglu_local
    assert f(None, P, P, 2, 8, 8, 1, 1, S) == NULL
    assert f(P, None, P, 2, 8, 8, 1, 1, S) == NULL          # swiglu needs up
    assert f(P, P, P, 2, 8, 4, 1, 1, S) == SHAPE            # ld < I
    assert f(P, P, P, 0, 8, 8, 1, 1, S) == SHAPE
    assert f(P, P, P, 2, 8, 8, 9, 1, S) == DTYPE            # bad activation
    assert f(P, P, P, 2, 8, 8, 1, 5, S) == DTYPE            # bad dtype
    assert f(P + 1, P, P, 2, 8, 8, 1, 1, S) == ALIGN


def _s3(*v):
    return (ctypes.c_int64 * 3)(*v)


@no_gpu
def test_attention_validation(lib):
    f = lib.tp_local_attention
    qs, kvs, os_ = _s3(1024, 1024, 128), _s3(2 * 64 * 128, 128, 64 * 128), _s3(1024, 1024, 128)
    args = dict(B=2, Sq=1, Skv=64, Hq=8, Hkv=2, D=128)

    def call(q=P, k=P, v=P, o=P, qs=qs, kvs=kvs, os_=os_, B=2, Sq=1, Skv=64, Hq=8, Hkv=2, D=128,
             causal=1, scale=0.088, dt=1, ws=None, wsb=0):
        return f(q, qs, k, v, kvs, o, os_, B, Sq, Skv, Hq, Hkv, D, causal, scale, dt, ws, wsb, S)

    assert call(q=None) == NULL
    assert call(os_=None) == NULL
    assert call(Hq=6, Hkv=4) == SHAPE                        # Hq % Hkv != 0
    assert call(Sq=65, Skv=64) == SHAPE                      # causal with more queries than keys
    assert call(B=0) == SHAPE
    assert call(scale=float("inf")) == SHAPE
    assert call(D=64) == UNSUPPORTED
    assert call(dt=0) == UNSUPPORTED
    assert call(dt=3) == DTYPE
    assert call(qs=_s3(1024, 1024, 100)) == ALIGN            # head stride not a multiple of 8
    assert call(q=P + 2) == ALIGN
    # decode with enough sequences x KV heads never needs a workspace; with a
    # long span and few pairs it does
    need = lib.tp_local_attention_workspace(1, 1, 4096, 8, 2, 128)
    assert need > 0
    assert call(B=1, Skv=4096, kvs=_s3(2 * 4096 * 128, 128, 4096 * 128)) == WORKSPACE
    assert call(B=1, Skv=4096, kvs=_s3(2 * 4096 * 128, 128, 4096 * 128), ws=P, wsb=need - 1) == WORKSPACE
    assert lib.tp_local_attention_workspace(1, 128, 4096, 8, 2, 128) == 0   # prefill: none
    assert lib.tp_local_attention_workspace(1, 1, 4096, 6, 4, 128) == 0     # invalid: none


@no_gpu
def test_reduce_validation(lib):
    f = lib.tp_reduce_partials
    arr = (ctypes.c_void_p * 2)(P, P)
    assert f(None, 2, None, 0, P, 4, 4, 0, S) == NULL
    assert f(arr, 0, None, 0, P, 4, 4, 0, S) == SHAPE
    assert f(arr, 17, None, 0, P, 4, 4, 0, S) == SHAPE
    bad = (ctypes.c_void_p * 2)(P, None)
    assert f(bad, 2, None, 0, P, 4, 4, 0, S) == NULL
    assert f(arr, 2, None, 0, P, 0, 4, 0, S) == SHAPE
    assert f(arr, 2, None, 0, P, 4, 4, 4, S) == DTYPE
    assert f(arr, 2, P + 256, 7, P, 4, 4, 0, S) == DTYPE          # bad residual dtype
    assert f(arr, 2, P + 258, 0, P, 4, 4, 0, S) == ALIGN
    odd = (ctypes.c_void_p * 2)(P, P + 2)
    assert f(odd, 2, None, 0, P, 4, 4, 0, S) == ALIGN
    # y may be the residual itself only with one storage type; other overlaps
    # are rejected (a 4x4 fp32 residual and a bf16 y inside it)
    assert f(arr, 2, P + 256, 0, P + 256, 4, 4, 1, S) == SHAPE
    assert f(arr, 2, P + 256, 0, P + 272, 4, 4, 0, S) == SHAPE
    assert f(arr, 2, P + 256, 1, P + 256, 4, 4, 0, S) == SHAPE


@no_gpu
def test_rmsnorm_and_append_validation(lib):
    assert lib.tp_rmsnorm(None, 1, P, P, 4, 8, 1e-5, 1, S) == NULL
    assert lib.tp_rmsnorm(P, 1, P, P, 4, 8, -1.0, 1, S) == SHAPE
    assert lib.tp_rmsnorm(P, 1, P, P, 4, 8, float("nan"), 1, S) == SHAPE
    assert lib.tp_rmsnorm(P, 1, P, P, 0, 8, 1e-5, 1, S) == SHAPE
    assert lib.tp_rmsnorm(P, 1, P, P + 1, 4, 8, 1e-5, 1, S) == ALIGN
    assert lib.tp_rmsnorm(P + 2, 0, P, P, 4, 8, 1e-5, 1, S) == ALIGN   # fp32 x on a 2-byte boundary
    assert lib.tp_rmsnorm(P, 3, P, P, 4, 8, 1e-5, 1, S) == DTYPE
    cs = _s3(2 * 64 * 128, 128, 64 * 128)
    f = lib.tp_kv_append
    assert f(None, P, 256, P, P, cs, 2, 2, 128, 64, 0, 1, S) == NULL
    assert f(P, P, 128, P, P, cs, 2, 2, 128, 64, 0, 1, S) == SHAPE     # row stride < Hkv*D
    assert f(P, P, 256, P, P, cs, 2, 2, 128, 64, -1, 1, S) == SHAPE
    assert f(P, P, 256, P, P, cs, 2, 2, 128, 64, 64, 1, S) == SHAPE    # pos past the cache
    assert f(P, P, 256, P, P, cs, 2, 2, 128, 64, 0, 0, S) == UNSUPPORTED


@no_gpu
def test_fused_entry_validation(lib):
    f = lib.tp_column_linear_act
    assert f(None, P, P, 4, 8, 8, 1, 1, S) == NULL
    assert f(P, P, None, 4, 8, 8, 2, 1, S) == NULL
    assert f(P, P, P, 4, 8, 8, 9, 1, S) == DTYPE             # bad activation
    assert f(P, P, P, 4, 8, 8, 1, 5, S) == DTYPE             # bad dtype
    assert f(P, P, P, 0, 8, 8, 1, 1, S) == SHAPE
    assert f(P, P, P, 4, 8, 0, 1, 1, S) == SHAPE
    assert f(P, P, P, 4, 8, 8, 1, 0, S) == UNSUPPORTED       # fused activations are bf16 only
    assert f(P, P, P, 4, 12, 8, 1, 1, S) == UNSUPPORTED      # K % 8 != 0
    assert f(P + 2, P, P, 4, 8, 8, 1, 1, S) == UNSUPPORTED   # x not 16-byte aligned
    assert f(P + 1, P, P, 4, 8, 8, 1, 1, S) == ALIGN
    assert f(P, P, P, 4, 1 << 20, 1 << 11, 1, 1, S) == UNSUPPORTED   # weight past 32-bit offsets
    g = lib.tp_reduce_partials_rmsnorm
    arr = (ctypes.c_void_p * 2)(P, P)
    assert g(None, 2, None, 1, P, 1, P, P, 4, 8, 1e-5, 1, S) == NULL
    assert g(arr, 2, None, 1, P, 1, None, P, 4, 8, 1e-5, 1, S) == NULL
    assert g(arr, 2, None, 1, P, 1, P, None, 4, 8, 1e-5, 1, S) == NULL
    assert g(arr, 0, None, 1, P, 1, P, P, 4, 8, 1e-5, 1, S) == SHAPE
    assert g(arr, 17, None, 1, P, 1, P, P, 4, 8, 1e-5, 1, S) == SHAPE
    assert g(arr, 2, None, 1, P, 1, P, P, 4, 8, -1.0, 1, S) == SHAPE
    assert g(arr, 2, None, 1, P, 1, P, P, 0, 8, 1e-5, 1, S) == SHAPE
    assert g(arr, 2, None, 1, P, 1, P, P, 4, 8, 1e-5, 4, S) == DTYPE
    assert g(arr, 2, None, 1, P, 4, P, P, 4, 8, 1e-5, 1, S) == DTYPE     # bad y dtype
    assert g(arr, 2, None, 1, P + 1, 1, P, P, 4, 8, 1e-5, 1, S) == ALIGN
    assert g(arr, 2, None, 1, P + 2, 0, P, P, 4, 8, 1e-5, 1, S) == ALIGN   # fp32 y
    odd = (ctypes.c_void_p * 2)(P, P + 2)
    assert g(odd, 2, None, 1, P, 1, P, P, 4, 8, 1e-5, 1, S) == ALIGN
    # a bf16 residual overlapping a float32 y (other than in place, same type)
    assert g(arr, 2, P + 256, 1, P + 256, 0, P, P, 4, 8, 1e-5, 1, S) == SHAPE


def _s2(*v):
    return (ctypes.c_int64 * 2)(*v)


@no_gpu
def test_paged_validation(lib):
    f = lib.tp_paged_attention_decode
    ps = _s3(16 * 2 * 128, 2 * 128, 128)

    def call(q=P, k=P, v=P, ps=ps, nb=64, tbl=P, ts=8, lens=P, maxl=100, bs=16, o=P, B=2, Hq=8,
             Hkv=2, D=128, scale=0.088, dt=1, ws=None, wsb=0):
        return f(q, _s2(1024, 128), k, v, ps, nb, tbl, ts, lens, maxl, bs, o, _s2(1024, 128), B, Hq,
                 Hkv, D, scale, dt, ws, wsb, S)

    assert call(tbl=None) == NULL
    assert call(lens=None) == NULL
    assert call(Hq=6, Hkv=4) == SHAPE
    assert call(nb=0) == SHAPE
    assert call(maxl=0) == SHAPE
    assert call(ts=6) == SHAPE                    # ceil(100 / 16) = 7 entries per row needed
    assert call(bs=24) == UNSUPPORTED             # block size not a multiple of 16
    assert call(bs=8, ts=13) == UNSUPPORTED
    assert call(D=64) == UNSUPPORTED
    assert call(dt=0) == UNSUPPORTED
    assert call(dt=7) == DTYPE
    assert call(Hq=66, Hkv=1) == UNSUPPORTED      # G > 32
    assert call(ps=_s3(16 * 2 * 128, 2 * 128, 100)) == ALIGN
    assert call(tbl=P + 2) == ALIGN
    assert call(k=P + 8) == ALIGN
    need = lib.tp_paged_attention_workspace(1, 8, 2, 4096, 16)
    assert need > 0
    assert call(B=1, maxl=4096, ts=256) == WORKSPACE
    assert lib.tp_paged_attention_workspace(1, 8, 2, 4096, 24) == 0
    g = lib.tp_paged_kv_append
    assert g(None, P, 256, P, P, ps, 64, P, 8, P, 2, 2, 128, 16, 1, S) == NULL
    assert g(P, P, 128, P, P, ps, 64, P, 8, P, 2, 2, 128, 16, 1, S) == SHAPE   # row stride < Hkv*D
    assert g(P, P, 256, P, P, ps, 0, P, 8, P, 2, 2, 128, 16, 1, S) == SHAPE
    assert g(P, P, 256, P, P, ps, 64, P, 8, P, 2, 2, 128, 16, 0, S) == UNSUPPORTED
    assert g(P, P, 256, P, P, ps, 64, P + 2, 8, P, 2, 2, 128, 16, 1, S) == ALIGN


@no_gpu
def test_argmax_validation(lib):
    f = lib.tp_vocab_argmax_local
    assert f(None, 4, 100, 0, P, P, S) == NULL
    assert f(P, 4, 100, 0, None, P, S) == NULL
    assert f(P, 0, 100, 0, P, P, S) == SHAPE
    assert f(P, 4, 0, 0, P, P, S) == SHAPE
    assert f(P, 4, 100, -1, P, P, S) == SHAPE
    assert f(P, 4, 1 << 31, 0, P, P, S) == UNSUPPORTED
    assert f(P + 2, 4, 100, 0, P, P, S) == ALIGN
    assert f(P, 4, 100, 0, P, P + 4, S) == ALIGN              # int64 ids need 8-byte alignment
    g = lib.tp_vocab_argmax_reduce
    va = (ctypes.c_void_p * 2)(P, P)
    assert g(None, va, 2, 4, P, P, S) == NULL
    assert g(va, va, 0, 4, P, P, S) == SHAPE
    assert g(va, va, 65, 4, P, P, S) == SHAPE
    assert g(va, va, 2, 0, P, P, S) == SHAPE
    assert g(va, (ctypes.c_void_p * 2)(P, None), 2, 4, P, P, S) == NULL
    assert g(va, (ctypes.c_void_p * 2)(P, P + 4), 2, 4, P, P, S) == ALIGN
    assert g(va, va, 2, 4, P, P + 4, S) == ALIGN


# ---------------------------------------------------------------------------
# host-side shard slicing of the binding (CPU tensors; pure indexing)
# ---------------------------------------------------------------------------

def test_shard_helpers_match_oracle_slices():
    import oracle.tp_oracle as O
    w = torch.arange(8 * 12, dtype=torch.float32).reshape(8, 12)
    for R in (1, 2, 4):
        for r in range(R):
            assert np.array_equal(tpl.shard_column(w, r, R).numpy(), O.column_shard(w.numpy(), r, R))
            assert np.array_equal(tpl.shard_row(w, r, R).numpy(), O.row_shard(w.numpy(), r, R))
    with pytest.raises(ValueError):
        tpl.shard_column(w, 0, 3)
    with pytest.raises(ValueError):
        tpl.shard_row(w, 0, 5)
    wq, wk, wv = (torch.randn(n * 4, 6) for n in (8, 2, 2))
    for r in range(2):
        assert np.array_equal(tpl.shard_qkv(wq, wk, wv, r, 2, 4).numpy(),
                              O.qkv_shard(wq.numpy(), wk.numpy(), wv.numpy(), r, 2, 4))
    # 2 KV heads over 4 ranks: each KV head replicated on 2 ranks
    for R in (4, 8):
        for r in range(R):
            assert tpl.kv_heads_of_rank(8, 2, r, R) == O.kv_heads_of_rank(8, 2, r, R)
            assert np.array_equal(tpl.shard_qkv(wq, wk, wv, r, R, 4).numpy(),
                                  O.qkv_shard(wq.numpy(), wk.numpy(), wv.numpy(), r, R, 4))
    assert tpl.kv_cache_bytes_per_rank(32, 8, 16, 2, 64, 128) == O.kv_cache_bytes_per_rank(
        32, 8, 16, 2, 64, 128)
    with pytest.raises(ValueError):
        tpl.shard_qkv(wq, wk, wv, 0, 3, 4)     # 8 q heads over 3 ranks
    with pytest.raises(ValueError):
        tpl.kv_heads_of_rank(12, 4, 0, 6)      # 4 KV heads over 6 ranks


def test_binding_rejects_cpu_tensors():
    x = torch.zeros(2, 8, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        tpl.column_linear(x, x)


@no_gpu
def test_decode_attention_append_validation(lib):
    """The fused append + decode attention entry points reject bad arguments on
    the host, before any launch (made-up addresses are never dereferenced)."""
    f = lib.tp_decode_attention_append
    cs = _s3(64 * 2 * 128, 2 * 128, 128)      # [B, T=64, Hkv=2, D=128]

    def call(q=P, qs=_s2(1536, 128), kn=P, vn=P, ns=1536, kc=P, vc=P, cs=cs, T=64, pos=10, o=P,
             os_=_s2(1024, 128), B=2, Hq=8, Hkv=2, D=128, scale=0.088, dt=1, ws=None, wsb=0):
        return f(q, qs, kn, vn, ns, kc, vc, cs, T, pos, o, os_, B, Hq, Hkv, D, scale, dt, ws, wsb, S)

    assert call(q=None) == NULL
    assert call(kn=None) == NULL
    assert call(cs=None) == NULL
    assert call(dt=7) == DTYPE
    assert call(Hq=6, Hkv=4) == SHAPE                 # Hq % Hkv != 0
    assert call(pos=64) == SHAPE                      # past the cache's capacity
    assert call(pos=-1) == SHAPE
    assert call(ns=128) == SHAPE                      # row stride < Hkv*D
    assert call(scale=float("nan")) == SHAPE
    assert call(D=64) == UNSUPPORTED
    assert call(dt=0) == UNSUPPORTED
    assert call(Hq=66, Hkv=1) == UNSUPPORTED          # G > 32
    assert call(cs=_s3(64 * 2 * 128, 2 * 128 + 4, 128)) == ALIGN
    assert call(ns=1540) == ALIGN
    assert call(kn=P + 2) == ALIGN
    assert call(qs=_s2(1536, 100)) == ALIGN
    # one sequence, long span: split-key path, workspace required
    need = lib.tp_local_attention_workspace(1, 1, 4096, 8, 2, 128)
    assert need > 0
    big = _s3(4096 * 2 * 128, 2 * 128, 128)
    assert call(B=1, T=4096, pos=4095, cs=big) == WORKSPACE
    assert call(B=1, T=4096, pos=4095, cs=big, ws=P, wsb=need - 1) == WORKSPACE

    # the allocation-free form: the same host validation (these cases all fail
    # before the library's buffer is looked up or anything is launched)
    h = lib.tp_decode_attention_append_noalloc

    def ncall(q=P, kn=P, cs=cs, pos=10, Hq=8, Hkv=2, D=128, dt=1, ns=1536):
        return h(q, _s2(1536, 128), kn, P, ns, P, P, cs, 64, pos, P, _s2(1024, 128), 2, Hq, Hkv, D,
                 0.088, dt, S)

    assert ncall(q=None) == NULL
    assert ncall(dt=7) == DTYPE
    assert ncall(Hq=6, Hkv=4) == SHAPE
    assert ncall(pos=64) == SHAPE
    assert ncall(ns=128) == SHAPE
    assert ncall(Hq=66, Hkv=1) == UNSUPPORTED
    assert ncall(D=64) == UNSUPPORTED
    assert ncall(kn=P + 2) == ALIGN

    g = lib.tp_paged_decode_attention_append
    ps = _s3(16 * 2 * 128, 2 * 128, 128)

    def pcall(kn=P, vn=P, ns=1536, ts=8, Hq=8, Hkv=2, maxl=100, B=2, ws=None, wsb=0):
        return g(P, _s2(1536, 128), kn, vn, ns, P, P, ps, 64, P, ts, P, maxl, 16, P, _s2(1024, 128),
                 B, Hq, Hkv, 128, 0.088, 1, ws, wsb, S)

    assert pcall(kn=None) == NULL
    assert pcall(ns=128) == SHAPE
    assert pcall(ns=1540) == ALIGN
    assert pcall(vn=P + 8) == ALIGN
    assert pcall(ts=6) == SHAPE                       # table rows shorter than max_context_len needs
    assert pcall(Hq=66, Hkv=1) == UNSUPPORTED
    assert pcall(B=1, maxl=4096, ts=256) == WORKSPACE
