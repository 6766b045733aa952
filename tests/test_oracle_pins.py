"""Pins for the CPU oracle: values the pages print, closed forms, invariants of
the method and brute force on tiny inputs.  CPU only (no GPU, no HIP library).

Sources:
  P1 "Tensor Parallel：当一张 GPU 放不下一个大模型" (mini vLLM series)
  P2 "张量并行（Tensor Parallelism）推理部署实战：从 Megatron-LM 切分原理到 vLLM 多卡配置与性能调优"
  P3 "Tensor Parallel 深入解析：多加 GPU，推理为什么可能更慢"
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle.tp_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _worked():
    with open(os.path.join(GOLDEN, "worked_example.json")) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# Worked example (P3 "两张卡如何共同算出一层")
# ---------------------------------------------------------------------------

def check_worked_example():
    g = _worked()
    X = np.array(g["X"], np.float64)
    w = np.array(g["W"], np.float64).T          # stored [out, in]
    v = np.array(g["V"], np.float64).T
    assert np.array_equal(O.linear(X, w), np.array(g["Y_full"]))
    shards = [O.column_linear(X, O.column_shard(w, r, 2)) for r in range(2)]
    for r in range(2):
        assert np.array_equal(shards[r], np.array(g["Y_col_shards"][r]))
    parts = [O.row_linear_partial(shards[r], O.row_shard(v, r, 2)) for r in range(2)]
    for r in range(2):
        assert np.array_equal(parts[r], np.array(g["row_partials"][r]))
    assert np.array_equal(O.reduce_partials(parts), np.array(g["Y_sum"]))
    assert np.array_equal(O.concat_columns(shards), np.array(g["Y_full"]))


def test_worked_example():
    check_worked_example()


# ---------------------------------------------------------------------------
# Matmul core against pure-Python loops
# ---------------------------------------------------------------------------

def _loop_matmul(x, w):
    M, K = len(x), len(x[0])
    N = len(w)
    out = [[0.0] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            s = 0.0
            for k in range(K):
                s += x[i][k] * w[j][k]
            out[i][j] = s
    return np.array(out)


def check_linear_bruteforce():
    rng = np.random.default_rng(7)
    for (M, K, N) in [(1, 2, 4), (2, 3, 5), (5, 17, 3), (3, 64, 17)]:
        x = rng.integers(-3, 4, (M, K)).astype(np.float64)
        w = rng.integers(-3, 4, (N, K)).astype(np.float64)
        assert np.array_equal(O.linear(x, w), _loop_matmul(x.tolist(), w.tolist()))
        # non-square, non-symmetric case catches a transposed operand
        assert O.linear(x, w).shape == (M, N)


def test_linear_bruteforce():
    check_linear_bruteforce()


# ---------------------------------------------------------------------------
# Sharding invariants (P1 "如何验证 tensor parallel 正确": concat of column
# shards equals the full linear, the sum of row partials equals the full linear)
# ---------------------------------------------------------------------------

def check_sharding_invariants():
    rng = np.random.default_rng(11)
    M, K, N = 5, 64, 48
    x = rng.integers(-3, 4, (M, K)).astype(np.float64)
    w = rng.integers(-3, 4, (N, K)).astype(np.float64)
    full = _loop_matmul(x.tolist(), w.tolist())
    for R in (1, 2, 4, 8):
        cols = [O.column_linear(x, O.column_shard(w, r, R)) for r in range(R)]
        assert np.array_equal(O.concat_columns(cols), full)
        parts = [O.row_linear_partial(O.input_shard(x, r, R), O.row_shard(w, r, R))
                 for r in range(R)]
        assert np.array_equal(O.reduce_partials(parts), full)


def test_sharding_invariants():
    check_sharding_invariants()


def test_indivisible_shards_rejected():
    w = np.zeros((6, 4))
    with pytest.raises(ValueError):
        O.column_shard(w, 0, 4)
    with pytest.raises(ValueError):
        O.row_shard(w, 0, 3)
    with pytest.raises(ValueError):
        O.qkv_shard(np.zeros((8 * 2, 4)), np.zeros((3 * 2, 4)), np.zeros((3 * 2, 4)), 0, 2, 2)


def check_toy_mlp_bitexact():
    """Config toy_mlp_int shapes: X[4,64], W1 64->256 column split, W2 256->64
    row split, no activation; integer values in {-3..3}, so every partial sum
    is an integer below 2**24 and the result is exact in any order."""
    rng = np.random.default_rng(101)
    x = rng.integers(-3, 4, (4, 64)).astype(np.float64)
    w1 = rng.integers(-3, 4, (256, 64)).astype(np.float64)
    w2 = rng.integers(-3, 4, (64, 256)).astype(np.float64)
    full = _loop_matmul(_loop_matmul(x.tolist(), w1.tolist()).tolist(), w2.tolist())
    assert np.array_equal(O.mlp_unsharded(x, w1, w2, "none"), full)
    parts = [O.mlp_rank_partial(x, w1, w2, "none", r, 2) for r in range(2)]
    assert np.array_equal(O.reduce_partials(parts), full)
    assert np.max(np.abs(full)) < 2 ** 24


def test_toy_mlp_bitexact():
    check_toy_mlp_bitexact()


def test_reduce_order_and_residual():
    p = [np.array([[1.0, 2.0]]), np.array([[10.0, 20.0]]), np.array([[100.0, 200.0]])]
    assert np.array_equal(O.reduce_partials(p), [[111.0, 222.0]])
    assert np.array_equal(O.reduce_partials(p, residual=np.array([[0.5, -0.5]])),
                          [[111.5, 221.5]])
    # rank order: (1e16 + 1) - 1e16 is 0 in double, 1e16 - 1e16 + 1 is 1
    q = [np.array([1e16]), np.array([1.0]), np.array([-1e16])]
    assert O.reduce_partials(q)[0] == 0.0
    q2 = [np.array([1e16]), np.array([-1e16]), np.array([1.0])]
    assert O.reduce_partials(q2)[0] == 1.0


# ---------------------------------------------------------------------------
# Activations: textbook values and symmetries
# ---------------------------------------------------------------------------

PHI_1 = 0.8413447460685429     # standard normal CDF at 1 (textbook table)
PHI_2 = 0.9772498680518208     # standard normal CDF at 2
PHI_M10 = 7.6198530241605e-24  # standard normal CDF at -10 (upper tail at 10)


def check_activations():
    assert O.silu(0.0) == 0.0 and O.gelu(0.0) == 0.0
    # sigmoid(ln 3) = 3/4 exactly
    assert math.isclose(float(O.silu(math.log(3.0))), 0.75 * math.log(3.0), rel_tol=1e-15)
    assert math.isclose(float(O.gelu(1.0)), PHI_1, rel_tol=1e-15)
    assert math.isclose(float(O.gelu(2.0)), 2 * PHI_2, rel_tol=1e-15)
    assert math.isclose(float(O.gelu(-1.0)), -(1 - PHI_1), rel_tol=1e-14)
    # far tail: full relative accuracy where 1 + erf(.) would cancel to 0
    assert math.isclose(float(O.gelu(-10.0)), -10.0 * PHI_M10, rel_tol=1e-10)
    x = np.linspace(-6, 6, 101)
    # f(x) - f(-x) = x for both (sigma(x)+sigma(-x)=1, Phi(x)+Phi(-x)=1)
    assert np.allclose(O.silu(x) - O.silu(-x), x, atol=1e-14)
    assert np.allclose(O.gelu(x) - O.gelu(-x), x, atol=1e-14)
    assert abs(float(O.gelu(40.0)) - 40.0) < 1e-12 and abs(float(O.silu(60.0)) - 60.0) < 1e-12
    g = np.array([1.0, -2.0]); u = np.array([3.0, 5.0])
    assert np.allclose(O.local_activation(g, u, "swiglu"), O.silu(g) * u)
    assert np.array_equal(O.local_activation(g, None, "none"), g)
    # the GELU dispatch against textbook normal-CDF values (independent of gelu())
    got = O.local_activation(np.array([1.0, 2.0, -1.0, -10.0, 0.0]), None, "gelu")
    want = np.array([PHI_1, 2 * PHI_2, -(1 - PHI_1), -10.0 * PHI_M10, 0.0])
    assert np.allclose(got, want, rtol=1e-10, atol=0.0)
    # and the SwiGLU dispatch against sigma(ln 3) = 3/4
    assert math.isclose(float(O.local_activation(np.array([math.log(3.0)]), np.array([2.0]),
                                                 "swiglu")[0]), 1.5 * math.log(3.0), rel_tol=1e-15)


def test_activations():
    check_activations()


# ---------------------------------------------------------------------------
# RMSNorm: closed forms (not on the pages; these pins are all it has)
# ---------------------------------------------------------------------------

def check_rmsnorm():
    y = O.rmsnorm(np.array([[3.0, 4.0]]), np.ones(2), eps=0.0)
    assert np.allclose(y, np.array([[3.0, 4.0]]) / math.sqrt(12.5), rtol=1e-15)
    c = -2.5
    y = O.rmsnorm(np.full((1, 8), c), np.full(8, 1.5), eps=1e-5)
    assert np.allclose(y, 1.5 * c / math.sqrt(c * c + 1e-5), rtol=1e-15)
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, 32))
    y = O.rmsnorm(x, np.ones(32), eps=0.0)
    assert np.allclose(np.mean(y * y, axis=-1), 1.0, rtol=1e-14)
    assert np.allclose(O.rmsnorm(7.0 * x, np.ones(32), 0.0), y, rtol=1e-14)
    gamma = rng.standard_normal(32)
    assert np.allclose(O.rmsnorm(x, gamma, 0.0), y * gamma, rtol=1e-14)


def test_rmsnorm():
    check_rmsnorm()


# ---------------------------------------------------------------------------
# Attention: closed forms and brute force
# ---------------------------------------------------------------------------

def _loop_attention(q, k, v, causal):
    B, Sq, Hq, D = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    out = np.zeros_like(q)
    for b in range(B):
        for s in range(Sq):
            pos = s + Skv - Sq
            for h in range(Hq):
                hk = h // G
                sc = []
                for t in range(Skv):
                    if causal and t > pos:
                        continue
                    sc.append((t, sum(q[b, s, h, d] * k[b, t, hk, d] for d in range(D)) / math.sqrt(D)))
                mx = max(val for _, val in sc)
                ws = [(t, math.exp(val - mx)) for t, val in sc]
                tot = sum(wv for _, wv in ws)
                for d in range(D):
                    out[b, s, h, d] = sum(wv * v[b, t, hk, d] for t, wv in ws) / tot
    return out


def check_attention():
    rng = np.random.default_rng(5)
    # one key -> output is that key's value
    q = rng.standard_normal((2, 1, 4, 8)); k = rng.standard_normal((2, 1, 2, 8))
    v = rng.standard_normal((2, 1, 2, 8))
    o = O.attention(q, k, v, causal=False)
    for h in range(4):
        assert np.allclose(o[:, 0, h], v[:, 0, h // 2], rtol=1e-15)
    # zero query -> uniform weights -> mean of visible values
    q = np.zeros((1, 5, 2, 4)); k = rng.standard_normal((1, 5, 1, 4))
    v = rng.standard_normal((1, 5, 1, 4))
    o = O.attention(q, k, v, causal=True)
    for s in range(5):
        assert np.allclose(o[0, s, 0], v[0, :s + 1, 0].mean(axis=0), rtol=1e-13)
        assert np.allclose(o[0, s, 1], v[0, :s + 1, 0].mean(axis=0), rtol=1e-13)
    # first causal row sees only key 0
    q = rng.standard_normal((1, 6, 2, 4)); k = rng.standard_normal((1, 6, 2, 4))
    v = rng.standard_normal((1, 6, 2, 4))
    o = O.attention(q, k, v, causal=True)
    assert np.array_equal(o[0, 0], v[0, 0])
    # two keys, scale 1/sqrt(D): D=4, q=(a,0,0,0), k0=0, k1=(1,0,0,0): p1 = sigmoid(a/2);
    # a = 2 ln 3 gives p1 = 3/4 exactly
    a = 2 * math.log(3.0)
    q = np.zeros((1, 1, 1, 4)); q[0, 0, 0, 0] = a
    k = np.zeros((1, 2, 1, 4)); k[0, 1, 0, 0] = 1.0
    v = np.zeros((1, 2, 1, 4)); v[0, 1, 0, :] = 1.0
    o = O.attention(q, k, v, causal=False)
    assert np.allclose(o[0, 0, 0], 0.75, rtol=1e-14)
    # GQA map: constant value c_j per KV head j, query head h must return c_{h // G}
    Hq, Hkv = 8, 2
    q = rng.standard_normal((1, 3, Hq, 4)); k = rng.standard_normal((1, 7, Hkv, 4))
    v = np.zeros((1, 7, Hkv, 4))
    for j in range(Hkv):
        v[:, :, j, :] = 10.0 * (j + 1)
    o = O.attention(q, k, v, causal=True)
    for h in range(Hq):
        assert np.allclose(o[0, :, h, :], 10.0 * (h // (Hq // Hkv) + 1), rtol=1e-14)
    # weights sum to one: all-ones values give all-ones output
    o = O.attention(q, k, np.ones_like(v), causal=False)
    assert np.allclose(o, 1.0, rtol=1e-14)
    # a dominant key takes all the weight
    k = rng.standard_normal((1, 4, 1, 4)); v = rng.standard_normal((1, 4, 1, 4))
    q = 500.0 * k[:, 2:3] / np.linalg.norm(k[0, 2, 0])
    o = O.attention(q, k, v, causal=False)
    assert np.allclose(o[0, 0, 0], v[0, 2, 0], atol=1e-6)
    # brute force on tiny shapes, MHA and GQA, causal and not, Sq < Skv
    for (B, Sq, Skv, Hq, Hkv, D) in [(1, 3, 3, 2, 2, 4), (2, 2, 5, 4, 2, 3), (1, 4, 4, 6, 3, 5)]:
        q = rng.standard_normal((B, Sq, Hq, D)); k = rng.standard_normal((B, Skv, Hkv, D))
        v = rng.standard_normal((B, Skv, Hkv, D))
        for causal in (False, True):
            assert np.allclose(O.attention(q, k, v, causal), _loop_attention(q, k, v, causal),
                               rtol=1e-12, atol=1e-13)


def test_attention():
    check_attention()


def test_attention_rows_subset():
    rng = np.random.default_rng(9)
    q = rng.standard_normal((1, 9, 4, 8)); k = rng.standard_normal((1, 9, 2, 8))
    v = rng.standard_normal((1, 9, 2, 8))
    full = O.attention(q, k, v, causal=True)
    rows = np.array([0, 4, 8])
    sub = O.attention(q[:, rows], k, v, causal=True, q_pos=rows)
    assert np.allclose(sub, full[:, rows], rtol=1e-14)


# ---------------------------------------------------------------------------
# Whole layer: sharded == unsharded (P1 "如何验证 tensor parallel 正确": TP=1
# and TP=N must agree; layered check column -> row -> attention -> MLP -> full)
# ---------------------------------------------------------------------------

def _small_layer(rng, H=32, n_q=8, n_kv=4, D=8, I=64):
    return {
        "g1": 1.0 + 0.1 * rng.standard_normal(H), "g2": 1.0 + 0.1 * rng.standard_normal(H),
        "wq": 0.2 * rng.standard_normal((n_q * D, H)), "wk": 0.2 * rng.standard_normal((n_kv * D, H)),
        "wv": 0.2 * rng.standard_normal((n_kv * D, H)), "wo": 0.2 * rng.standard_normal((H, n_q * D)),
        "wg": 0.2 * rng.standard_normal((I, H)), "wu": 0.2 * rng.standard_normal((I, H)),
        "wd": 0.2 * rng.standard_normal((H, I)),
    }


def check_layer_sharded_equals_unsharded():
    rng = np.random.default_rng(21)
    p = _small_layer(rng)
    x = rng.standard_normal((10, 32))
    ref = O.layer_unsharded(x, p, 8, 1e-5)
    for R in (1, 2, 4):
        y, h, pa, pm = O.layer_sharded(x, p, 8, 1e-5, R)
        assert len(pa) == R and len(pm) == R
        assert np.allclose(y, ref, rtol=1e-11, atol=1e-11)
    rows = np.array([0, 3, 9])
    assert np.allclose(O.layer_unsharded(x, p, 8, 1e-5, rows=rows), ref[rows], rtol=1e-12)
    y, *_ = O.layer_sharded(x, p, 8, 1e-5, 2, rows=rows)
    assert np.allclose(y, ref[rows], rtol=1e-11, atol=1e-11)
    # the layer is not trivially the residual
    assert np.max(np.abs(ref - x)) > 0.1


def test_layer_sharded_equals_unsharded():
    check_layer_sharded_equals_unsharded()


def test_gelu_mlp_sharded_equals_unsharded():
    rng = np.random.default_rng(23)
    x = rng.standard_normal((6, 16)); a = rng.standard_normal((64, 16)); b = rng.standard_normal((16, 64))
    ref = O.mlp_unsharded(x, a, b, "gelu")
    for R in (1, 2, 4, 8):
        y = O.reduce_partials([O.mlp_rank_partial(x, a, b, "gelu", r, R) for r in range(R)])
        assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_layer_attention_block_matches_bruteforce():
    """The attention block wiring (QKV split, GQA, o_proj) against loops."""
    rng = np.random.default_rng(29)
    p = _small_layer(rng, H=8, n_q=4, n_kv=2, D=2, I=8)
    x = rng.standard_normal((4, 8))
    q = (x @ p["wq"].T).reshape(1, 4, 4, 2)
    k = (x @ p["wk"].T).reshape(1, 4, 2, 2)
    v = (x @ p["wv"].T).reshape(1, 4, 2, 2)
    o = _loop_attention(q, k, v, causal=True).reshape(4, 8)
    ref = _loop_matmul(o.tolist(), p["wo"].tolist())
    assert np.allclose(O.attention_block_unsharded(x, p["wq"], p["wk"], p["wv"], p["wo"], 2), ref,
                       rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------------------
# GQA with fewer KV heads than ranks (P3 "权重变小，不代表所有显存都按比例变小":
# 32 q / 8 KV heads; from TP 8 to TP 16 the q heads keep halving per rank but
# the KV heads per rank do not; vLLM's QKVParallelLinear replicates them)
# ---------------------------------------------------------------------------

def check_gqa_replication():
    # the page's structural example
    per = {R: len(O.kv_heads_of_rank(32, 8, 0, R)) for R in (1, 2, 4, 8, 16, 32)}
    assert per == {1: 8, 2: 4, 4: 2, 8: 1, 16: 1, 32: 1}
    b8 = O.kv_cache_bytes_per_rank(32, 8, 8, 4, 1024, 128)
    assert b8 == 2 * 4 * 1024 * 1 * 128 * 2
    assert O.kv_cache_bytes_per_rank(32, 8, 16, 4, 1024, 128) == b8        # no longer halves
    assert O.kv_cache_bytes_per_rank(32, 8, 4, 4, 1024, 128) == 2 * b8
    # TP 16: ranks 2k and 2k+1 hold KV head k; every KV head is held; each
    # rank's q heads (2 of them) read the KV head it holds
    for R, rep in ((16, 2), (32, 4)):
        held = [O.kv_heads_of_rank(32, 8, r, R) for r in range(R)]
        assert all(len(h) == 1 for h in held)
        assert [h[0] for h in held] == [r // rep for r in range(R)]
        hq = 32 // R
        for r in range(R):
            assert {j // 4 for j in range(r * hq, (r + 1) * hq)} == set(held[r])
    # sharded == unsharded with replicated KV heads (the Σ of rank partials
    # is the unsharded block only if every rank reads the right KV head)
    rng = np.random.default_rng(31)
    H, D, n_q, n_kv = 16, 4, 8, 2
    wq = rng.standard_normal((n_q * D, H)); wk = rng.standard_normal((n_kv * D, H))
    wv = rng.standard_normal((n_kv * D, H)); wo = rng.standard_normal((H, n_q * D))
    x = rng.standard_normal((5, H))
    ref = O.attention_block_unsharded(x, wq, wk, wv, wo, D)
    for R in (1, 2, 4, 8):
        parts = [O.attention_rank_partial(x, wq, wk, wv, wo, D, r, R) for r in range(R)]
        assert np.allclose(O.reduce_partials(parts), ref, rtol=1e-12, atol=1e-12)
    # the replicated slice is the KV head's rows of wk / wv
    w = O.qkv_shard(wq, wk, wv, 5, 8, D)
    assert w.shape == ((1 + 2) * D, H)
    assert np.array_equal(w[:D], wq[5 * D:6 * D])
    assert np.array_equal(w[D:2 * D], wk[D:2 * D]) and np.array_equal(w[2 * D:], wv[D:2 * D])   # q head 5 -> KV head 5 // 4
    for bad in ((8, 3, 4), (8, 4, 6), (6, 2, 4)):
        with pytest.raises(ValueError):
            O.kv_heads_of_rank(bad[0], bad[1], 0, bad[2])


def test_gqa_replication():
    check_gqa_replication()


# ---------------------------------------------------------------------------
# Paged KV cache (P1 "Tensor parallel 对 KV cache 的影响")
# ---------------------------------------------------------------------------

def check_paged_attention():
    rng = np.random.default_rng(43)
    B, Hq, Hkv, D, bs, L = 3, 4, 2, 8, 4, 10
    nblk = (L + bs - 1) // bs
    kc = rng.standard_normal((B, L, Hkv, D)); vc = rng.standard_normal((B, L, Hkv, D))
    q = rng.standard_normal((B, Hq, D))
    lens = [10, 1, 7]
    ref = np.stack([O.attention(q[b][None, None], kc[b:b + 1, :lens[b]], vc[b:b + 1, :lens[b]],
                                causal=True)[0, 0] for b in range(B)])
    # identity layout: sequence b owns blocks b*nblk .. b*nblk + nblk - 1
    pad = nblk * bs
    kp = np.zeros((B * nblk, bs, Hkv, D)); vp = np.zeros_like(kp)
    for b in range(B):
        kk = np.zeros((pad, Hkv, D)); vv = np.zeros((pad, Hkv, D))
        kk[:L] = kc[b]; vv[:L] = vc[b]
        kp[b * nblk:(b + 1) * nblk] = kk.reshape(nblk, bs, Hkv, D)
        vp[b * nblk:(b + 1) * nblk] = vv.reshape(nblk, bs, Hkv, D)
    table = [[b * nblk + i for i in range(nblk)] for b in range(B)]
    assert np.allclose(O.paged_decode_attention(q, kp, vp, table, lens, bs), ref, rtol=1e-13, atol=1e-14)
    # shuffled physical blocks (and spare blocks of garbage) give the same result
    perm = rng.permutation(B * nblk + 5)
    kp2 = np.full((B * nblk + 5, bs, Hkv, D), np.nan); vp2 = np.full_like(kp2, np.nan)
    table2 = [[int(perm[b * nblk + i]) for i in range(nblk)] for b in range(B)]
    for b in range(B):
        for i in range(nblk):
            kp2[table2[b][i]] = kp[table[b][i]]; vp2[table2[b][i]] = vp[table[b][i]]
    assert np.allclose(O.paged_decode_attention(q, kp2, vp2, table2, lens, bs), ref, rtol=1e-13,
                       atol=1e-14)
    # heads split over ranks, one block table: each rank's pool holds its KV
    # heads; the ranks' outputs over their q heads make up the whole
    for R in (1, 2):
        parts = []
        for r in range(R):
            hk = O.kv_heads_of_rank(Hq, Hkv, r, R)
            hq = list(range(r * Hq // R, (r + 1) * Hq // R))
            parts.append(O.paged_decode_attention(q[:, hq], kp2[:, :, hk], vp2[:, :, hk], table2, lens, bs))
        assert np.allclose(np.concatenate(parts, axis=1), ref, rtol=1e-13, atol=1e-14)
    # append then attend: the new token is the last key
    kn = rng.standard_normal((B, Hkv, D)); vn = rng.standard_normal((B, Hkv, D))
    lens3 = [11, 2, 8]
    table3 = [[*row, int(perm[-1 - b])] for b, row in enumerate(table2)]   # a 4th block each
    kp3, vp3 = O.paged_append(kp2, vp2, kn, vn, table3, lens3, bs)
    assert np.array_equal(kp3[table3[0][2], 2], kn[0]) and np.array_equal(vp3[table3[1][0], 1], vn[1])
    assert np.array_equal(kp3[table3[2][1], 3], kn[2])


def test_paged_attention():
    check_paged_attention()


# ---------------------------------------------------------------------------
# Vocab-parallel greedy argmax (P1 "lm_head 怎么处理")
# ---------------------------------------------------------------------------

def _loop_argmax(row, offset):
    best_v, best_i = -math.inf, None
    for j, z in enumerate(row):
        z = -math.inf if math.isnan(z) else z
        if best_i is None or z > best_v:
            best_v, best_i = z, j
    return best_v, best_i + offset


def check_vocab_argmax():
    rng = np.random.default_rng(41)
    z = rng.standard_normal((6, 37))
    z[1, 30] = z[1, 5] = z[1].max() + 1.0              # tie: the lower id wins
    z[2, :] = np.nan; z[2, 11] = -np.inf                # no number but -inf at 11
    z[3, :] = np.nan                                    # nothing: id 0, value -inf
    z[4, 0] = np.nan; z[4, 9] = 50.0                    # NaN never wins
    z[5, 3] = -0.0; z[5, :] = np.minimum(z[5, :], -1.0); z[5, 3] = -0.0; z[5, 8] = 0.0   # -0 == +0
    v, i = O.vocab_argmax_local(z, 100)
    for m in range(6):
        lv, li = _loop_argmax(z[m], 100)
        assert v[m] == lv and i[m] == li, (m, v[m], i[m], lv, li)
    assert i[1] == 105 and i[2] == 100 and i[3] == 100 and i[4] == 109 and i[5] == 103
    # sharding the vocab and combining the ranks' pairs gives the full argmax,
    # including maxima tied across ranks (the lower rank's block wins)
    V = 48
    z = rng.standard_normal((5, V))
    z[0, 7] = z[0, 40] = 9.0
    z[1, 13] = z[1, 12] = 9.0
    z[2, 47] = 9.0
    for R in (1, 2, 3, 4, 8, 16):
        b = V // R
        pairs = [O.vocab_argmax_local(z[:, r * b:(r + 1) * b], r * b) for r in range(R)]
        gv, gi = O.vocab_argmax_reduce([p[0] for p in pairs], [p[1] for p in pairs])
        fv, fi = O.vocab_argmax_local(z, 0)
        assert np.array_equal(gi, fi) and np.array_equal(gv, fv)
        assert gi[0] == 7 and gi[1] == 12 and gi[2] == 47
    # end to end through the lm_head: integer-valued h and W with duplicated
    # vocab rows (equal logits in different ranks' blocks)
    h = rng.integers(-3, 4, (4, 16)).astype(np.float64)
    w = rng.integers(-3, 4, (32, 16)).astype(np.float64)
    w[25] = w[3] = 3.0 * np.sign(h[0] + 0.5)            # the same, largest logit for row 0
    for R in (1, 2, 4, 8):
        sv, si = O.greedy_token_sharded(h, w, R)
        fv, fi = O.greedy_token(h, w)
        assert np.array_equal(si, fi) and np.array_equal(sv, fv)
    assert fi[0] == 3


def test_vocab_argmax():
    check_vocab_argmax()


# ---------------------------------------------------------------------------
# bf16 rounding used by the storage-faithful mode
# ---------------------------------------------------------------------------

def test_bf16_storage_policy():
    """The diagnostic storage policy rounds exactly the named intermediates."""
    a = np.array([1.0 + 2.0 ** -8 + 2.0 ** -20, -3.0000001])
    everything = O.bf16_storage()
    only_a = O.bf16_storage("a")
    for name in O.STORED:
        assert np.array_equal(everything(name, a), O.round_bf16(a))
        assert np.array_equal(only_a(name, a), O.round_bf16(a) if name == "a" else a)
    with pytest.raises(ValueError):
        O.bf16_storage("g")
    with pytest.raises(ValueError):
        only_a("u", a)
    # in a layer, rounding nothing equals the exact default; rounding the
    # activation changes the MLP partial by at most its bf16 rounding through Wd
    rng = np.random.default_rng(5)
    x = rng.standard_normal((3, 16)); wg = rng.standard_normal((8, 16)) / 4
    wu = rng.standard_normal((8, 16)) / 4; wd = rng.standard_normal((16, 8)) / 4
    exact = O.mlp_rank_partial(x, wg, wd, "swiglu", 0, 1, w_up=wu)
    assert np.array_equal(O.mlp_rank_partial(x, wg, wd, "swiglu", 0, 1, w_up=wu,
                                             store=O.bf16_storage("xn")), exact)
    a_exact = O.local_activation(x @ wg.T, x @ wu.T, "swiglu")
    stored = O.mlp_rank_partial(x, wg, wd, "swiglu", 0, 1, w_up=wu, store=O.bf16_storage("a"))
    assert np.allclose(stored, O.round_bf16(a_exact) @ wd.T, rtol=0, atol=1e-12)
    assert not np.array_equal(stored, exact)


def test_round_bf16():
    assert O.round_bf16(1.0 + 2.0 ** -8) == 1.0                      # tie -> even
    assert O.round_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6      # tie -> even (up)
    assert O.round_bf16(1.0 + 2.0 ** -8 + 2.0 ** -20) == 1.0 + 2.0 ** -7
    assert O.round_bf16(-3.0) == -3.0 and O.round_bf16(0.0) == 0.0
    rng = np.random.default_rng(0)
    a = rng.standard_normal(100000).astype(np.float32)
    ref = torch.from_numpy(a).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.round_bf16(a.astype(np.float64)), ref)


# ---------------------------------------------------------------------------
# Planted mistakes: each plausible slip in the oracle must trip a pin above
# ---------------------------------------------------------------------------

def _mut_linear_transposed(x, w):
    x = np.asarray(x, np.float64); w = np.asarray(w, np.float64)
    return x @ w.reshape(w.shape[1], w.shape[0])


def _mut_row_shard_wrong_axis(w, r, R):
    w = np.asarray(w)
    b = w.shape[0] // R
    return w[r * b:(r + 1) * b, :]


def _mut_reduce_drops_residual(partials, residual=None):
    acc = np.zeros_like(np.asarray(partials[0], np.float64))
    for p in partials:
        acc = acc + p
    return acc


def _mut_reduce_skips_last(partials, residual=None):
    acc = np.zeros_like(np.asarray(partials[0], np.float64))
    for p in partials[:-1]:
        acc = acc + p
    return acc if residual is None else acc + residual


def _mut_gelu_sign(g):
    g = np.asarray(g, np.float64)
    from scipy.special import erf
    return 0.5 * g * (1.0 - erf(g / math.sqrt(2.0)))


def _mut_silu(g):
    g = np.asarray(g, np.float64)
    return g / (1.0 + np.exp(g))


def _mut_rmsnorm_sum(x, gamma, eps):
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps) * gamma


def _mut_rmsnorm_no_gamma(x, gamma, eps):
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


_orig_attention = O.attention


def _mut_attention_gqa_modulo(q, k, v, causal, scale=None, q_pos=None):
    # q head h reads KV head h % Hkv instead of h // G
    Hq, Hkv = q.shape[2], k.shape[2]
    perm = [h % Hkv for h in range(Hq)]
    G = Hq // Hkv
    kk = np.stack([k[:, :, perm[h], :] for h in range(Hq)], axis=2)
    vv = np.stack([v[:, :, perm[h], :] for h in range(Hq)], axis=2)
    return _orig_attention(q, kk, vv, causal, scale, q_pos)


def _mut_attention_no_scale(q, k, v, causal, scale=None, q_pos=None):
    return _orig_attention(q, k, v, causal, 1.0, q_pos)


def _mut_attention_mask_off_by_one(q, k, v, causal, scale=None, q_pos=None):
    Sq, Skv = q.shape[1], k.shape[1]
    if q_pos is None:
        q_pos = np.arange(Sq) + (Skv - Sq)
    return _orig_attention(q, k, v, causal, scale, np.minimum(np.asarray(q_pos) + 1, Skv - 1))


_orig_qkv_shard = O.qkv_shard


def _mut_qkv_order(wq, wk, wv, r, R, head_dim):
    return _orig_qkv_shard(wq, wv, wk, r, R, head_dim)


_orig_kv_heads = O.kv_heads_of_rank


def _mut_kv_heads_modulo(n_q, n_kv, r, R):
    # replicated ranks take KV head r % Hkv instead of the head their q heads read
    if n_kv % R == 0:
        return _orig_kv_heads(n_q, n_kv, r, R)
    return [r % n_kv]


def _mut_argmax_last(logits, vocab_offset=0):
    z = np.asarray(logits, np.float64)
    z = np.where(np.isnan(z), -np.inf, z)
    n = z.shape[-1]
    j = n - 1 - np.argmax(z[..., ::-1], axis=-1)          # last maximum instead of the first
    return np.take_along_axis(z, j[..., None], axis=-1)[..., 0], j.astype(np.int64) + vocab_offset


def _mut_argmax_nan_wins(logits, vocab_offset=0):
    z = np.asarray(logits, np.float64)
    j = np.argmax(z, axis=-1)                             # numpy's argmax picks a NaN
    return np.take_along_axis(z, j[..., None], axis=-1)[..., 0], j.astype(np.int64) + vocab_offset


def _mut_reduce_later_rank(vals, ids):
    best_v = np.array(vals[0], np.float64); best_i = np.array(ids[0], np.int64)
    for v, i in zip(vals[1:], ids[1:]):
        take = np.asarray(v) >= best_v
        best_v = np.where(take, v, best_v); best_i = np.where(take, i, best_i)
    return best_v, best_i


def _mut_paged_swapped(pool, table_row, length, block_size):
    pool = np.asarray(pool, np.float64)
    n = len(table_row)
    rows = [pool[int(table_row[t % n]), (t // n) % block_size] for t in range(length)]
    return np.stack(rows, axis=0)


_orig_local_activation = O.local_activation


def _mut_activation_gelu_as_silu(g, u=None, act="swiglu"):
    # the GELU branch dispatching to SiLU
    return O.silu(g) if act == "gelu" else _orig_local_activation(g, u, act)


MUTATIONS = [
    ("local_activation", _mut_activation_gelu_as_silu),
    ("paged_gather", _mut_paged_swapped),
    ("kv_heads_of_rank", _mut_kv_heads_modulo),
    ("vocab_argmax_local", _mut_argmax_last),
    ("vocab_argmax_local", _mut_argmax_nan_wins),
    ("vocab_argmax_reduce", _mut_reduce_later_rank),
    ("linear", _mut_linear_transposed),
    ("row_shard", _mut_row_shard_wrong_axis),
    ("reduce_partials", _mut_reduce_drops_residual),
    ("reduce_partials", _mut_reduce_skips_last),
    ("gelu", _mut_gelu_sign),
    ("silu", _mut_silu),
    ("rmsnorm", _mut_rmsnorm_sum),
    ("rmsnorm", _mut_rmsnorm_no_gamma),
    ("attention", _mut_attention_gqa_modulo),
    ("attention", _mut_attention_no_scale),
    ("attention", _mut_attention_mask_off_by_one),
    ("qkv_shard", _mut_qkv_order),
]

ALL_CHECKS = [check_worked_example, check_linear_bruteforce, check_sharding_invariants,
              check_toy_mlp_bitexact, check_activations, check_rmsnorm, check_attention,
              check_layer_sharded_equals_unsharded, check_gqa_replication, check_vocab_argmax,
              check_paged_attention]


@pytest.mark.parametrize("name,fn", MUTATIONS, ids=[f"{n}:{f.__name__}" for n, f in MUTATIONS])
def test_planted_mistake_is_caught(monkeypatch, name, fn):
    monkeypatch.setattr(O, name, fn)
    caught = False
    for chk in ALL_CHECKS:
        try:
            chk()
        except (AssertionError, ValueError, IndexError):
            caught = True
            break
    assert caught, f"no pin catches the planted mistake in {name}"
