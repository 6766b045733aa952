"""CPU float64 oracle for one tensor-parallel rank's share of a decoder layer.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import this module.  It shares no code with
the HIP library (no kernels, headers, helpers or tables) and imports nothing
from it; inputs reach it as plain float64 numpy arrays.

Everything is written as the plain definition of what the method computes,
with numpy's matmul, exp and scipy's erfc as the only library primitives:
no blocking, fusion or reordering.

Sources (web pages; each function names the section it follows):
  P1  "Tensor Parallel：当一张 GPU 放不下一个大模型" (mini vLLM series)
  P2  "张量并行（Tensor Parallelism）推理部署实战：从 Megatron-LM 切分原理到 vLLM
       多卡配置与性能调优"
  P3  "Tensor Parallel 深入解析：多加 GPU，推理为什么可能更慢"

Conventions (readings where the pages leave a choice open):
  * ``Y = X W`` with X ``[tokens, in]``.  Weights are stored as ``nn.Linear``
    stores them, ``w = W^T`` of shape ``[out, in]`` (P2 section 1.1/1.2
    sketches; P3 "两张卡如何共同算出一层" notes frameworks may keep the
    transpose).  ``linear(x, w) = x @ w.T``.
  * Shards are contiguous blocks in rank order (P1 "Attention 里的 tensor
    parallel": heads 0..7 on GPU 0, 8..15 on GPU 1, ...; P3: left/right halves).
  * A fused local QKV weight stacks the rank's q heads, then its k heads, then
    its v heads, each head ``D`` consecutive output features.
  * GQA: global q head j reads KV head ``j // (Hq/Hkv)``; with contiguous
    sharding local q head h reads local KV head ``h // (Hq_l/Hkv_l)``.  With
    fewer KV heads than ranks each rank keeps one replicated KV head.
  * Attention scale ``1/sqrt(D)``; causal masking aligned at the end of the key
    span (key t is visible to query position p iff t <= p); softmax with the
    row maximum subtracted.
  * No positional encoding (the pages never specify one); no bias; dropout is
    the identity at inference (P2 section 二).
  * RMSNorm ``x * (mean(x^2) + eps)^(-1/2) * gamma`` -- not on the pages,
    parity unpinned by them (pinned here by closed forms only).
  * GELU is the exact (erf/erfc) form, ``g * Phi(g)``, not the tanh approximation.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erfc as _erfc

__all__ = [
    "round_bf16", "bf16_storage", "STORED", "linear", "column_shard", "row_shard", "input_shard",
    "column_linear", "row_linear_partial", "reduce_partials", "concat_columns",
    "silu", "gelu", "local_activation", "rmsnorm", "attention", "qkv_shard",
    "kv_heads_of_rank", "kv_cache_bytes_per_rank", "vocab_argmax_local", "vocab_argmax_reduce",
    "greedy_token", "greedy_token_sharded", "paged_gather", "paged_decode_attention",
    "paged_append",
    "mlp_unsharded", "mlp_rank_partial", "attention_block_unsharded",
    "attention_rank_partial", "layer_unsharded", "layer_sharded",
]


def _exact(name: str, a):
    """The default storage policy: every intermediate is kept exactly."""
    return np.asarray(a, np.float64)


# ---------------------------------------------------------------------------
# bf16 storage rounding (used only by the storage-faithful diagnostic mode)
# ---------------------------------------------------------------------------

def round_bf16(a) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value, ties to even.

    bfloat16 keeps 8 significant bits: with ``a = m * 2**e`` and
    ``0.5 <= |m| < 1`` the result is ``rint(m * 2**8) * 2**(e - 8)``.
    """
    a = np.asarray(a, dtype=np.float64)
    m, e = np.frexp(a)
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)


# Named intermediates of the layer, in the order the layer produces them:
# xn (first pre-norm), qkv (the projections q, k, v), o (attention output),
# h (the residual stream after the attention sub-block), hn (second pre-norm),
# gu (the gate/up or fc1 projections), a (the activation).
STORED = ("xn", "qkv", "o", "h", "hn", "gu", "a")


def bf16_storage(*names):
    """A storage policy for the diagnostic mode: the named intermediates
    (default: all of ``STORED``) are rounded to bfloat16 where an
    implementation stores them, every other one is kept exactly.  A policy is
    called as ``store(name, value)``."""
    chosen = frozenset(names or STORED)
    unknown = chosen - set(STORED)
    if unknown:
        raise ValueError(f"unknown intermediates {sorted(unknown)}")

    def store(name: str, a):
        if name not in STORED:
            raise ValueError(f"unknown intermediate {name!r}")
        return round_bf16(a) if name in chosen else np.asarray(a, np.float64)
    return store


# ---------------------------------------------------------------------------
# Linear layers and their shards (P1 "Column Parallel Linear：按输出维度切",
# "Row Parallel Linear：按输入维度切"; P2 sections 1.1 and 1.2; P3
# "两张卡如何共同算出一层")
# ---------------------------------------------------------------------------

def linear(x, w):
    """Unsharded ``Y = X W`` with ``w = W^T`` stored ``[out, in]``."""
    return np.asarray(x, np.float64) @ np.asarray(w, np.float64).T


def _block(n: int, r: int, R: int) -> slice:
    if R <= 0 or not (0 <= r < R):
        raise ValueError(f"rank {r} out of range for TP size {R}")
    if n % R != 0:
        raise ValueError(f"dimension {n} is not divisible by TP size {R}")
    b = n // R
    return slice(r * b, (r + 1) * b)


def column_shard(w, r: int, R: int):
    """Rank r's block of output features: rows ``[r*N/R, (r+1)*N/R)`` of the
    stored ``[N, K]`` weight (the column block of the math W)."""
    w = np.asarray(w)
    return w[_block(w.shape[0], r, R), :]


def row_shard(w, r: int, R: int):
    """Rank r's block of input features: columns ``[r*K/R, (r+1)*K/R)`` of the
    stored ``[N, K]`` weight (the row block of the math W)."""
    w = np.asarray(w)
    return w[:, _block(w.shape[1], r, R)]


def input_shard(x, r: int, R: int):
    """Rank r's block of the last dimension of an activation."""
    x = np.asarray(x)
    return x[..., _block(x.shape[-1], r, R)]


def column_linear(x, w_shard):
    """Column-parallel linear on one rank: the full input times the rank's
    output block gives the rank's output slice ``Y_r = X W_r``; no exchange."""
    return linear(x, w_shard)


def row_linear_partial(x_shard, w_shard):
    """Row-parallel linear on one rank: the rank's input slice times the rank's
    input block gives a partial sum of the full output ``Y_r = X_r W_r``."""
    return linear(x_shard, w_shard)


def concat_columns(parts):
    """Reassemble column-parallel outputs: ``Y = [Y_0, Y_1, ...]``."""
    return np.concatenate([np.asarray(p, np.float64) for p in parts], axis=-1)


def reduce_partials(partials, residual=None):
    """The arithmetic of the all-reduce: ``Y = sum_r Y_r``, taken in rank order
    0..R-1, plus an optional residual added once after the sum."""
    acc = np.zeros_like(np.asarray(partials[0], np.float64))
    for p in partials:
        acc = acc + np.asarray(p, np.float64)
    if residual is not None:
        acc = acc + np.asarray(residual, np.float64)
    return acc


# ---------------------------------------------------------------------------
# Local elementwise work (P1 "MLP 里的 tensor parallel": activation(gate_i) *
# up_i is rank-local; P2 section 二: GELU between fc1 and fc2)
# ---------------------------------------------------------------------------

def silu(g):
    g = np.asarray(g, np.float64)
    return g / (1.0 + np.exp(-g))


def gelu(g):
    """``g * Phi(g)`` with the standard normal CDF ``Phi(g) = erfc(-g/sqrt 2)/2``
    (equal to ``(1 + erf(g/sqrt 2))/2``; the erfc form does not cancel for
    negative g)."""
    g = np.asarray(g, np.float64)
    return 0.5 * g * _erfc(-g / math.sqrt(2.0))


def local_activation(g, u=None, act: str = "swiglu"):
    """``swiglu``: SiLU(gate) * up;  ``gelu``: GELU(g);  ``none``: g."""
    if act == "swiglu":
        return silu(g) * np.asarray(u, np.float64)
    if act == "gelu":
        return gelu(g)
    if act == "none":
        return np.asarray(g, np.float64)
    raise ValueError(f"unknown activation {act!r}")


def rmsnorm(x, gamma, eps: float):
    """Row-wise RMS normalisation with a learned scale (pre-norm)."""
    x = np.asarray(x, np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(gamma, np.float64)


# ---------------------------------------------------------------------------
# Attention over the rank's local heads (P1 "Attention 里的 tensor parallel";
# P2 section 2.1; GQA placement: P3 "权重变小，不代表所有显存都按比例变小")
# ---------------------------------------------------------------------------

def attention(q, k, v, causal: bool, scale: float | None = None, q_pos=None):
    """Scaled dot-product attention with grouped KV heads.

    q ``[B, Sq, Hq, D]``, k/v ``[B, Skv, Hkv, D]`` -> o ``[B, Sq, Hq, D]``.
    q head h reads KV head ``h // (Hq // Hkv)``.  ``q_pos[s]`` is the absolute
    position of query row s (default: the last Sq positions of the key span);
    with ``causal`` key t is visible to row s iff ``t <= q_pos[s]``.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, Sq, Hq, D = q.shape
    _, Skv, Hkv, _ = k.shape
    if Hq % Hkv != 0:
        raise ValueError("q heads must be a multiple of KV heads")
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if q_pos is None:
        q_pos = np.arange(Sq) + (Skv - Sq)
    q_pos = np.asarray(q_pos)
    visible = np.arange(Skv)[None, :] <= q_pos[:, None]          # [Sq, Skv]
    out = np.empty_like(q)
    for b in range(B):
        for h in range(Hq):
            hk = h // G
            s = (q[b, :, h, :] @ k[b, :, hk, :].T) * scale        # [Sq, Skv]
            if causal:
                s = np.where(visible, s, -np.inf)
            s = s - np.max(s, axis=-1, keepdims=True)
            p = np.exp(s)
            p = p / np.sum(p, axis=-1, keepdims=True)
            out[b, :, h, :] = p @ v[b, :, hk, :]
    return out


def kv_heads_of_rank(n_q: int, n_kv: int, r: int, R: int):
    """The KV heads rank r holds, as a list of global KV head ids.

    The q heads are split into R contiguous blocks (P1 "Attention 里的 tensor
    parallel").  When the KV heads divide by R they are split the same way.
    When there are fewer KV heads than ranks (P3 "权重变小，不代表所有显存都按
    比例变小": 32 q / 8 KV heads at TP 16), KV heads cannot be split further:
    each rank keeps the one KV head its q heads read, j // (Hq/Hkv) for its
    q heads j, so every KV head is replicated on R / Hkv ranks.  This needs
    R % Hkv == 0, so that a rank's q heads all fall in one KV group."""
    if n_q % R:
        raise ValueError("q heads must divide by the TP size")
    if n_q % n_kv:
        raise ValueError("q heads must be a multiple of KV heads")
    if n_kv % R == 0:
        c = n_kv // R
        return list(range(r * c, (r + 1) * c))
    if R % n_kv:
        raise ValueError("KV heads must divide by the TP size or the TP size by the KV heads")
    hq = n_q // R
    group = n_q // n_kv
    heads = sorted({j // group for j in range(r * hq, (r + 1) * hq)})
    assert len(heads) == 1
    return heads


def kv_cache_bytes_per_rank(n_q: int, n_kv: int, R: int, batch: int, kv_len: int,
                            head_dim: int, elem_bytes: int = 2) -> int:
    """Bytes of K and V cache one rank keeps for ``batch`` sequences of
    ``kv_len`` keys (P3: the KV cache is stored per the actual head layout, so
    it stops shrinking once every rank holds a single replicated KV head)."""
    return 2 * batch * kv_len * len(kv_heads_of_rank(n_q, n_kv, 0, R)) * head_dim * elem_bytes


def qkv_shard(wq, wk, wv, r: int, R: int, head_dim: int):
    """Rank r's fused QKV weight ``[(Hq_l + 2*Hkv_l)*D, H]``: its block of q
    heads, then its KV heads for k, then for v (a replicated KV head when
    there are fewer KV heads than ranks; see ``kv_heads_of_rank``)."""
    wq, wk, wv = (np.asarray(a) for a in (wq, wk, wv))
    for a in (wq, wk, wv):
        if a.shape[0] % head_dim != 0:
            raise ValueError("projection rows must be whole heads")
    n_q, n_kv = wq.shape[0] // head_dim, wk.shape[0] // head_dim
    heads = kv_heads_of_rank(n_q, n_kv, r, R)
    kv_rows = np.concatenate([np.arange(j * head_dim, (j + 1) * head_dim) for j in heads])
    return np.concatenate([column_shard(wq, r, R), wk[kv_rows], wv[kv_rows]], axis=0)


# ---------------------------------------------------------------------------
# Paged KV cache (P1 "Tensor parallel 对 KV cache 的影响": each rank's KV pool
# holds only its own heads; the block table is the same on every rank)
# ---------------------------------------------------------------------------

def paged_gather(pool, table_row, length: int, block_size: int):
    """The first ``length`` key rows of one sequence, ``[length, Hkv, D]``:
    key t is slot ``t % block_size`` of physical block
    ``table_row[t // block_size]`` of ``pool [num_blocks, block_size, Hkv, D]``."""
    pool = np.asarray(pool, np.float64)
    rows = [pool[int(table_row[t // block_size]), t % block_size] for t in range(length)]
    return np.stack(rows, axis=0)


def paged_decode_attention(q, k_pool, v_pool, table, lens, block_size: int, scale=None):
    """Decode attention (one query token per sequence, seeing all its keys)
    over a paged cache.  q ``[B, Hq, D]`` -> o ``[B, Hq, D]``."""
    q = np.asarray(q, np.float64)
    B, Hq, D = q.shape
    out = np.zeros_like(q)
    for b in range(B):
        L = int(lens[b])
        k = paged_gather(k_pool, table[b], L, block_size)
        v = paged_gather(v_pool, table[b], L, block_size)
        out[b] = attention(q[b][None, None], k[None], v[None], causal=True, scale=scale)[0, 0]
    return out


def paged_append(k_pool, v_pool, k_new, v_new, table, lens, block_size: int):
    """Copies of the pools with each sequence's new k/v ``[B, Hkv, D]`` stored
    at position ``lens[b] - 1``."""
    kp = np.array(k_pool, np.float64); vp = np.array(v_pool, np.float64)
    for b in range(len(lens)):
        t = int(lens[b]) - 1
        blk = int(table[b][t // block_size])
        kp[blk, t % block_size] = k_new[b]
        vp[blk, t % block_size] = v_new[b]
    return kp, vp


# ---------------------------------------------------------------------------
# Vocab-parallel lm_head, greedy decoding (P1 "lm_head 怎么处理": the lm_head
# is split by vocab, column-parallel; each rank takes its largest logit and an
# all-gather / all-reduce picks the global one)
# ---------------------------------------------------------------------------

def vocab_argmax_local(logits, vocab_offset: int = 0):
    """Per row: the largest logit of the rank's vocab block and its global
    vocab id.  Reading where the page is silent: a NaN logit counts as -inf,
    and equal logits go to the lowest vocab id (numpy's argmax returns the
    first maximum)."""
    z = np.asarray(logits, np.float64)
    z = np.where(np.isnan(z), -np.inf, z)
    j = np.argmax(z, axis=-1)
    return np.take_along_axis(z, j[..., None], axis=-1)[..., 0], j.astype(np.int64) + vocab_offset


def vocab_argmax_reduce(vals, ids):
    """The exchange: the ranks' (value, id) pairs, combined rank by rank; a
    larger value wins, an equal value keeps the lower id."""
    best_v = np.array(vals[0], np.float64)
    best_i = np.array(ids[0], np.int64)
    for v, i in zip(vals[1:], ids[1:]):
        v = np.asarray(v, np.float64); i = np.asarray(i, np.int64)
        take = (v > best_v) | ((v == best_v) & (i < best_i))
        best_v = np.where(take, v, best_v)
        best_i = np.where(take, i, best_i)
    return best_v, best_i


def greedy_token(h, w_vocab):
    """Unsharded greedy choice: argmax over the full vocab of ``h W^T``."""
    return vocab_argmax_local(linear(h, w_vocab), 0)


def greedy_token_sharded(h, w_vocab, R: int):
    """The same choice made the vocab-parallel way: rank r's logits over its
    contiguous vocab block, its local argmax, then the combine over ranks."""
    V = np.asarray(w_vocab).shape[0]
    pairs = [vocab_argmax_local(column_linear(h, column_shard(w_vocab, r, R)), r * (V // R))
             for r in range(R)]
    return vocab_argmax_reduce([p[0] for p in pairs], [p[1] for p in pairs])


# ---------------------------------------------------------------------------
# MLP block (P1 "MLP 里的 tensor parallel"; P2 section 二 MegatronMLP)
# ---------------------------------------------------------------------------

def mlp_unsharded(x, w_in, w_out, act: str, w_up=None):
    """Unsharded MLP.  gated: ``(act(x Wg) * (x Wu)) Wd``; gelu: ``GELU(x A) B``;
    none: ``(x A) B``.  ``w_in`` is the gate (or fc1) weight."""
    g = linear(x, w_in)
    u = linear(x, w_up) if act == "swiglu" else None
    return linear(local_activation(g, u, act), w_out)


def mlp_rank_partial(x, w_in, w_out, act: str, r: int, R: int, w_up=None,
                     store=_exact):
    """Rank r's MLP share: column-parallel gate/up (or fc1), the local
    activation on the rank's intermediate slice, row-parallel down (or fc2)
    giving the rank's partial of the hidden output.  ``store`` (a policy from
    ``bf16_storage``) is applied to the named intermediates ``gu`` and ``a``."""
    g = store("gu", column_linear(x, column_shard(w_in, r, R)))
    u = store("gu", column_linear(x, column_shard(w_up, r, R))) if act == "swiglu" else None
    a = store("a", local_activation(g, u, act))
    return row_linear_partial(a, row_shard(w_out, r, R))


# ---------------------------------------------------------------------------
# Attention block and the pre-norm decoder layer
# ---------------------------------------------------------------------------

def _split_heads(a, n_heads: int, head_dim: int):
    M = a.shape[0]
    return a.reshape(1, M, n_heads, head_dim)


def attention_block_unsharded(x, wq, wk, wv, wo, head_dim: int, causal: bool = True,
                              rows=None):
    """Unsharded multi-head (GQA) attention block ``attn(x) Wo`` over one
    sequence ``x [S, H]``.  ``rows`` selects which query rows to return (all
    keys are always used)."""
    S = x.shape[0]
    n_q, n_kv = wq.shape[0] // head_dim, wk.shape[0] // head_dim
    k = _split_heads(linear(x, wk), n_kv, head_dim)
    v = _split_heads(linear(x, wv), n_kv, head_dim)
    rows = np.arange(S) if rows is None else np.asarray(rows)
    q = _split_heads(linear(x[rows], wq), n_q, head_dim)
    o = attention(q, k, v, causal=causal, q_pos=rows)
    return linear(o.reshape(len(rows), n_q * head_dim), wo)


def attention_rank_partial(x, wq, wk, wv, wo, head_dim: int, r: int, R: int,
                           causal: bool = True, rows=None, store=_exact):
    """Rank r's attention share: its fused QKV slice (column-parallel), local
    attention over its q heads and their KV heads, its o_proj input block
    (row-parallel) giving a partial of the hidden output."""
    S = x.shape[0]
    n_q, n_kv = wq.shape[0] // head_dim, wk.shape[0] // head_dim
    hq, hkv = n_q // R, len(kv_heads_of_rank(n_q, n_kv, r, R))
    wqkv = qkv_shard(wq, wk, wv, r, R, head_dim)
    dq, dkv = hq * head_dim, hkv * head_dim
    kv = store("qkv", column_linear(x, wqkv[dq:, :]))
    k = _split_heads(kv[:, :dkv], hkv, head_dim)
    v = _split_heads(kv[:, dkv:], hkv, head_dim)
    rows = np.arange(S) if rows is None else np.asarray(rows)
    q = _split_heads(store("qkv", column_linear(x[rows], wqkv[:dq, :])), hq, head_dim)
    o = store("o", attention(q, k, v, causal=causal, q_pos=rows))
    return row_linear_partial(o.reshape(len(rows), dq), row_shard(wo, r, R))


def layer_unsharded(x, p: dict, head_dim: int, eps: float, act: str = "swiglu",
                    rows=None):
    """Pre-norm decoder layer on one sequence, unsharded:
    ``h = x + attn(rmsnorm(x))``, ``y = h + mlp(rmsnorm(h))``.
    ``p`` holds g1, wq, wk, wv, wo, g2, wg, wu, wd.  Returns y at ``rows``."""
    x = np.asarray(x, np.float64)
    rows = np.arange(x.shape[0]) if rows is None else np.asarray(rows)
    xn = rmsnorm(x, p["g1"], eps)
    h = x[rows] + attention_block_unsharded(xn, p["wq"], p["wk"], p["wv"], p["wo"],
                                            head_dim, causal=True, rows=rows)
    hn = rmsnorm(h, p["g2"], eps)
    return h + mlp_unsharded(hn, p["wg"], p["wd"], act, w_up=p.get("wu"))


def layer_sharded(x, p: dict, head_dim: int, eps: float, R: int, act: str = "swiglu",
                  rows=None, store=_exact):
    """The same layer computed the tensor-parallel way: every rank's attention
    partial, their sum plus the residual, every rank's MLP partial on the
    normalised sum, their sum plus the residual (two all-reduces per layer:
    P2 section 2.1 table; P3 "两张卡如何共同算出一层").  Returns
    ``(y, h, attn_partials, mlp_partials)`` at ``rows``."""
    x = np.asarray(x, np.float64)
    rows = np.arange(x.shape[0]) if rows is None else np.asarray(rows)
    xn = store("xn", rmsnorm(x, p["g1"], eps))
    pa = [attention_rank_partial(xn, p["wq"], p["wk"], p["wv"], p["wo"], head_dim,
                                 r, R, causal=True, rows=rows, store=store)
          for r in range(R)]
    h = store("h", reduce_partials(pa, residual=x[rows]))
    hn = store("hn", rmsnorm(h, p["g2"], eps))
    pm = [mlp_rank_partial(hn, p["wg"], p["wd"], act, r, R, w_up=p.get("wu"),
                           store=store) for r in range(R)]
    y = reduce_partials(pm, residual=h)
    return y, h, pa, pm
