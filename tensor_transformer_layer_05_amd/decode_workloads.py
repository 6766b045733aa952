"""Seeded decode-shard workloads: the weights, caches and library calls of one
decode step of each shard, shared by the benchmark (timings) and the
hardware-counter driver (HBM bytes), so both measure the same launches.
Setup only: every step is a library call; no arithmetic of the method here.

Each builder returns a ``Workload``: ``steps[j]()`` issues one step on
rotating copy ``j`` of the weights and caches (copies are separate device
buffers; a builder takes at least as many copies as make up ``span`` bytes,
twice the 256 MB Infinity Cache by default, so that the rotation cannot be
served from it), ``bytes`` the algorithmic HBM bytes of one step (each
operand read once, each result written once), ``flops`` its arithmetic.
"""
from __future__ import annotations

import math

from dataclasses import dataclass, field

import numpy as np
import torch

from . import inputs as I
from . import kv_cache_bytes_per_rank, kv_heads_of_rank, shard_qkv, shard_row
from .shard import AttnShard, MlpShard, VocabShard

DEV = "cuda:0"
SPAN = 2 * 256 * 2**20   # bytes a rotation of copies covers at least


def _copies(copies: int, byts: float, span: float) -> int:
    return max(copies, math.ceil(span / byts)) if span > 0 else copies


@dataclass
class Workload:
    name: str
    steps: list
    bytes: float
    flops: float
    extra: dict = field(default_factory=dict)


def mlp_tp8(M: int, copies: int, span: float = SPAN) -> Workload:
    """Rank 0's decode MLP shard at TP 8 (hidden 8192, 3584 local
    intermediate, SwiGLU fused into the gate|up projection)."""
    c = I.config("decode_mlp_tp8")
    H, il = c.hidden, c.inter // c.tp
    wg = I.normal(c.seed, "wg", (il, H), c.w_std).dev
    wu = I.normal(c.seed, "wu", (il, H), c.w_std).dev
    wd = I.normal(c.seed, "wd", (H, il), c.w_std).dev
    wgu = torch.cat([wg, wu], 0)
    # weights once, x read, act(g)*u written and read back, fp32 partial written
    byts = (wgu.numel() + wd.numel()) * 2 + M * H * 2 + M * il * 2 * 2 + M * H * 4
    copies = _copies(copies, byts, span)
    mlps = [MlpShard(wgu.to(DEV), wd.to(DEV), "swiglu", 64) for _ in range(copies)]
    X = I.normal(c.seed, "x", (M, H)).dev.to(DEV)
    Ps = [torch.empty((M, H), dtype=torch.float32, device=DEV) for _ in range(copies)]
    steps = [(lambda j=j: mlps[j].partial(X, Ps[j])) for j in range(copies)]
    return Workload(f"mlp_tp8_M{M}", steps, byts, 2.0 * M * (H * 2 * il + il * H))


def attn_tp4(copies: int, span: float = SPAN) -> Workload:
    """Rank 0's decode attention shard at TP 4 (8 q / 2 KV heads of 128, batch
    32, 2048 keys, cache [B, Hkv, L, D]): QKV, append + attention, o_proj."""
    c = I.config("decode_attn_tp4")
    H, R, D, B, L = c.hidden, c.tp, c.head_dim, c.batch, c.kv_len
    hq, hkv = c.n_q // R, c.n_kv // R
    x = I.normal(c.seed, "x", (B, H)).dev.to(DEV)
    wqkv = I.normal(c.seed, "wqkv", ((hq + 2 * hkv) * D, H), c.w_std).dev
    wo = I.normal(c.seed, "wo", (H, hq * D), c.w_std).dev
    kc = I.normal(c.seed, "kcache", (B, hkv, L, D)).dev
    vc = I.normal(c.seed, "vcache", (B, hkv, L, D)).dev
    byts = (wqkv.numel() + wo.numel() + kc.numel() + vc.numel()) * 2 + B * H * 2 + B * H * 4
    copies = _copies(copies, byts, span)
    sets = [(AttnShard(wqkv.to(DEV), wo.to(DEV), hq, hkv, D, B), kc.to(DEV), vc.to(DEV),
             torch.empty((B, H), dtype=torch.float32, device=DEV)) for _ in range(copies)]

    def step(j):
        a, k_, v_, P = sets[j]
        a.decode_partial(x, k_.transpose(1, 2), v_.transpose(1, 2), L - 1, P)

    fl = 2.0 * B * H * (hq + 2 * hkv) * D + 4.0 * B * hq * L * D + 2.0 * B * hq * D * H
    return Workload("attn_tp4_B32_L2048", [(lambda j=j: step(j)) for j in range(copies)], byts, fl)


def attn_tp16_rep(copies: int, span: float = SPAN) -> Workload:
    """Rank 0's decode attention shard when KV heads are replicated (32 q / 8
    KV heads at TP 16: 2 q heads and one KV head per rank)."""
    c = I.config("decode_attn_tp16_rep")
    H, R, D, B, L = c.hidden, c.tp, c.head_dim, c.batch, c.kv_len
    hq = c.n_q // R
    heads = kv_heads_of_rank(c.n_q, c.n_kv, 0, R)
    x = I.normal(c.seed, "x", (B, H)).dev.to(DEV)
    wq = I.normal(c.seed, "wq", (c.n_q * D, H), c.w_std).dev
    wk = I.normal(c.seed, "wk", (c.n_kv * D, H), c.w_std).dev
    wv = I.normal(c.seed, "wv", (c.n_kv * D, H), c.w_std).dev
    wo = I.normal(c.seed, "wo", (H, c.n_q * D), c.w_std).dev
    wqkv = shard_qkv(wq, wk, wv, 0, R, D)
    wo0 = shard_row(wo, 0, R)
    kc = I.normal(c.seed, "kcache", (B, c.n_kv, L, D)).dev[:, heads[0]:heads[0] + 1].contiguous()
    vc = I.normal(c.seed, "vcache", (B, c.n_kv, L, D)).dev[:, heads[0]:heads[0] + 1].contiguous()
    byts = (wqkv.numel() + wo0.numel() + kc.numel() + vc.numel()) * 2 + B * H * 2 + B * H * 4
    copies = _copies(copies, byts, span)
    sets = [(AttnShard(wqkv.to(DEV), wo0.to(DEV), hq, len(heads), D, B), kc.to(DEV), vc.to(DEV),
             torch.empty((B, H), dtype=torch.float32, device=DEV)) for _ in range(copies)]

    def step(j):
        a, k_, v_, P = sets[j]
        a.decode_partial(x, k_.transpose(1, 2), v_.transpose(1, 2), L - 1, P)

    fl = 2.0 * B * H * wqkv.shape[0] + 4.0 * B * hq * L * D + 2.0 * B * hq * D * H
    return Workload("attn_tp16_rep_B32_L2048", [(lambda j=j: step(j)) for j in range(copies)], byts, fl,
                    {"kv_cache_bytes_per_rank": kv_cache_bytes_per_rank(c.n_q, c.n_kv, R, B, L, D)})


def attn_tp4_paged(copies: int, span: float = SPAN, bs: int = 16) -> Workload:
    """The TP 4 decode attention shard with a paged cache: block size 16,
    physical blocks shuffled, every sequence at the full 2048 keys."""
    c = I.config("decode_attn_tp4")
    H, R, D, B, L = c.hidden, c.tp, c.head_dim, c.batch, c.kv_len
    hq, hkv = c.n_q // R, c.n_kv // R
    nblk = L // bs
    x = I.normal(c.seed, "x", (B, H)).dev.to(DEV)
    wqkv = I.normal(c.seed, "wqkv", ((hq + 2 * hkv) * D, H), c.w_std).dev
    wo = I.normal(c.seed, "wo", (H, hq * D), c.w_std).dev
    kc = I.normal(c.seed, "kcache", (B * nblk, bs, hkv, D)).dev
    vc = I.normal(c.seed, "vcache", (B * nblk, bs, hkv, D)).dev
    table = torch.from_numpy(np.random.default_rng(c.seed).permutation(B * nblk).astype(np.int32))
    table = table.reshape(B, nblk).to(DEV)
    lens = torch.full((B,), L, dtype=torch.int32, device=DEV)
    byts = (wqkv.numel() + wo.numel() + kc.numel() + vc.numel()) * 2 + B * H * 2 + B * H * 4
    copies = _copies(copies, byts, span)
    sets = [(AttnShard(wqkv.to(DEV), wo.to(DEV), hq, hkv, D, B), kc.to(DEV), vc.to(DEV),
             torch.empty((B, H), dtype=torch.float32, device=DEV)) for _ in range(copies)]

    def step(j):
        a, k_, v_, P = sets[j]
        a.decode_partial_paged(x, k_, v_, table, lens, L, P)

    fl = 2.0 * B * H * (hq + 2 * hkv) * D + 4.0 * B * hq * L * D + 2.0 * B * hq * D * H
    return Workload("attn_tp4_paged_B32_L2048", [(lambda j=j: step(j)) for j in range(copies)], byts, fl)


def lm_head_tp8(M: int, copies: int, span: float = SPAN) -> Workload:
    """Rank 0's vocab-parallel lm_head shard with its local greedy argmax
    (128256-token vocab at TP 8: 16032 x 8192 bf16 rows, 263 MB per copy)."""
    c = I.config("lm_head_tp8")
    H, R, V = c.hidden, c.tp, c.extra["vocab"]
    b = V // R
    w = I.normal(c.seed, "w", (b, H), c.w_std, rank=0).dev
    byts = b * H * 2 + M * H * 2 + M * b * 4 * 2 + M * 12
    copies = _copies(copies, byts, span)
    shards = [VocabShard(w.to(DEV), 0, M) for _ in range(copies)]
    h = I.normal(c.seed, "h", (M, H)).dev.to(DEV)
    return Workload(f"lm_head_tp8_M{M}", [(lambda j=j: shards[j].local_greedy(h)) for j in range(copies)],
                    byts, 2.0 * M * H * b)


DECODE_NAMES = ["mlp_tp8_M1", "mlp_tp8_M8", "mlp_tp8_M64", "attn_tp4_B32_L2048",
                "attn_tp16_rep_B32_L2048", "attn_tp4_paged_B32_L2048", "lm_head_tp8_M1",
                "lm_head_tp8_M8"]


def all_decode(copies: int = 4, span: float = SPAN):
    """Every decode shard in the benchmark's order, built one at a time (the
    caller drops each before the next is built), each with at least
    ``copies`` copies and enough of them to cover ``span`` bytes."""
    for M in (1, 8, 64):
        yield lambda M=M: mlp_tp8(M, copies, span)
    yield lambda: attn_tp4(copies, span)
    yield lambda: attn_tp16_rep(copies, span)
    yield lambda: attn_tp4_paged(copies, span)
    for M in (1, 8):
        yield lambda M=M: lm_head_tp8(M, copies, span)
