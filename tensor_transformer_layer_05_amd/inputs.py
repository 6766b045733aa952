"""Seeded synthetic inputs shared by the HIP path's tests/bench and the CPU oracle.

This module draws random numbers and rounds them to the storage type; it holds
none of the tensor-parallel method's arithmetic (no products, no activations,
no sums of partials).  Both sides receive exactly the same values: the GPU side
gets the bf16 (or fp32) tensor, the oracle gets the same values widened to
float64 (the widening of a bf16 value is exact).

Weights are stored the way ``nn.Linear`` stores them, ``[out_features,
in_features]`` with the input dimension contiguous, which is the layout of the
ColumnParallelLinear / RowParallelLinear sketches in section 1.1 / 1.2 of the
page "张量并行（Tensor Parallelism）推理部署实战：从 Megatron-LM 切分原理到 vLLM 多卡配置与性能调优".
The mathematical weight of ``Y = X W`` is the transpose of what is stored.

Every weight is generated per TP rank block from a seed derived from
(config seed, tensor name, rank), so one rank's shard can be drawn without
drawing the others, and the unsharded matrix is the concatenation of the rank
blocks (row blocks for column-parallel weights, column blocks for row-parallel
weights).
"""
from __future__ import annotations

import zlib
from dataclasses import dataclass, field

import numpy as np
import torch

__all__ = [
    "Tensor2",
    "normal",
    "uniform_int",
    "CONFIGS",
    "config",
]


@dataclass
class Tensor2:
    """One synthetic tensor in two forms: ``dev`` (storage dtype, CPU torch
    tensor, to be moved to the GPU) and ``ref`` (float64 numpy, same values)."""

    dev: torch.Tensor
    ref: np.ndarray


def _rng(seed: int, name: str, rank: int = 0) -> np.random.Generator:
    tag = zlib.crc32(name.encode("utf-8"))
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tag, rank])))


def _to_storage(a32: np.ndarray, dtype: torch.dtype) -> Tensor2:
    t = torch.from_numpy(np.ascontiguousarray(a32))
    if dtype == torch.bfloat16:
        t = t.to(torch.bfloat16)  # round to nearest even
    elif dtype != torch.float32:
        raise ValueError(f"unsupported storage dtype {dtype}")
    ref = t.to(torch.float64).numpy()
    return Tensor2(dev=t, ref=ref)


def normal(seed: int, name: str, shape, std: float = 1.0, dtype=torch.bfloat16,
           rank: int = 0) -> Tensor2:
    """N(0, std^2) values rounded to ``dtype``."""
    g = _rng(seed, name, rank)
    a = g.standard_normal(size=tuple(shape), dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return _to_storage(a, dtype)


def uniform_int(seed: int, name: str, shape, lo: int = -3, hi: int = 3,
                dtype=torch.float32, rank: int = 0) -> Tensor2:
    """Integers drawn uniformly from {lo..hi}, stored exactly in ``dtype``."""
    g = _rng(seed, name, rank)
    a = g.integers(lo, hi + 1, size=tuple(shape)).astype(np.float32)
    return _to_storage(a, dtype)


# ---------------------------------------------------------------------------
# Workload definitions (shapes, sizes and distributions only).
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class Config:
    name: str
    seed: int
    tp: int                     # R, the tensor-parallel size
    hidden: int                 # H
    tokens: tuple = ()          # M values (decode) or (S,) for prefill
    inter: int = 0              # full intermediate size (0: no MLP)
    n_q: int = 0                # full number of q heads (0: no attention)
    n_kv: int = 0               # full number of KV heads
    head_dim: int = 0
    kv_len: int = 0             # decode KV span including the current token
    batch: int = 1
    act: str = "none"           # "swiglu" | "gelu" | "none"
    dtype: str = "bf16"
    w_std: float = 0.02
    x_std: float = 1.0
    integer: bool = False
    rmsnorm: bool = False
    eps: float = 1e-5
    extra: dict = field(default_factory=dict)


CONFIGS = {
    # Toy two-rank MLP on integer-valued fp32 inputs.
    "toy_mlp_int": Config(name="toy_mlp_int", seed=101, tp=2, hidden=64, tokens=(4,),
                          inter=256, act="none", dtype="f32", integer=True),
    # Decode MLP shard of a 70B-class layer at TP=8 (SwiGLU).
    "decode_mlp_tp8": Config(name="decode_mlp_tp8", seed=102, tp=8, hidden=8192,
                             tokens=(1, 8, 64), inter=28672, act="swiglu"),
    # Decode attention shard, 32 q / 8 KV heads at TP=4, batch 32, 2048 keys.
    "decode_attn_tp4": Config(name="decode_attn_tp4", seed=103, tp=4, hidden=4096,
                              tokens=(1,), n_q=32, n_kv=8, head_dim=128, kv_len=2048,
                              batch=32),
    # Prefill full decoder-layer shard at TP=2, 4096 tokens, RMSNorm pre-norm.
    "prefill_layer_tp2": Config(name="prefill_layer_tp2", seed=104, tp=2, hidden=8192,
                                tokens=(4096,), inter=28672, n_q=64, n_kv=8,
                                head_dim=128, act="swiglu", rmsnorm=True),
    # The same attention at TP=16: fewer KV heads than ranks, so each rank holds
    # 2 q heads and one KV head replicated on 2 ranks.
    "decode_attn_tp16_rep": Config(name="decode_attn_tp16_rep", seed=106, tp=16, hidden=4096,
                                   tokens=(1,), n_q=32, n_kv=8, head_dim=128, kv_len=2048,
                                   batch=32),
    # Vocab-parallel lm_head at TP=8 (128256-token vocab, 16032 rows per rank),
    # greedy choice of the next token for 1 and 8 sequences.
    "lm_head_tp8": Config(name="lm_head_tp8", seed=107, tp=8, hidden=8192, tokens=(1, 8),
                          extra={"vocab": 128256}),
    # GPT-style GELU MLP at TP=8, 4x expansion, all 8 ranks + in-HBM reduce.
    "gelu_mlp_tp8": Config(name="gelu_mlp_tp8", seed=105, tp=8, hidden=12288,
                           tokens=(2048,), inter=49152, act="gelu"),
}


def config(name: str) -> Config:
    return CONFIGS[name]
