"""Host orchestration of one tensor-parallel rank's decoder-layer share.

Each class holds one rank's device weights and preallocated buffers and issues
the library's calls in the order of a pre-norm layer (P1 "Attention 里的 tensor
parallel" / "MLP 里的 tensor parallel"; P2 sections 二 and 2.1):

    xn = RMSNorm(x)                                   replicated
    qkv = xn Wqkv_r                                   column-parallel
    o = attention over the rank's heads               local
    P_attn_r = o Wo_r                                 row-parallel partial
    h = x + sum_r P_attn_r                            all-reduce arithmetic
                                                      (h stays float32)
    hn = RMSNorm(h)                                   (fused with the sum)
    g|u = hn Wgu_r                                    column-parallel
    a = SiLU(g) * u   (or GELU(g))                    local (fused into g|u)
    P_mlp_r = a Wd_r                                  row-parallel partial
    y = h + sum_r P_mlp_r                             all-reduce arithmetic

(P1 = page "Tensor Parallel：当一张 GPU 放不下一个大模型"; P2 = page
"张量并行（Tensor Parallelism）推理部署实战：从 Megatron-LM 切分原理到 vLLM 多卡配置与性能调优".)

On one GPU the other ranks' partials are buffers in HBM (computed by running
their shards on the same GPU, or supplied by the caller); the all-reduce is
``reduce_partials`` over all of them in rank order.  No arithmetic happens
here: every step is a library call.
"""
from __future__ import annotations

import torch

from . import (column_linear, column_linear_act, decode_attention_append, kv_append,
               local_attention, paged_attention_workspace, paged_decode_attention_append,
               reduce_partials, reduce_partials_rmsnorm, rmsnorm, row_linear_partial,
               swiglu_local, vocab_argmax_local, vocab_argmax_reduce)


class MlpShard:
    """gate|up (or fc1) column-parallel, local activation, down (or fc2)
    row-parallel partial for one rank.  ``w_in`` is ``[2*I_l, H]`` (gate rows
    then up rows) for SwiGLU or ``[I_l, H]`` for GELU/none; ``w_out`` is
    ``[H, I_l]``.  With ``fused`` (the default) a bf16 shard takes the
    activation in the projection's epilogue (``column_linear_act``), on the
    float32 sums; unfused, the projection is stored as bf16 before the
    activation kernel reads it."""

    def __init__(self, w_in: torch.Tensor, w_out: torch.Tensor, act: str, max_tokens: int,
                 fused: bool = True):
        self.w_in, self.w_out, self.act = w_in, w_out, act
        self.fused = (fused and act in ("swiglu", "gelu") and w_in.dtype == torch.bfloat16
                      and w_in.shape[1] % 8 == 0 and w_in.data_ptr() % 16 == 0)
        self.I = w_out.shape[1]
        self.H = w_out.shape[0]
        n_in = w_in.shape[0]
        if n_in != (2 * self.I if act == "swiglu" else self.I):
            raise ValueError("w_in rows do not match the activation")
        dev, dt = w_in.device, w_in.dtype
        self.gu = torch.empty((max_tokens, n_in), dtype=dt, device=dev)
        self.a = torch.empty((max_tokens, self.I), dtype=dt, device=dev)

    def partial(self, x: torch.Tensor, out: torch.Tensor):
        M = x.shape[0]
        a = self.a[:M]
        if self.fused and x.is_contiguous() and x.data_ptr() % 16 == 0:
            column_linear_act(x, self.w_in, self.act, out=a)
            row_linear_partial(a, self.w_out, out=out)
            return out
        gu = self.gu[:M]
        column_linear(x, self.w_in, out=gu)
        if self.act == "swiglu":
            swiglu_local(gu[:, :self.I], gu[:, self.I:], "swiglu", out=a)
        else:
            swiglu_local(gu, None, self.act, out=a)
        row_linear_partial(a, self.w_out, out=out)
        return out


class AttnShard:
    """Fused QKV column-parallel, local attention, o_proj row-parallel partial
    for one rank.  ``wqkv`` is ``[(Hq_l + 2*Hkv_l)*D, H]``, ``wo`` ``[H, Hq_l*D]``."""

    def __init__(self, wqkv: torch.Tensor, wo: torch.Tensor, n_q: int, n_kv: int, head_dim: int,
                 max_tokens: int):
        self.wqkv, self.wo = wqkv, wo
        self.n_q, self.n_kv, self.D = n_q, n_kv, head_dim
        if wqkv.shape[0] != (n_q + 2 * n_kv) * head_dim or wo.shape[1] != n_q * head_dim:
            raise ValueError("weight shapes do not match the head counts")
        dev, dt = wqkv.device, wqkv.dtype
        self.qkv = torch.empty((max_tokens, wqkv.shape[0]), dtype=dt, device=dev)
        self.o = torch.empty((max_tokens, n_q * head_dim), dtype=dt, device=dev)
        self.ws = None

    def _views(self, qkv: torch.Tensor, B: int, S: int):
        D, hq, hkv = self.D, self.n_q, self.n_kv
        W = qkv.shape[1]
        base = qkv.view(B, S, W)
        q = base[:, :, :hq * D].unflatten(2, (hq, D))
        k = base[:, :, hq * D:(hq + hkv) * D].unflatten(2, (hkv, D))
        v = base[:, :, (hq + hkv) * D:].unflatten(2, (hkv, D))
        return q, k, v

    def prefill_partial(self, xn: torch.Tensor, out: torch.Tensor, causal: bool = True):
        """One sequence of S tokens (``xn [S, H]``), causal self-attention."""
        S = xn.shape[0]
        qkv = self.qkv[:S]
        column_linear(xn, self.wqkv, out=qkv)
        q, k, v = self._views(qkv, 1, S)
        o = self.o[:S]
        local_attention(q, k, v, causal=causal, out=o.view(1, S, self.n_q, self.D))
        row_linear_partial(o, self.wo, out=out)
        return out

    def decode_partial(self, x: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                       pos: int, out: torch.Tensor):
        """One new token for each of B sequences (``x [B, H]``); the caches are
        ``[B, T, Hkv_l, D]``; the token is appended at ``pos`` and attends over
        keys ``0..pos``."""
        B = x.shape[0]
        qkv = self.qkv[:B]
        column_linear(x, self.wqkv, out=qkv)
        q, k, v = self._views(qkv, B, 1)
        o = self.o[:B]
        ws = self._workspace(B, pos + 1, x.device)
        if self.n_q // self.n_kv <= 32:   # append and attention in one launch
            decode_attention_append(q[:, 0], k[:, 0], v[:, 0], k_cache, v_cache, pos,
                                    out=o.view(B, self.n_q, self.D), workspace=ws)
        else:
            kv_append(k[:, 0], v[:, 0], k_cache, v_cache, pos)
            local_attention(q, k_cache[:, :pos + 1], v_cache[:, :pos + 1], causal=True,
                            out=o.view(B, 1, self.n_q, self.D), workspace=ws)
        row_linear_partial(o, self.wo, out=out)
        return out

    def decode_partial_paged(self, x: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                             block_table: torch.Tensor, context_lens: torch.Tensor,
                             max_context_len: int, out: torch.Tensor):
        """One new token per sequence with a paged cache: pools
        ``[num_blocks, block_size, Hkv_l, D]`` holding this rank's KV heads,
        the block table shared by all ranks; ``context_lens[b]`` counts the
        new token, which is stored at position ``context_lens[b] - 1``."""
        B = x.shape[0]
        qkv = self.qkv[:B]
        column_linear(x, self.wqkv, out=qkv)
        q, k, v = self._views(qkv, B, 1)
        o = self.o[:B]
        need = paged_attention_workspace(B, self.n_q, self.n_kv, max_context_len, k_pool.shape[1])
        if need and (self.ws is None or self.ws.numel() < need):
            self.ws = torch.empty(need, dtype=torch.uint8, device=x.device)
        # append and attention in one launch (the kernel takes G <= 32 in both forms)
        paged_decode_attention_append(q[:, 0], k[:, 0], v[:, 0], k_pool, v_pool, block_table,
                                      context_lens, max_context_len,
                                      out=o.view(B, self.n_q, self.D), workspace=self.ws)
        row_linear_partial(o, self.wo, out=out)
        return out

    def _workspace(self, B, L, device):
        from . import local_attention_workspace
        need = local_attention_workspace(B, 1, L, self.n_q, self.n_kv, self.D)
        if need and (self.ws is None or self.ws.numel() < need):
            self.ws = torch.empty(need, dtype=torch.uint8, device=device)
        return self.ws


class LayerShard:
    """One rank's share of a pre-norm decoder layer (prefill of one sequence).

    The residual stream ``h`` (the attention sub-block's sum plus the input)
    is kept in float32: it is never a GEMM operand, only the residual of the
    final sum and the input of the second pre-norm.  The layer input ``x``,
    the normalised ``xn``/``hn`` and the output ``y`` are bf16."""

    def __init__(self, g1, g2, wqkv, wo, wgu, wd, n_q, n_kv, head_dim, eps, max_tokens,
                 act="swiglu", fused=True):
        self.g1, self.g2, self.eps, self.fused = g1, g2, eps, fused
        self.attn = AttnShard(wqkv, wo, n_q, n_kv, head_dim, max_tokens)
        self.mlp = MlpShard(wgu, wd, act, max_tokens, fused=fused)
        H = wo.shape[0]
        dev, dt = wqkv.device, wqkv.dtype
        self.xn = torch.empty((max_tokens, H), dtype=dt, device=dev)
        self.h = torch.empty((max_tokens, H), dtype=torch.float32, device=dev)
        self.hn = torch.empty((max_tokens, H), dtype=dt, device=dev)

    def attn_partial(self, x, out):
        S = x.shape[0]
        rmsnorm(x, self.g1, self.eps, out=self.xn[:S])
        return self.attn.prefill_partial(self.xn[:S], out)

    def mlp_partial(self, h, out):
        S = h.shape[0]
        rmsnorm(h, self.g2, self.eps, out=self.hn[:S])
        return self.mlp.partial(self.hn[:S], out)

    def step(self, x, attn_parts, mlp_parts, rank: int, y):
        """The rank's full step.  ``attn_parts``/``mlp_parts`` are the R
        partial buffers; this rank writes slot ``rank`` of each, the other
        slots hold what the other ranks contributed."""
        S = x.shape[0]
        self.attn_partial(x, attn_parts[rank])
        h = self.h[:S]
        if self.fused:
            # the all-reduce's sum and the MLP's pre-norm in one pass
            reduce_partials_rmsnorm(attn_parts, self.g2, residual=x, eps=self.eps, out=h,
                                    out_norm=self.hn[:S])
            self.mlp.partial(self.hn[:S], mlp_parts[rank])
        else:
            reduce_partials(attn_parts, residual=x, out=h)
            self.mlp_partial(h, mlp_parts[rank])
        reduce_partials(mlp_parts, residual=h, out=y)
        return y


class VocabShard:
    """One rank's block of a vocab-parallel lm_head (P1 "lm_head 怎么处理"):
    ``w`` is the rank's ``[V_r, H]`` rows of the ``[V, H]`` lm_head, starting at
    vocab id ``offset``.  ``local_greedy`` gives the rank's float32 logits and
    its (largest logit, global id) per token; ``greedy`` combines all ranks'
    pairs (the all-gather's arithmetic) into the next token ids."""

    def __init__(self, w: torch.Tensor, offset: int, max_tokens: int):
        self.w, self.offset = w, offset
        self.logits = torch.empty((max_tokens, w.shape[0]), dtype=torch.float32, device=w.device)

    def local_greedy(self, h: torch.Tensor):
        z = self.logits[:h.shape[0]]
        row_linear_partial(h, self.w, out=z)     # fp32 output of h @ w.T
        return vocab_argmax_local(z, self.offset)

    @staticmethod
    def greedy(pairs):
        return vocab_argmax_reduce([p[0] for p in pairs], [p[1] for p in pairs])
