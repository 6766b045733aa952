"""Vocab-parallel greedy decoding (page P1, section "lm_head 怎么处理"): each
rank's local (largest logit, vocab id) and the combine over ranks, against
the oracle.  The argmax entry points take float32 logits; their parity cases
feed both sides the same seeded logits, so the integer results must match bit
for bit (ties, NaN and -inf planted).  End to end through the lm_head GEMM:
integer-valued inputs give exact logits (bit-exact ids, ties across ranks
included); normal inputs are checked against the float64 oracle's logits with
the GEMM's derived error bound."""
import numpy as np
import pytest
import torch

import oracle.tp_oracle as O
import tensor_transformer_layer_05_amd as tpl
from tensor_transformer_layer_05_amd import inputs as I
from tensor_transformer_layer_05_amd.shard import VocabShard
from util import U32, log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _planted_logits(seed, M, V):
    z = I.normal(seed, "logits", (M, V), 3.0, dtype=torch.float32).dev.clone()
    if V >= 8:
        for m in range(M):
            j = (7 * m + 3) % V
            k = (13 * m + 5) % V
            z[m, max(j, k)] = z[m, min(j, k)] = z[m].max() + 1.0   # tie inside the row
        if M > 1:
            z[1, :] = float("nan")                                  # nothing: id offset, -inf
        if M > 2:
            z[2, :] = float("nan"); z[2, V // 2] = float("-inf")
        if M > 3:
            z[3, 0] = float("nan"); z[3, V - 1] = 1e30              # NaN never wins
        if M > 4:
            z[4, :] = -1.0; z[4, V - 2] = 0.0; z[4, 1] = -0.0       # -0 == +0: lower id
    return z


@pytest.mark.parametrize("M,V", [(1, 1), (1, 7), (3, 1000), (8, 16032), (64, 16032), (5, 128256),
                                 (2, 130), (6, 131),
                                 # 16-byte path: a second pass over the row with one live
                                 # element, where row 3 has its max; 4-byte path (V % 4 != 0)
                                 # over several passes
                                 (4, 4 * 8192 + 4), (5, 70001)])
def test_vocab_argmax_local_exact(M, V):
    log(f"vocab argmax local M={M} V={V}")
    z = _planted_logits(50, M, V)
    off = 3 * V
    mv, mi = tpl.vocab_argmax_local(z.to(DEV), off)
    rv, ri = O.vocab_argmax_local(z.double().numpy(), off)
    assert np.array_equal(mi.cpu().numpy(), ri), (mi.cpu().numpy(), ri)
    assert np.array_equal(mv.cpu().double().numpy(), rv)


@pytest.mark.parametrize("R", [1, 2, 3, 8, 64])
def test_vocab_argmax_reduce_exact(R):
    log(f"vocab argmax reduce R={R}")
    M, b = 300, 1000
    vals = [I.normal(51, "v", (M,), 1.0, dtype=torch.float32, rank=r).dev.clone() for r in range(R)]
    ids = [torch.from_numpy(np.random.default_rng(r).integers(0, b, M)) + r * b for r in range(R)]
    for r in range(1, R):                      # equal values across ranks: lowest id wins
        vals[r][r::7] = vals[0][r::7]
    if R > 1:
        vals[R - 1][0] = 1e30
    ov, oi = tpl.vocab_argmax_reduce([v.to(DEV) for v in vals], [i.to(DEV) for i in ids])
    rv, ri = O.vocab_argmax_reduce([v.double().numpy() for v in vals], [i.numpy() for i in ids])
    assert np.array_equal(oi.cpu().numpy(), ri) and np.array_equal(ov.cpu().double().numpy(), rv)


@pytest.mark.parametrize("R", [1, 2, 4, 8])
def test_lm_head_integer_bitexact(R):
    """Integer-valued h and W: exact logits, duplicated vocab rows in
    different ranks' blocks plant ties that must go to the lowest id."""
    log(f"lm_head integer R={R}")
    M, H, V = 9, 64, 1000
    h = I.uniform_int(52, "h", (M, H), dtype=torch.bfloat16)
    w = I.uniform_int(52, "w", (V, H), dtype=torch.bfloat16)
    wd, wr = w.dev.clone(), w.ref.copy()
    best = np.sign(h.ref + 0.5) * 3.0
    for m, (a, c) in enumerate([(10, 990), (500, 501), (3, 260)]):
        wd[a] = wd[c] = torch.from_numpy(best[m]).to(torch.bfloat16)
        wr[a] = wr[c] = best[m]
    H_ = h.dev.to(DEV)
    b = V // R
    pairs = [VocabShard(tpl.shard_column(wd, r, R).to(DEV), r * b, M).local_greedy(H_) for r in range(R)]
    gv, gi = VocabShard.greedy(pairs)
    rv, ri = O.greedy_token(h.ref, wr)
    assert np.array_equal(gi.cpu().numpy(), ri) and np.array_equal(gv.cpu().double().numpy(), rv)
    assert gi[0].item() == 10 and gi[1].item() == 500 and gi[2].item() == 3


@pytest.mark.parametrize("M", [1, 8])
def test_lm_head_tp8_greedy(M):
    c = I.config("lm_head_tp8")
    H, R, V = c.hidden, c.tp, c.extra["vocab"]
    log(f"config lm_head_tp8 M={M} V={V}")
    h = I.normal(c.seed, "h", (M, H))
    H_ = h.dev.to(DEV)
    b = V // R
    pairs, refs = [], []
    for r in range(R):
        w = I.normal(c.seed, "w", (b, H), c.w_std, rank=r)      # rank r's vocab rows
        pairs.append(VocabShard(w.dev.to(DEV), r * b, M).local_greedy(H_))
        refs.append((O.linear(h.ref, w.ref), 1.01 * H * U32 * (np.abs(h.ref) @ np.abs(w.ref).T)))
    gv, gi = VocabShard.greedy(pairs)
    z = np.concatenate([a for a, _ in refs], 1)        # float64 logits over the full vocab
    bound = np.concatenate([e for _, e in refs], 1)    # fp32 accumulation error bound per logit
    ids = gi.cpu().numpy()
    for m in range(M):
        j = ids[m]
        top = np.argsort(z[m])[::-1][:2]
        # the chosen token's exact logit is within the rounding of the best
        assert z[m, j] >= z[m, top[0]] - bound[m, j] - bound[m, top[0]], (m, j, top)
        # and when the best is separated by more than the rounding, it is the best
        if z[m, top[0]] - z[m, top[1]] > bound[m, top[0]] + bound[m, top[1]]:
            assert j == top[0]
        assert abs(gv[m].item() - z[m, j]) <= bound[m, j]
