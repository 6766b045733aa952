"""The allocation-free decode entry point (tp_decode_attention_append_noalloc,
for callers that cannot allocate device memory) against the entry point it
varies, tp_decode_attention_append with a caller workspace: the same output
and cache bits, call after call on one GPU, the second call of each pair
smaller than the first, and the first case the largest partials buffer any
call can need (255 (sequence, KV head) pairs of 32 q heads, two chunks each).
Also under HIP graph capture, the use it exists for, and against the oracle."""
import numpy as np
import pytest
import torch

import oracle.tp_oracle as O
import tensor_transformer_layer_05_amd as tpl
from tensor_transformer_layer_05_amd import inputs as I
from util import assert_normwise, log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
D = 128


def _case(seed, B, Hq, Hkv, T):
    qkv = I.normal(seed, "qkv", (B, (Hq + 2 * Hkv) * D)).dev.to(DEV)
    q = qkv[:, :Hq * D].unflatten(1, (Hq, D))
    kn = qkv[:, Hq * D:(Hq + Hkv) * D].unflatten(1, (Hkv, D))
    vn = qkv[:, (Hq + Hkv) * D:].unflatten(1, (Hkv, D))
    kc = I.normal(seed, "kc", (B, Hkv, T, D)).dev.to(DEV)
    vc = I.normal(seed, "vc", (B, Hkv, T, D)).dev.to(DEV)
    return q, kn, vn, kc, vc


def _both(q, kn, vn, kc, vc, pos):
    B, Hq = q.shape[:2]
    k1, v1, k2, v2 = kc.clone(), vc.clone(), kc.clone(), vc.clone()
    o1 = tpl.decode_attention_append(q, kn, vn, k1.transpose(1, 2), v1.transpose(1, 2), pos)
    o2 = torch.full((B, Hq, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    tpl.decode_attention_append_noalloc(q, kn, vn, k2.transpose(1, 2), v2.transpose(1, 2), pos, out=o2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2), "no-alloc output differs from the workspace entry point"
    assert torch.equal(k1, k2) and torch.equal(v1, v2), "caches differ"
    return o2, k2, v2


SEQUENCES = [
    # (B, Hq, Hkv, T, pos), each list run in order on one GPU
    [(255, 32, 1, 300, 299), (32, 8, 2, 2048, 2047)],     # the largest buffer, then the shard
    [(32, 8, 2, 2048, 2047), (3, 16, 2, 700, 500)],       # the shard, then a smaller call
    [(2, 8, 2, 4096, 4000), (300, 4, 1, 200, 150)],       # many chunks, then no split at all
]


@pytest.mark.parametrize("seq", SEQUENCES, ids=["max-then-shard", "shard-then-small", "split-then-none"])
def test_noalloc_equals_workspace_entry(seq):
    for i, (B, Hq, Hkv, T, pos) in enumerate(seq):
        log(f"no-alloc decode call {i}: B={B} Hq={Hq} Hkv={Hkv} T={T} pos={pos}")
        q, kn, vn, kc, vc = _case(80 + i, B, Hq, Hkv, T)
        o, k2, v2 = _both(q, kn, vn, kc, vc, pos)
        if i == 0:
            # the oracle on the first call: the new key/value at pos, attention over 0..pos
            kref = kc.double().cpu().numpy(); vref = vc.double().cpu().numpy()
            kref[:, :, pos] = kn.double().cpu().numpy(); vref[:, :, pos] = vn.double().cpu().numpy()
            ref = O.attention(q.double().cpu().numpy()[:, None],
                              kref[:, :, :pos + 1].transpose(0, 2, 1, 3),
                              vref[:, :, :pos + 1].transpose(0, 2, 1, 3), causal=True)[:, 0]
            assert_normwise(o, ref, 1e-2, "no-alloc decode attention vs oracle")


def test_noalloc_under_graph_capture():
    """Captured in a HIP graph (no allocation inside the capture), replayed
    with eager work between replays: every replay gives the eager bits."""
    B, Hq, Hkv, T, pos = 16, 8, 2, 1024, 1000
    log(f"no-alloc decode under graph capture B={B} Hq={Hq} Hkv={Hkv} pos={pos}")
    q, kn, vn, kc, vc = _case(90, B, Hq, Hkv, T)
    out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=DEV)
    run = lambda: tpl.decode_attention_append_noalloc(q, kn, vn, kc.transpose(1, 2),
                                                      vc.transpose(1, 2), pos, out=out)
    run()
    torch.cuda.synchronize()
    ref = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    other = _case(91, 4, 8, 2, 600)
    for i in range(3):
        _both(*other, 599)                  # eager calls of both entry points between replays
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"graph replay {i} differs from the eager result"


def test_noalloc_rejects_before_launch():
    q, kn, vn, kc, vc = _case(92, 2, 64, 1, 256)     # 64 q heads per KV head: unsupported
    out = torch.empty((2, 64, D), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(tpl.TPError):
        tpl.decode_attention_append_noalloc(q, kn, vn, kc.transpose(1, 2), vc.transpose(1, 2), 10,
                                            out=out)
