"""The decode shards captured in a HIP graph (as a serving loop issues them)
give the same bits as the same calls issued eagerly, on every replay, with
eager work and synchronisations between the replays."""
import pytest
import torch

import tensor_transformer_layer_05_amd as tpl
from tensor_transformer_layer_05_amd import inputs as I
from tensor_transformer_layer_05_amd.shard import AttnShard, MlpShard
from util import log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _replays_match(fn, outs, n=3):
    fn()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for i in range(n):
        for o in outs:
            o.fill_(float("nan"))
        fn()                           # eager work between replays
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            assert torch.equal(o, r), "eager run changed"
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            assert torch.equal(o, r), f"graph replay {i} differs from the eager result"


@pytest.mark.parametrize("M", [1, 8, 64, 100])
def test_mlp_shard_graph_replay(M):
    log(f"graph replay MLP shard M={M}")
    H, I_ = 1024, 448
    wgu = I.normal(30, "wgu", (2 * I_, H), 0.02).dev.to(DEV)
    wd = I.normal(30, "wd", (H, I_), 0.02).dev.to(DEV)
    x = I.normal(30, "x", (M, H)).dev.to(DEV)
    sh = MlpShard(wgu, wd, "swiglu", M)
    out = torch.empty((M, H), dtype=torch.float32, device=DEV)
    _replays_match(lambda: sh.partial(x, out), [out])


def test_decode_attention_shard_graph_replay():
    log("graph replay decode attention shard")
    B, H, hq, hkv, D, L = 4, 1024, 4, 2, 128, 300
    wqkv = I.normal(31, "wqkv", ((hq + 2 * hkv) * D, H), 0.02).dev.to(DEV)
    wo = I.normal(31, "wo", (H, hq * D), 0.02).dev.to(DEV)
    kc = I.normal(31, "k", (B, hkv, L, D)).dev.to(DEV)
    vc = I.normal(31, "v", (B, hkv, L, D)).dev.to(DEV)
    x = I.normal(31, "x", (B, H)).dev.to(DEV)
    sh = AttnShard(wqkv, wo, hq, hkv, D, B)
    out = torch.empty((B, H), dtype=torch.float32, device=DEV)
    _replays_match(lambda: sh.decode_partial(x, kc.transpose(1, 2), vc.transpose(1, 2), L - 1, out),
                   [out])
