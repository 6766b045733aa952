"""Small GPU drivers for the hardware-counter runs whose summaries live in
``profiles/`` (they only call the library; no measurement logic here).

    python3 -m tensor_transformer_layer_05_amd.profile_drivers gemm_traffic

``gemm_traffic``: one plain 256 MiB device-to-device copy (a calibration
dispatch of known size: 256 MiB read, 256 MiB written), then one launch of the
prefill gate|up projection with SwiGLU in its epilogue (M=4096, K=8192,
2I=28672, output [4096, 14336], bf16), then one launch of the plain gate|up
GEMM on the same operands (output [4096, 28672]).  Run it under
``rocprofv3 --pmc FETCH_SIZE`` and, separately, ``--pmc WRITE_SIZE``.

``decode_attn_span``: decode attention of the TP=4 shard shape (32 sequences,
8 q / 2 KV heads of 128) over key spans of 512 .. 16384, 20 calls each on
rotating cache copies, for ``rocprofv3 --kernel-trace``: the kernel durations
per span separate the fixed cost of a launch from the streaming rate.

``decode_traffic``: the HBM bytes of each decode shard's step.  One plain
256 MiB device-to-device copy (calibration), then for every decode shard of
the benchmark, in its order (``decode_workloads.DECODE_NAMES``): its setup, a
1 GiB read-only stream (``libtpref``; it evicts the caches and marks where the
step's dispatches start), one step of the shard, and a 4 KiB read by the same
stream kernel that marks where they end.  Run it under ``rocprofv3 --pmc
FETCH_SIZE`` and, separately, ``--pmc WRITE_SIZE``; a shard's bytes are the
sums over the dispatches between its two markers.

``stream_ref``: 20 reads of 1 GiB by the reference stream kernel of
``libtpref`` in a given configuration (workgroups, waves, KB per wave per
chunk, load flags: 1 = non-temporal, 2 = chunks interleaved over all waves),
for ``rocprofv3 --kernel-trace``.

``vendor_gemm``: the plain gate|up GEMM (M=4096, K=8192, N=28672, bf16
output) three times through ``torch.matmul`` (the vendor library's GEMM) and
three times through the library, on the same operands, for ``rocprofv3
--pmc`` runs that compare the two kernels' instruction mix and stalls.

``prefill_attention``: the prefill attention of the TP=2 layer shard (one
sequence of 4096 tokens, causal, 32 q / 4 KV heads of 128 on strided views of
the fused QKV output, as the layer shard issues it), three launches, for
``rocprofv3 --pmc`` runs of its instruction mix and MFMA utilisation.

``ffn_gemms``: the GELU FFN shard's two GEMMs at TP=8 (2048 tokens, hidden
12288, local intermediate 6144): one plain 256 MiB device-to-device copy
(calibration), then fc1 with GELU in its epilogue three times and fc2 to
float32 partials three times, for ``rocprofv3 --pmc`` runs of their HBM bytes
(FETCH_SIZE, WRITE_SIZE) and MFMA and LDS counters.

``hbm_reference``: what plain streaming reaches on this GPU, next to the
library's own decode weight stream: 20 device-to-device copies of 1 GiB, 20
full sums of a 1 GiB float32 tensor (read only), then 20 one-token decode
gate|up + SwiGLU calls (weight [7168, 8192] bf16, four rotating copies), for
``rocprofv3 --kernel-trace``.
"""
from __future__ import annotations

import sys

import torch

from . import (column_linear, column_linear_act, lib, local_attention, local_attention_workspace,
               row_linear_partial)


def gemm_traffic() -> None:
    lib()
    n = 256 << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    M, K, N = 4096, 8192, 28672
    x = torch.randn(M, K, device="cuda").to(torch.bfloat16)
    w = (torch.randn(N, K, device="cuda") * 0.02).to(torch.bfloat16)
    h = torch.empty(M, N // 2, device="cuda", dtype=torch.bfloat16)
    y = torch.empty(M, N, device="cuda", dtype=torch.bfloat16)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    column_linear_act(x, w, "swiglu", out=h)
    torch.cuda.synchronize()
    column_linear(x, w, out=y)
    torch.cuda.synchronize()
    print("gemm_traffic done", flush=True)


SPANS = (512, 1024, 2048, 4096, 8192, 16384)


def decode_attn_span() -> None:
    lib()
    B, Hq, Hkv, D = 32, 8, 2, 128
    for L in SPANS:
        copies = 4 if L <= 4096 else 2
        sets = []
        for _ in range(copies):
            q = torch.randn(B, 1, Hq, D, device="cuda").to(torch.bfloat16)
            k = torch.randn(B, L, Hkv, D, device="cuda").to(torch.bfloat16)
            v = torch.randn(B, L, Hkv, D, device="cuda").to(torch.bfloat16)
            o = torch.empty(B, 1, Hq, D, device="cuda", dtype=torch.bfloat16)
            ws = torch.empty(max(1, local_attention_workspace(B, 1, L, Hq, Hkv, D)), dtype=torch.uint8,
                             device="cuda")
            sets.append((q, k, v, o, ws))
        torch.cuda.synchronize()
        for i in range(20):
            q, k, v, o, ws = sets[i % copies]
            local_attention(q, k, v, causal=True, out=o, workspace=ws)
        torch.cuda.synchronize()
        print(f"decode_attn_span L={L} done", flush=True)
        del sets


HBM_REF_BYTES = 1 << 30
HBM_REF_CALLS = 20


def vendor_gemm() -> None:
    lib()
    M, K, N = 4096, 8192, 28672
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    x = torch.randn(M, K, device="cuda", generator=g).to(torch.bfloat16)
    w = (torch.randn(N, K, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    y = torch.empty(M, N, device="cuda", dtype=torch.bfloat16)
    for _ in range(3):
        torch.matmul(x, w.t(), out=y)
    torch.cuda.synchronize()
    for _ in range(3):
        column_linear(x, w, out=y)
    torch.cuda.synchronize()


def prefill_attention() -> None:
    lib()
    S, hq, hkv, D = 4096, 32, 4, 128
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    qkv = torch.randn(S, (hq + 2 * hkv) * D, device="cuda", generator=g).to(torch.bfloat16)
    base = qkv.view(1, S, -1)
    q = base[:, :, :hq * D].unflatten(2, (hq, D))
    k = base[:, :, hq * D:(hq + hkv) * D].unflatten(2, (hkv, D))
    v = base[:, :, (hq + hkv) * D:].unflatten(2, (hkv, D))
    o = torch.empty(1, S, hq, D, device="cuda", dtype=torch.bfloat16)
    for _ in range(3):
        local_attention(q, k, v, causal=True, out=o)
    torch.cuda.synchronize()


def ffn_gemms() -> None:
    lib()
    M, H, F = 2048, 12288, 6144
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    x = torch.randn(M, H, device="cuda", generator=g).to(torch.bfloat16)
    w1 = (torch.randn(F, H, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    w2 = (torch.randn(H, F, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    a = torch.empty(M, F, device="cuda", dtype=torch.bfloat16)
    p = torch.empty(M, H, device="cuda", dtype=torch.float32)
    n = 256 << 20
    c0 = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    c1 = torch.empty_like(c0)
    torch.cuda.synchronize()
    c1.copy_(c0)
    torch.cuda.synchronize()
    for _ in range(3):
        column_linear_act(x, w1, "gelu", out=a)
    torch.cuda.synchronize()
    for _ in range(3):
        row_linear_partial(a, w2, out=p)
    torch.cuda.synchronize()
    print("ffn_gemms done", flush=True)


def hbm_reference() -> None:
    lib()
    a = torch.ones(HBM_REF_BYTES, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    f = torch.ones(HBM_REF_BYTES // 4, dtype=torch.float32, device="cuda")
    ws = [(torch.randn(7168, 8192, device="cuda") * 0.02).to(torch.bfloat16) for _ in range(4)]
    x = torch.randn(1, 8192, device="cuda").to(torch.bfloat16)
    torch.cuda.synchronize()
    for _ in range(HBM_REF_CALLS):
        b.copy_(a)
    torch.cuda.synchronize()
    for _ in range(HBM_REF_CALLS):
        f.sum()
    torch.cuda.synchronize()
    for i in range(HBM_REF_CALLS):
        column_linear_act(x, ws[i % 4], "swiglu")
    torch.cuda.synchronize()
    print("hbm_reference done", flush=True)


def decode_traffic() -> None:
    from . import ref
    from .decode_workloads import all_decode
    lib()
    ref.lib()
    n = 256 << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    flush = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
    words = torch.empty(256 * 8 * 64, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    for build in all_decode(copies=1, span=0):
        w = build()
        torch.cuda.synchronize()
        ref.stream_read(flush, words)
        torch.cuda.synchronize()
        w.steps[0]()
        torch.cuda.synchronize()
        ref.stream_read(flush[:4096], words)
        torch.cuda.synchronize()
        print(f"decode_traffic {w.name} done", flush=True)
        del w


def stream_ref(workgroups: int = 256, waves: int = 8, loads: int = 8, flags: int = 0) -> None:
    from . import ref
    ref.lib()
    buf = torch.ones(HBM_REF_BYTES, dtype=torch.uint8, device="cuda")
    words = torch.empty(workgroups * waves * 64, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    for _ in range(HBM_REF_CALLS):
        ref.stream_read(buf, words, workgroups, waves, loads, flags)
    torch.cuda.synchronize()
    print("stream_ref done", flush=True)


DRIVERS = {"gemm_traffic": gemm_traffic, "vendor_gemm": vendor_gemm, "ffn_gemms": ffn_gemms, "prefill_attention": prefill_attention, "decode_attn_span": decode_attn_span, "hbm_reference": hbm_reference,
           "decode_traffic": decode_traffic, "stream_ref": stream_ref}

if __name__ == "__main__":
    name = sys.argv[1] if len(sys.argv) > 1 else "gemm_traffic"
    DRIVERS[name](*[int(v) for v in sys.argv[2:]])
