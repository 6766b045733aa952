"""Small GPU drivers for the hardware-counter runs whose summaries live in
``profiles/`` (they only call the library; no measurement logic here).

    python3 -m tensor_transformer_layer_05_amd.profile_drivers gemm_traffic

``gemm_traffic``: one plain 256 MiB device-to-device copy (a calibration
dispatch of known size: 256 MiB read, 256 MiB written), then one launch of the
prefill gate|up projection with SwiGLU in its epilogue (M=4096, K=8192,
2I=28672, output [4096, 14336], bf16), then one launch of the plain gate|up
GEMM on the same operands (output [4096, 28672]).  Run it under
``rocprofv3 --pmc FETCH_SIZE`` and, separately, ``--pmc WRITE_SIZE``.
"""
from __future__ import annotations

import sys

import torch

from . import column_linear, column_linear_act, lib


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


DRIVERS = {"gemm_traffic": gemm_traffic}

if __name__ == "__main__":
    DRIVERS[sys.argv[1] if len(sys.argv) > 1 else "gemm_traffic"]()
