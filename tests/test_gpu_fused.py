"""The fused entry points against the oracle, and against the unfused calls
they replace:
  * column_linear_act: the column-parallel gate|up (or fc1) projection with
    the rank-local activation in its epilogue (the activation needs no
    exchange because gate_i and up_i live on the same rank).  The activation
    is taken on the float32 sums, so the reference is the activation of the
    EXACT projections; the unfused calls store g and u as bf16 first and are
    checked against the activation of the rounded projections.
  * reduce_partials_rmsnorm: the all-reduce's sum of rank partials plus the
    residual, followed by the next sub-block's pre-norm, in one pass; equal
    bit for bit to the two unfused calls, for every pair of residual and
    output storage types.
Shapes cover every dispatch of the fused linear (one and two 16-token tiles
with 4, 8 and 16 waves splitting K, the 3-4 tile LDS-ring kernel with one to
four token row groups, both tile sizes of the prefill kernel) with ragged
token and feature counts."""
import numpy as np
import pytest
import torch

import oracle.tp_oracle as O
import tensor_transformer_layer_05_amd as tpl
from tensor_transformer_layer_05_amd import inputs as I
from util import assert_normwise, assert_within, U16, U32, log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def dev(t2):
    return t2.dev.to(DEV)


def _unfused(X, W, act, I_):
    y = tpl.column_linear(X, W)
    if act == "swiglu":
        return tpl.swiglu_local(y[:, :I_], y[:, I_:], "swiglu")
    return tpl.swiglu_local(y, None, "gelu")


ACT_SHAPES = [
    (1, 1024, 448),      # one token tile, 4 waves
    (1, 8192, 1000),     # one token tile, 16 waves
    (1, 8192, 3584),     # decode gate|up shard (7168 rows): dot-product kernel
    (2, 8192, 3584),     # two tokens, two 8-row groups per part
    (3, 4104, 4100),     # three tokens, ragged K ranges, four row groups per part
    (3, 16384, 40),      # the largest staged K, one row per workgroup
    (8, 4096, 4100),     # SwiGLU on 8200 rows: dot-product kernel at 8 tokens; GELU not
    (5, 520, 130),       # ragged K range per wave, ragged rows
    (8, 8192, 3584),     # decode gate|up shard at 8 tokens: register kernel, 8 waves
    (13, 16384, 200),    # register kernel, 16 waves, ragged tokens
    (4, 3584, 4096),     # LDS-ring kernel, one token tile, one 4-row token group (8192 rows)
    (8, 3584, 4096),     # LDS-ring kernel, one token tile, two token row groups
    (11, 3584, 4096),    # LDS-ring kernel, one token tile, three token row groups
    (17, 4096, 1000),    # two token tiles; the plain call (2000 rows) splits them over workgroups
    (32, 4096, 3584),    # two token tiles, two row tiles per wave
    (33, 1024, 300),     # LDS-ring kernel, three token tiles
    (64, 3584, 264),     # LDS-ring kernel, four token tiles
    (64, 520, 3001),     # LDS-ring kernel, 12 gate|up pairs per workgroup, last one 1
    (40, 520, 2501),     # LDS-ring kernel, 3 token tiles: SwiGLU cut to 10 pairs, last 1
    (48, 264, 4999),     # LDS-ring kernel: GELU cut to 20 rows per workgroup, last 19
    (65, 1024, 448),     # prefill tile kernel, ragged tokens
    (300, 520, 1000),
    (1000, 2048, 700),
    (2048, 1024, 3584),  # 256x256 tiles
    (4000, 520, 5100),   # GELU: 256x320 tiles
    (1800, 264, 4700),   # GELU: 256x192 tiles; SwiGLU: 256x192 pairs (96 outputs each)
]


def _lip(act, g, u, ag, au):
    """Bounds on |d act/d g| and |d act/d u| over the box g +- ag, u +- au:
    SiLU' <= 1.0999 (its maximum, near g = 2.4), |SiLU(g)| <= |g| + 0.28,
    and GELU' = Phi(g) + g phi(g) <= 1.1289 (its maximum, near g = 1.41)."""
    if act == "swiglu":
        return 1.0999 * (np.abs(u) + au), np.abs(g) + ag + 0.28
    return 1.1289 + 0 * g, 0 * g


def _act_bound(act, g, u, ref, ag, au):
    """|h - act(g, u)| for h = RNE_bf16(fp32 act(g32, u32)), |g32 - g| <= ag,
    |u32 - u| <= au: the perturbation of the arguments (mean value theorem in
    each argument), the fp32 evaluation of the activation (relative error
    below (8 + |g|^2 + |g|) fp32 units: the exponential or erfc argument's
    rounding times its condition number), then one bf16 rounding."""
    lg, lu = _lip(act, g, u, ag, au)
    cond = 8 + np.abs(g) * np.abs(g) + np.abs(g)
    e = (lg * ag + lu * au) * (1 + 1e-3) + cond * U32 * (np.abs(ref) + lg * ag + lu * au)
    return U16 * (np.abs(ref) + e) + e + 1e-30


@pytest.mark.parametrize("act", ["swiglu", "gelu"])
@pytest.mark.parametrize("M,K,I_", ACT_SHAPES)
def test_column_linear_act(act, M, K, I_):
    log(f"column_linear_act {act} M={M} K={K} I={I_}")
    rows = 2 * I_ if act == "swiglu" else I_
    x = I.normal(40, "x", (M, K))
    w = I.normal(40, "w", (rows, K), 1.5 / np.sqrt(K))   # activation arguments of O(1)
    X, W = dev(x), dev(w)
    h = tpl.column_linear_act(X, W, act)
    ax = np.abs(x.ref)
    g = O.linear(x.ref, w.ref[:I_])
    ag = 1.01 * K * U32 * (ax @ np.abs(w.ref[:I_]).T)     # fp32 accumulation of exact products
    if act == "swiglu":
        u = O.linear(x.ref, w.ref[I_:])
        au = 1.01 * K * U32 * (ax @ np.abs(w.ref[I_:]).T)
    else:
        u, au = None, 0.0
    ref = O.local_activation(g, u, act)
    assert_within(h, ref, _act_bound(act, g, u if u is not None else 0 * g, ref, ag, au),
                  f"fused {act} vs activation of the exact projections")
    assert_normwise(h, ref, 1e-2, f"fused {act} vs oracle")
    # the unfused calls round g and u to bf16 before the activation
    hu = _unfused(X, W, act, I_)
    agu = U16 * (np.abs(g) + ag) + ag
    auu = U16 * (np.abs(u) + au) + au if act == "swiglu" else 0.0
    assert_within(hu, ref, _act_bound(act, g, u if u is not None else 0 * g, ref, agu, auu),
                  f"unfused {act} vs activation of the exact projections")


@pytest.mark.parametrize("act", ["swiglu", "gelu"])
@pytest.mark.parametrize("M,K,I_", [(1, 64, 40), (3, 520, 700), (40, 136, 130), (200, 264, 300),
                                    (11, 264, 4096),
                                    # 256x256 tiles (outputs staged through LDS when full):
                                    # SwiGLU full and ragged (GELU on 128x128 there), then both
                                    # full
                                    (4096, 136, 2048), (4000, 136, 2048), (4096, 136, 4096)])
def test_column_linear_act_integer(act, M, K, I_):
    """Integer inputs: every projection is an exact integer in float32, so the
    fused route's only roundings are the fp32 activation and one bf16 store;
    the unfused route first stores g and u as bf16 (integers above 256 round)."""
    log(f"column_linear_act int {act} M={M} K={K} I={I_}")
    rows = 2 * I_ if act == "swiglu" else I_
    x = I.uniform_int(41, "x", (M, K), -2, 2, dtype=torch.bfloat16)
    w = I.uniform_int(41, "w", (rows, K), -1, 1, dtype=torch.bfloat16)
    X, W = dev(x), dev(w)
    g = O.linear(x.ref, w.ref[:I_])
    u = O.linear(x.ref, w.ref[I_:]) if act == "swiglu" else None
    for name, h, gg, uu in (
            ("fused", tpl.column_linear_act(X, W, act), g, u),
            ("unfused", _unfused(X, W, act, I_), O.round_bf16(g),
             O.round_bf16(u) if u is not None else None)):
        ref = O.local_activation(gg, uu, act)
        cond = 8 + np.abs(gg) * np.abs(gg) + np.abs(gg)
        assert_within(h, ref, (U16 * (1 + 1e-5) + cond * U32) * np.abs(ref) + 1e-30, f"{name} {act}")


@pytest.mark.parametrize("act", ["swiglu", "gelu"])
@pytest.mark.parametrize("M,K,I_", [(1, 8192, 3584), (2, 520, 700), (3, 4104, 1000), (8, 8192, 3584),
                                    (4, 3584, 4096), (6, 4096, 4100)])
def test_fused_equals_activation_of_float32_sums(act, M, K, I_):
    """Decode routes (dot-product kernel at 1..3 tokens and at 4..8 on tall
    weights, register kernel, one-token-tile LDS ring): the fused call's
    float32 sums are the plain
    call's on the same weight (same K split), so its output is, bit for bit,
    the activation kernel applied to the float32 partials, rounded to bf16."""
    log(f"fused == act(fp32 partials) {act} M={M} K={K} I={I_}")
    rows = 2 * I_ if act == "swiglu" else I_
    X = dev(I.normal(43, "x", (M, K)))
    W = dev(I.normal(43, "w", (rows, K), 1.5 / np.sqrt(K)))
    h = tpl.column_linear_act(X, W, act)
    P = tpl.row_linear_partial(X, W)
    a = tpl.swiglu_local(P[:, :I_], P[:, I_:] if act == "swiglu" else None, act)
    expect = O.round_bf16(a.cpu().numpy().astype(np.float64))
    got = h.float().cpu().numpy().astype(np.float64)
    assert np.array_equal(got, expect), f"{np.sum(got != expect)} of {got.size} differ"


def test_column_linear_act_none_is_column_linear():
    x = dev(I.normal(42, "x", (9, 256)))
    w = dev(I.normal(42, "w", (100, 256), 0.05))
    assert torch.equal(tpl.column_linear_act(x, w, "none"), tpl.column_linear(x, w))


def test_column_linear_act_rejects_unsupported():
    x = torch.zeros(4, 12, dtype=torch.bfloat16, device=DEV)      # K % 8 != 0
    w = torch.zeros(16, 12, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(tpl.TPError):
        tpl.column_linear_act(x, w, "swiglu")
    xf = torch.zeros(4, 16, dtype=torch.float32, device=DEV)
    wf = torch.zeros(16, 16, dtype=torch.float32, device=DEV)
    with pytest.raises(tpl.TPError):
        tpl.column_linear_act(xf, wf, "gelu")


_DT = {"bf16": torch.bfloat16, "f32": torch.float32}


@pytest.mark.parametrize("R", [1, 2, 8])
@pytest.mark.parametrize("M,N", [(1, 8192), (7, 4096), (300, 1024), (3, 8), (5, 100), (2, 14344), (2, 20480)])
@pytest.mark.parametrize("res,ydt", [(None, "bf16"), ("bf16", "bf16"), ("bf16", "f32"),
                                     ("f32", "f32"), ("f32", "bf16"), (None, "f32")])
def test_reduce_partials_rmsnorm(R, M, N, res, ydt):
    """The layer's step after the attention partials: a bf16 input x plus the
    partials into a float32 residual stream h, and h normalised to bf16 (the
    ("bf16", "f32") case); the other storage pairs take the same kernels."""
    log(f"reduce_partials_rmsnorm R={R} M={M} N={N} residual={res} y={ydt}")
    parts = [I.normal(43, "p", (M, N), 1.0, dtype=torch.float32, rank=r) for r in range(R)]
    resid = I.normal(43, "res", (M, N), 2.0, dtype=_DT[res]) if res else None
    gam = I.normal(43, "gamma", (N,), 1.0)
    P = [dev(p) for p in parts]
    RES = dev(resid) if res else None
    G = dev(gam)
    y, yn = tpl.reduce_partials_rmsnorm(P, G, residual=RES, eps=1e-5, out_dtype=_DT[ydt])
    assert y.dtype == _DT[ydt] and yn.dtype == torch.bfloat16
    y2 = tpl.reduce_partials(P, residual=RES, out_dtype=_DT[ydt])
    yn2 = tpl.rmsnorm(y2, G, 1e-5)
    assert torch.equal(y, y2), "sum differs from tp_reduce_partials"
    assert torch.equal(yn, yn2), "norm differs from tp_rmsnorm"
    ref_y = O.reduce_partials([p.ref for p in parts], residual=resid.ref if res else None)
    ay = sum(np.abs(p.ref) for p in parts) + (np.abs(resid.ref) if res else 0)
    uy = U16 if ydt == "bf16" else U32
    bound_y = uy * (np.abs(ref_y) + R * U32 * ay) + (R + 1) * U32 * ay + 1e-30
    assert_within(y, ref_y, bound_y, "sum vs oracle")
    assert_normwise(yn, O.rmsnorm(ref_y, gam.ref, 1e-5), 1e-2, "norm vs oracle")


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_reduce_partials_rmsnorm_in_place_residual(dt):
    """y may be the residual buffer itself (the residual stream updated in
    place) when the two share a storage type."""
    M, N = 33, 2048
    P = [dev(I.normal(44, "p", (M, N), 1.0, dtype=torch.float32, rank=r)) for r in range(4)]
    res = dev(I.normal(44, "res", (M, N), dtype=dt))
    G = dev(I.normal(44, "gamma", (N,)))
    y, yn = tpl.reduce_partials_rmsnorm(P, G, residual=res.clone(), out_dtype=dt)
    buf = res.clone()
    y2, yn2 = tpl.reduce_partials_rmsnorm(P, G, residual=buf, out=buf)
    assert y2.data_ptr() == buf.data_ptr()
    assert torch.equal(y, y2) and torch.equal(yn, yn2)
