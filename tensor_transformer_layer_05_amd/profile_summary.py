"""Turn the rocprofv3 outputs of the profiling runs into the text summaries
kept in ``profiles/`` (no measurement happens here; it only reads CSV files).

    python3 -m tensor_transformer_layer_05_amd.profile_summary <out_dir>

``<out_dir>`` holds ``prof_bench/`` (kernel trace + stats of a bench run, with
``prof_bench.log`` beside it), ``pmc_fetch/`` and ``pmc_write/`` (FETCH_SIZE and
WRITE_SIZE runs of ``profile_drivers gemm_traffic``)."""
from __future__ import annotations

import collections
import csv
import glob
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GEMM_SRCS = ["tensor_transformer_layer_05_amd/csrc/gemm_dma.hip",
             "tensor_transformer_layer_05_amd/csrc/common.h"]
FUSED = "DmaTile<256, 256, 2, 4>, false, true, 1>"


def _od(out):
    """The raw-output directory as it appears in the commands of a summary
    (the directory the summary script was given)."""
    return os.path.normpath(out)


def _csv(pattern):
    files = glob.glob(pattern, recursive=True)
    if not files:
        raise FileNotFoundError(pattern)
    return list(csv.DictReader(open(files[0])))


def _counters(d):
    agg = collections.OrderedDict()
    for r in _csv(os.path.join(d, "**", "*counter_collection.csv")):
        k = (int(r["Dispatch_Id"]), r["Kernel_Name"])
        agg[k] = agg.get(k, 0.0) + float(r["Counter_Value"])
    return agg


def traffic(out):
    fetch, write = _counters(os.path.join(out, "pmc_fetch")), _counters(os.path.join(out, "pmc_write"))

    def pick(agg, needle):
        return [v for (i, n), v in sorted(agg.items()) if needle in n]
    cf, cw = pick(fetch, "copyBuffer")[0], pick(write, "copyBuffer")[0]
    gemm_f = pick(fetch, "gemm_bf16_dma_kernel")
    gemm_w = pick(write, "gemm_bf16_dma_kernel")
    fs, ws = 262144.0 / cf, 262144.0 / cw
    S, H, il = 4096, 8192, 14336
    alg_fused = (S * H + 2 * il * H + S * il) * 2
    alg_plain = (S * H + 2 * il * H + S * 2 * il) * 2
    tf = (gemm_f[0] * fs + gemm_w[0] * ws) * 1024
    tp = (gemm_f[1] * fs + gemm_w[1] * ws) * 1024
    h = hashlib.sha256()
    for f in GEMM_SRCS:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    sha = h.hexdigest()[:16]
    data = {"kernel": "gemm_bf16_dma_kernel<DmaTile<256,256,2,4>,false,true,1> (SwiGLU epilogue)",
            "shape_mkn": [S, H, 2 * il], "sources": GEMM_SRCS, "sources_sha256_16": sha,
            "fetch_kib": round(gemm_f[0], 1), "write_kib": round(gemm_w[0], 1),
            "copy_fetch_kib": round(cf, 1), "copy_write_kib": round(cw, 1),
            "fetch_scale": round(fs, 4), "write_scale": round(ws, 4),
            "traffic_bytes": int(tf), "algorithmic_bytes": alg_fused}
    return f"""# HBM traffic of the gate|up projection (rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE)

Commands (from the repository root; the driver runs one plain 256 MiB device-to-device copy, then one
gate|up launch with the SwiGLU epilogue, then one plain gate|up launch; M=4096 K=8192 2I=28672 bf16):

```
rocprofv3 --pmc FETCH_SIZE --output-format csv -d {_od(out)}/pmc_fetch -o f -- python3 -m tensor_transformer_layer_05_amd.profile_drivers gemm_traffic
rocprofv3 --pmc WRITE_SIZE --output-format csv -d {_od(out)}/pmc_write -o w -- python3 -m tensor_transformer_layer_05_amd.profile_drivers gemm_traffic
python3 -m tensor_transformer_layer_05_amd.profile_summary {_od(out)}
```

| dispatch | FETCH_SIZE KiB | WRITE_SIZE KiB |
|---|---:|---:|
| plain copy, 256 MiB read + 256 MiB written | {cf:.1f} | {cw:.1f} |
| gate\\|up + SwiGLU epilogue (output [4096, 14336]) | {gemm_f[0]:.1f} | {gemm_w[0]:.1f} |
| plain gate\\|up (output [4096, 28672]) | {gemm_f[1]:.1f} | {gemm_w[1]:.1f} |

Calibration: the copy moves 262144 KiB each way, so FETCH_SIZE is scaled by {fs:.4f} and WRITE_SIZE by {ws:.4f}.

- Fused launch: {tf / 1e9:.3f} GB (algorithmic {alg_fused / 1e9:.3f} GB: X and W read once, act(g)*u written once).
- Plain launch: {tp / 1e9:.3f} GB (algorithmic {alg_plain / 1e9:.3f} GB).
- The epilogue saves the write of the [4096, 28672] intermediate and the SwiGLU pass that read it back.
- FETCH_SIZE counts reads that miss an XCD's L2; they may still hit the Infinity Cache. Each XCD runs 7
  successive rounds of 32 tiles (4 M-tiles x 8 N-tiles), and its 4 MB L2 holds only the k-slices in flight,
  so every round fetches its 4 X and 8 W row blocks (4 MB each) again: 8 XCDs x 7 rounds x 48 MB = 2.69 GB
  of reads plus 0.12 GB of output is the floor for this tile order. The rest of the excess is small.

bench.py reports `roofline.traffic` from the line below only while the kernel's sources still have this hash.

DATA {json.dumps(data)}
"""


def kernel_stats(out):
    rows = _csv(os.path.join(out, "prof_bench", "**", "*kernel_stats.csv"))
    trace = _csv(os.path.join(out, "prof_bench", "**", "*kernel_trace.csv"))
    bench = [l for l in open(os.path.join(out, "prof_bench.log")) if l.startswith('{"metric"')][0]
    d = json.loads(bench)
    f = sorted((r for r in trace if FUSED in r["Kernel_Name"]), key=lambda r: int(r["Start_Timestamp"]))
    durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in f]
    # launch order: set-up, warm-up, the timed steps, then as many steps with
    # an event pair around every call (the per-call breakdown)
    timed = durs[-2 * d["steps"]:-d["steps"]]
    lines = []
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        name = r["Name"].replace("void ", "")
        name = name[:name.rfind("(")] if name.endswith(")") else name   # drop the parameter list
        lines.append(f'| `{name[:100]}` | {r["Calls"]} | {float(r["AverageNs"]) / 1e3:.1f} | '
                     f'{float(r["MinNs"]) / 1e3:.1f} | {float(r["MaxNs"]) / 1e3:.1f} | {float(r["Percentage"]):.2f} |')
    return f"""# Kernel stats: bench.py (prefill layer shard + decode shards), rocprofv3 --kernel-trace --stats

Command (from /tmp with TMPDIR=/tmp; REPO = repository root), then the summary script:

```
rocprofv3 --kernel-trace --stats --output-format csv -d $REPO/{_od(out)}/prof_bench -o bench -- python3 $REPO/bench.py --steps 5 --warmup 2 --no-cpu-baseline
python3 -m tensor_transformer_layer_05_amd.profile_summary {_od(out)}
```

The bench line of the same run (under the profiler): value {d['value']} TFLOP/s, {d['ms_per_step']} ms per step;
the dominant kernel's event-timed average {d['roofline']['avg_launch_ms'] * 1e3:.1f} us. From the trace of the same
run, the {len(timed)} timed-step launches of that kernel (`gemm_bf16_dma_kernel<..., 1>`, launches
{len(durs) - 2 * len(timed) + 1}-{len(durs) - len(timed)} of its {len(durs)}; the last {len(timed)} are the per-call breakdown pass) average
{sum(timed) / len(timed):.1f} us ({', '.join(f'{x:.1f}' for x in timed)}); the table's averages include the set-up and
warm-up launches.

| kernel | calls | avg us | min us | max us | % time |
|---|---:|---:|---:|---:|---:|
""" + "\n".join(lines) + """

Mapping (prefill calls = 2 set-up passes over both ranks + 2 warm-up + 5 timed steps + 5 breakdown steps = 14
per rank-0 call):
- `gemm_bf16_dma_kernel<DmaTile<256,256,2,4>, false, true, 1>`: gate|up with the SwiGLU epilogue, M=4096 K=8192
  2I=28672 -> [4096, 14336].
- `gemm_bf16_dma_kernel<DmaTile<256,256,2,4>, true, true, 0>`: o_proj (K=4096) and down (K=14336), fp32 partials.
- `gemm_bf16_dma_kernel<DmaTile<256,320,4,2>, false, true, 0>`: fused QKV, N=5120 (16 x 16 tiles).
- `attn_prefill_tr_kernel`: causal 4096-token attention over 32 local q heads / 4 KV heads.
- `reduce_rmsnorm_reg_kernel<4>`: sum of the two ranks' attention partials + residual, then the MLP's RMSNorm.
- `reduce_kernel`, `rmsnorm_reg_kernel<4>`: the final sum of MLP partials; the first RMSNorm.
- `gemv_dot_kernel<...>`: decode linears with 1..3 tokens, and 4..8 tokens on weights of more than 8192 rows (the
  lm_head shard); `gemm_stream_kernel<*, 1, *, *, *>`: 4..16 tokens on the decode gate|up weight;
  `gemm_stream_dma_kernel<...>`: the other decode linears up to 64 tokens
  (weights and tokens through the per-wave LDS ring).
- `attn_decode_kernel<false|true>` + `attn_decode_combine_kernel`: decode attention (contiguous / paged cache).
- `vocab_argmax_kernel`: the lm_head shard's local greedy step.
- `gemm_bf16_dma_kernel<DmaTile<256,192,4,2>, false, true, 2>`: the GELU FFN's fc1 with GELU in its epilogue
  (M=2048 K=12288 N=6144, 8 x 32 tiles); `<..., true, true, 0>`: its fc2 to fp32 partials (N=12288).
- `reduce_kernel<true, true>` also runs the sum of the FFN's 8 partials.
- `stream_read_kernel<...>` (libtpref, measurement only): the plain read-only stream behind `hbm_read_ceiling`
  and each decode shard's `size_stream_ms` (every configuration warmed with 100 ms of back-to-back calls).

Decode calls come from the eager and graph-replayed decode figures; kernel durations are per launch.
"""


def _dispatches(d):
    """dispatch id -> (kernel name, duration us, {counter: value}) of one --pmc run."""
    out = collections.OrderedDict()
    for r in _csv(os.path.join(d, "**", "*counter_collection.csv")):
        i = int(r["Dispatch_Id"])
        if i not in out:
            out[i] = (r["Kernel_Name"], (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3, {})
        c = out[i][2]
        c[r["Counter_Name"]] = c.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return out


def counters(out):
    """MFMA and LDS counters of the fused gate|up launch (and the copy), from
    two --pmc runs of the gemm_traffic driver.  GRBM_GUI_ACTIVE is summed over
    the 8 XCDs here, so GUI_ACTIVE / 8 / duration is the clock the chip ran
    during the dispatch; MFMA utilisation = SQ_VALU_MFMA_BUSY_CYCLES / (GUI_ACTIVE
    per XCD x 1024 SIMDs), the MfmaUtil expression rocprofv3 lists."""
    m, l = _dispatches(os.path.join(out, "pmc_mfma")), _dispatches(os.path.join(out, "pmc_lds"))
    gm = [v for v in m.values() if FUSED in v[0].replace("tpl::", "")][0]
    gl = [v for v in l.values() if FUSED in v[0].replace("tpl::", "")][0]
    cp = [v for v in m.values() if "copyBuffer" in v[0]][0]
    xcd, simds, cus = 8, 1024, 256
    gui = gm[2]["GRBM_GUI_ACTIVE"] / xcd
    clk = gui / gm[1] / 1e3
    clk_copy = cp[2]["GRBM_GUI_ACTIVE"] / xcd / cp[1] / 1e3
    flops = gm[2]["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512
    util = gm[2]["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui * simds)
    lds_active = gl[2]["SQ_LDS_IDX_ACTIVE"] / (gl[2]["GRBM_GUI_ACTIVE"] / xcd * cus)
    h = hashlib.sha256()
    for f in GEMM_SRCS:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    data = {"kernel": "gemm_bf16_dma_kernel<DmaTile<256,256,2,4>,false,true,1> (SwiGLU epilogue)",
            "sources": GEMM_SRCS, "sources_sha256_16": h.hexdigest()[:16],
            "mfma_flop_counted": flops, "mfma_util": round(util, 4), "sclk_ghz": round(clk, 3),
            "lds_idx_active": round(lds_active, 4), "lds_bank_conflicts": gl[2]["SQ_LDS_BANK_CONFLICT"]}
    return f"""# MFMA and LDS counters of the gate|up projection (rocprofv3 --pmc, two runs)

Commands (from the repository root), then the summary script:

```
rocprofv3 --pmc SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES GRBM_GUI_ACTIVE --output-format csv -d {_od(out)}/pmc_mfma -o m -- python3 -m tensor_transformer_layer_05_amd.profile_drivers gemm_traffic
rocprofv3 --pmc SQ_LDS_IDX_ACTIVE SQ_LDS_BANK_CONFLICT SQ_INSTS_LDS SQ_WAIT_INST_LDS GRBM_GUI_ACTIVE --output-format csv -d {_od(out)}/pmc_lds -o l -- python3 -m tensor_transformer_layer_05_amd.profile_drivers gemm_traffic
python3 -m tensor_transformer_layer_05_amd.profile_summary {_od(out)}
```

Fused gate|up launch (M=4096, K=8192, 2I=28672, SwiGLU epilogue), as profiled: {gm[1]:.1f} us.

| quantity | value |
|---|---:|
| bf16 MFMA FLOP counted (`SQ_INSTS_VALU_MFMA_MOPS_BF16` x 512) | {flops / 1e12:.4f} T (algorithmic 1.9241 T) |
| `GRBM_GUI_ACTIVE` per XCD | {gui:.4g} cycles |
| engine clock estimate (GUI_ACTIVE per XCD / duration) | {clk:.2f} GHz (the 256 MiB copy in the same run: {clk_copy:.2f} GHz, above the 2.4 GHz maximum: for a short dispatch the counter window extends past the kernel) |
| MFMA busy (`SQ_VALU_MFMA_BUSY_CYCLES` / (GUI_ACTIVE per XCD x 1024 SIMDs)) | {100 * util:.1f}% |
| LDS index-active (`SQ_LDS_IDX_ACTIVE` / (GUI_ACTIVE per XCD x 256 CUs)) | {100 * lds_active:.1f}% |
| LDS bank conflicts (`SQ_LDS_BANK_CONFLICT`) | {gl[2]["SQ_LDS_BANK_CONFLICT"]:.0f} |

The counted MFMA work equals the algorithmic FLOPs. The MFMA pipes are busy {100 * util:.0f}% of the counted cycles
(rocprofv3's MfmaUtil expression), while the launch reaches about half of the 2.5 PFLOP/s peak: the engine
clock under this load is far below the 2.4 GHz that the published peak assumes.

bench.py reports these figures next to the roofline only while the kernel's sources still have this hash.

DATA {json.dumps(data)}
"""


VENDOR_PASSES = [
    "SQ_INSTS_VALU SQ_INSTS_SALU SQ_INSTS_LDS SQ_INSTS_VMEM_RD SQ_INSTS_MFMA SQ_INSTS_SMEM SQ_INSTS_BRANCH "
    "SQ_WAVES TA_BUFFER_READ_LDS_WAVEFRONTS TA_BUFFER_READ_WAVEFRONTS GRBM_GUI_ACTIVE",
    "SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES SQ_WAIT_INST_LDS SQ_WAIT_INST_ANY SQ_WAVE_CYCLES "
    "SQ_INST_LEVEL_VMEM SQ_ACTIVE_INST_VMEM SQ_ACTIVE_INST_LDS GRBM_GUI_ACTIVE TA_TA_BUSY "
    "TA_ADDR_STALLED_BY_TC_CYCLES",
    "SQ_LDS_IDX_ACTIVE SQ_LDS_BANK_CONFLICT SQ_INSTS_LDS_LOAD_BANDWIDTH SQ_LDS_DATA_FIFO_FULL "
    "SQ_LDS_CMD_FIFO_FULL SQ_VMEM_TA_ADDR_FIFO_FULL SQ_VMEM_TA_CMD_FIFO_FULL SQ_ACTIVE_INST_VALU "
    "GRBM_GUI_ACTIVE TA_DATA_STALLED_BY_TC_CYCLES TA_BUFFER_TOTAL_CYCLES TCP_PENDING_STALL_CYCLES "
    "TCP_READ_TAGCONFLICT_STALL_CYCLES",
]


def vendor_counters(out):
    """The vendor GEMM (torch.matmul) against the library's plain gate|up GEMM
    on the same operands, from three --pmc runs of the vendor_gemm driver.
    Every ratio is formed within one dispatch (each run counts
    GRBM_GUI_ACTIVE, summed over the 8 XCDs); the tables give the median over
    the kernel's launches."""
    import statistics
    xcd, simds, cus = 8, 1024, 256
    ratios = {   # label -> (counter, denominator: "simd" | "cu" | "ghz" | "lds" | None, format)
        "engine clock (GUI_ACTIVE per XCD / launch duration)": ("GRBM_GUI_ACTIVE", "ghz", "{:.2f} GHz"),
        "MFMA busy (SQ_VALU_MFMA_BUSY_CYCLES / (GUI_ACTIVE per XCD x 1024 SIMDs))":
            ("SQ_VALU_MFMA_BUSY_CYCLES", "simd", "{:.1f}%"),
        "LDS index-active (SQ_LDS_IDX_ACTIVE / (GUI_ACTIVE per XCD x 256 CUs))": ("SQ_LDS_IDX_ACTIVE", "cu", "{:.1f}%"),
        "LDS bank-conflict cycles / LDS index-active cycles": ("SQ_LDS_BANK_CONFLICT", "lds", "{:.2f}"),
        "LDS command FIFO full (SQ_LDS_CMD_FIFO_FULL / (GUI_ACTIVE per XCD x 256 CUs))":
            ("SQ_LDS_CMD_FIFO_FULL", "cu", "{:.2f}%"),
        "TA busy (TA_TA_BUSY / (GUI_ACTIVE per XCD x 256 CUs))": ("TA_TA_BUSY", "cu", "{:.1f}%"),
        "TA address stalled by the L1 (TA_ADDR_STALLED_BY_TC_CYCLES, same)":
            ("TA_ADDR_STALLED_BY_TC_CYCLES", "cu", "{:.1f}%"),
        "waves per launch (SQ_WAVES)": ("SQ_WAVES", None, "{:.0f}"),
        "direct-to-LDS buffer loads (TA_BUFFER_READ_LDS_WAVEFRONTS)": ("TA_BUFFER_READ_LDS_WAVEFRONTS", None, "{:.4g}"),
        "LDS bytes read (SQ_INSTS_LDS_LOAD_BANDWIDTH x 64)": ("SQ_INSTS_LDS_LOAD_BANDWIDTH", 64e-9, "{:.1f} GB"),
        "MFMA instructions (SQ_INSTS_MFMA)": ("SQ_INSTS_MFMA", None, "{:.4g}"),
    }
    vals = {"vendor": collections.defaultdict(list), "library": collections.defaultdict(list)}
    raw = {"vendor": collections.defaultdict(list), "library": collections.defaultdict(list)}
    names = {}
    for i in range(len(VENDOR_PASSES)):
        for name, us, cs in _dispatches(os.path.join(out, f"pmc_vendor{i + 1}")).values():
            k = "vendor" if "Cijk" in name else "library" if "gemm_bf16_dma" in name else None
            if k is None:
                continue
            names[k] = name
            raw[k]["duration_us"].append(us)
            for c, v in cs.items():
                raw[k][c].append(v)
            gui = cs.get("GRBM_GUI_ACTIVE", 0.0) / xcd
            for label, (c, den, _) in ratios.items():
                if c not in cs or (den in ("simd", "cu", "ghz") and not gui):
                    continue
                v = cs[c]
                if den == "simd":
                    v = 100 * v / (gui * simds)
                elif den == "cu":
                    v = 100 * v / (gui * cus)
                elif den == "ghz":
                    v = gui / us / 1e3
                elif den == "lds":
                    v = v / cs["SQ_LDS_IDX_ACTIVE"]
                elif den is not None:
                    v = v * den
                vals[k][label].append(v)
    med = {k: {c: statistics.median(v) for c, v in d.items()} for k, d in vals.items()}
    rmed = {k: {c: statistics.median(v) for c, v in d.items()} for k, d in raw.items()}
    rows = "\n".join(f"| {q} | {f.format(med['vendor'][q])} | {f.format(med['library'][q])} |"
                     for q, (_, _, f) in ratios.items())
    craw = sorted(set(rmed["vendor"]) | set(rmed["library"]))
    raw_rows = "\n".join(f"| `{c}` | {rmed['vendor'].get(c, 0):.4g} | {rmed['library'].get(c, 0):.4g} |" for c in craw)
    cmds = "\n".join(f"rocprofv3 --pmc {p} --output-format csv -d $REPO/{_od(out)}/pmc_vendor{i + 1} -o v -- "
                      f"python3 -m tensor_transformer_layer_05_amd.profile_drivers vendor_gemm"
                      for i, p in enumerate(VENDOR_PASSES))
    data = {"vendor_kernel": names.get("vendor"), "library_kernel": names.get("library"),
            "ratios": med, "counters": rmed}
    return f"""# The plain gate|up GEMM: vendor library against this library (rocprofv3 --pmc, three runs)

Commands (from /tmp with TMPDIR=/tmp and PYTHONPATH=$REPO, REPO = repository root; each under
`timeout -s KILL 90`), then the summary script (from the repository root):

```
{cmds}
python3 -m tensor_transformer_layer_05_amd.profile_summary {_od(out)} gate_up_vendor_counters
```

M=4096, K=8192, N=28672, bf16 in and out, the same operands for both. Three launches of each kernel per
run; ratios are formed within a dispatch, then the median is taken over the kernel's nine dispatches.
Vendor kernel (torch.matmul): `{names.get("vendor")}`.
Library kernel: `{names.get("library")}`.

| quantity | vendor | library |
|---|---:|---:|
| launch duration, as profiled (counters slow both) | {rmed['vendor']['duration_us']:.1f} us | {rmed['library']['duration_us']:.1f} us |
{rows}

All counters, medians over the kernel's launches (sums over the XCDs, shader engines and CUs):

| counter | vendor | library |
|---|---:|---:|
{raw_rows}

DATA {json.dumps(data)}
"""


FFN_SQ_PASS = ("SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES SQ_LDS_IDX_ACTIVE "
               "SQ_LDS_BANK_CONFLICT GRBM_GUI_ACTIVE")
FFN_PASSES = [("pmc_ffn_fetch", "FETCH_SIZE"), ("pmc_ffn_write", "WRITE_SIZE"), ("pmc_ffn_sq", FFN_SQ_PASS)]


def ffn_counters(out):
    """HBM bytes, MFMA and LDS counters of the GELU FFN shard's fc1 (GELU
    epilogue) and fc2 (float32 partials), three launches each, from three
    --pmc runs of the ffn_gemms driver.  Traffic = FETCH_SIZE and WRITE_SIZE
    scaled by what they read for the driver's 256 MiB copy; every other ratio
    is formed within one dispatch; the table gives medians over the launches."""
    import statistics
    xcd, simds, cus = 8, 1024, 256
    M, H, F = 2048, 12288, 6144
    kinds = {"fc1": "false, true, 2>", "fc2": "true, true, 0>"}
    alg = {"fc1": {"flop": 2.0 * M * H * F, "bytes": (M * H + F * H + M * F) * 2},
           "fc2": {"flop": 2.0 * M * F * H, "bytes": (M * F + H * F) * 2 + M * H * 4}}
    runs = {d: _dispatches(os.path.join(out, d)) for d, _ in FFN_PASSES}

    def copy_of(d):
        return [cs for n, us, cs in runs[d].values() if "copyBuffer" in n][0]
    fs = 262144.0 / copy_of("pmc_ffn_fetch")["FETCH_SIZE"]
    ws = 262144.0 / copy_of("pmc_ffn_write")["WRITE_SIZE"]
    vals = {k: collections.defaultdict(list) for k in kinds}
    names = {}
    for d, _ in FFN_PASSES:
        for name, us, cs in runs[d].values():
            k = next((k for k, t in kinds.items() if "gemm_bf16_dma_kernel" in name and t in name), None)
            if k is None:
                continue
            names[k] = name
            v = vals[k]
            if d == "pmc_ffn_sq":
                v["duration_us"].append(us)
                gui = cs["GRBM_GUI_ACTIVE"] / xcd
                v["clock_ghz"].append(gui / us / 1e3)
                v["mfma_busy"].append(cs["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui * simds))
                v["lds_idx_active"].append(cs["SQ_LDS_IDX_ACTIVE"] / (gui * cus))
                v["lds_bank_conflicts"].append(cs["SQ_LDS_BANK_CONFLICT"])
                v["mfma_flop_counted"].append(cs["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512)
            elif d == "pmc_ffn_fetch":
                v["fetch_bytes"].append(cs["FETCH_SIZE"] * fs * 1024)
            else:
                v["write_bytes"].append(cs["WRITE_SIZE"] * ws * 1024)
    med = {k: {c: statistics.median(x) for c, x in d.items()} for k, d in vals.items()}
    for k in kinds:
        m = med[k]
        m["traffic_bytes"] = m["fetch_bytes"] + m["write_bytes"]
        m["tflops_as_profiled"] = alg[k]["flop"] / m["duration_us"] / 1e6
        m["algorithmic_bytes"] = alg[k]["bytes"]
    cmds = "\n".join(f"timeout -s KILL 90 rocprofv3 --pmc {p} --output-format csv -d $REPO/{_od(out)}/{d} -o f -- "
                      f"python3 -m tensor_transformer_layer_05_amd.profile_drivers ffn_gemms"
                      for d, p in FFN_PASSES)

    def row(label, key, fmt):
        return f"| {label} | {fmt.format(med['fc1'][key])} | {fmt.format(med['fc2'][key])} |"
    rows = "\n".join([
        row("launch duration, as profiled (counters slow it)", "duration_us", "{:.1f} us"),
        row("rate as profiled", "tflops_as_profiled", "{:.0f} TFLOP/s"),
        row("engine clock (GUI_ACTIVE per XCD / duration)", "clock_ghz", "{:.2f} GHz"),
        row("MFMA busy (SQ_VALU_MFMA_BUSY_CYCLES / (GUI_ACTIVE per XCD x 1024 SIMDs))", "mfma_busy", "{:.1%}"),
        row("bf16 MFMA FLOP counted (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512)", "mfma_flop_counted", "{:.4g}"),
        row("LDS index-active (SQ_LDS_IDX_ACTIVE / (GUI_ACTIVE per XCD x 256 CUs))", "lds_idx_active", "{:.1%}"),
        row("LDS bank conflicts (SQ_LDS_BANK_CONFLICT)", "lds_bank_conflicts", "{:.0f}"),
        row("HBM bytes read (FETCH_SIZE, scaled)", "fetch_bytes", "{:.4g}"),
        row("HBM bytes written (WRITE_SIZE, scaled)", "write_bytes", "{:.4g}"),
        row("algorithmic bytes (operands once, output once)", "algorithmic_bytes", "{:.4g}"),
    ])
    data = {"kernels": names, "fetch_scale": round(fs, 4), "write_scale": round(ws, 4), "medians": med}
    return f"""# The GELU FFN shard's GEMMs at TP=8: HBM bytes, MFMA and LDS counters (rocprofv3 --pmc, three runs)

Commands (from /tmp with TMPDIR=/tmp and PYTHONPATH=$REPO, REPO = repository root), then the summary script
(from the repository root):

```
{cmds}
python3 -m tensor_transformer_layer_05_amd.profile_summary {_od(out)} ffn_gemm_counters
```

Rank 0 of the GELU FFN at TP=8: fc1 = [2048, 12288] x [6144, 12288]^T with GELU in the epilogue (bf16 out),
fc2 = [2048, 6144] x [12288, 6144]^T to float32 partials; both on 256x192 tiles (fc1: 8 x 32 tiles, one
round on 256 CUs; fc2: 8 x 64 tiles, two rounds). 309.2 GFLOP each. Three launches of each per run; the
traffic is scaled by what the counters read for a 256 MiB copy in the same run (FETCH_SIZE x {fs:.4f},
WRITE_SIZE x {ws:.4f}); the other ratios are formed within a dispatch; medians over the launches.

| quantity | fc1 + GELU | fc2 |
|---|---:|---:|
{rows}

DATA {json.dumps(data)}
"""


ATTN_PASS = ("SQ_INSTS_VALU SQ_INSTS_MFMA SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_TRANS_F32 SQ_INSTS_LDS "
             "SQ_INSTS_SALU SQ_WAVES SQ_BUSY_CU_CYCLES GRBM_GUI_ACTIVE")


def attention_counters(out):
    """Instruction mix and MFMA utilisation of the prefill attention launch
    (one --pmc run of the prefill_attention driver; medians over its three
    launches, every ratio formed within a dispatch)."""
    import statistics
    xcd, simds = 8, 1024
    S, hq, D = 4096, 32, 128
    vals = collections.defaultdict(list)
    name = None
    for nm, us, cs in _dispatches(os.path.join(out, "pmc_attn")).values():
        if "attn_prefill" not in nm:
            continue
        name = nm
        gui = cs["GRBM_GUI_ACTIVE"] / xcd
        vals["duration_us"].append(us)
        vals["clock"].append(gui / us / 1e3)
        vals["mfma_busy"].append(cs["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui * simds))
        vals["valu_per_mfma"].append(cs["SQ_INSTS_VALU"] / cs["SQ_INSTS_MFMA"])
        vals["trans_per_mfma"].append(cs["SQ_INSTS_VALU_TRANS_F32"] / cs["SQ_INSTS_MFMA"])
        vals["lds_per_mfma"].append(cs["SQ_INSTS_LDS"] / cs["SQ_INSTS_MFMA"])
        vals["mfma"].append(cs["SQ_INSTS_MFMA"])
        vals["valu"].append(cs["SQ_INSTS_VALU"])
        vals["waves"].append(cs["SQ_WAVES"])
    m = {k: statistics.median(v) for k, v in vals.items()}
    fl = 4.0 * S * S / 2 * hq * D   # QK^T and PV over the causal half of the score matrix
    data = {"kernel": name, "medians": m, "pass": ATTN_PASS}
    return f"""# Prefill attention of the TP=2 layer shard: instruction mix (rocprofv3 --pmc)

Command (from /tmp with TMPDIR=/tmp and PYTHONPATH=$REPO, REPO = repository root), then the summary script
(from the repository root):

```
timeout -s KILL 90 rocprofv3 --pmc {ATTN_PASS} --output-format csv -d $REPO/{_od(out)}/pmc_attn -o a -- python3 -m tensor_transformer_layer_05_amd.profile_drivers prefill_attention
python3 -m tensor_transformer_layer_05_amd.profile_summary {_od(out)} prefill_attention_counters
```

One sequence of 4096 tokens, causal, 32 q / 4 KV heads of 128 on strided views of the fused QKV output;
medians over three launches of `{name}`.

| quantity | value |
|---|---:|
| launch duration, as profiled | {m['duration_us']:.1f} us ({fl / m['duration_us'] / 1e6:.0f} TFLOP/s on the causal half, {fl / 1e12:.3f} TFLOP) |
| engine clock (GUI_ACTIVE per XCD / duration) | {m['clock']:.2f} GHz |
| MFMA busy (`SQ_VALU_MFMA_BUSY_CYCLES` / (GUI_ACTIVE per XCD x 1024 SIMDs)) | {100 * m['mfma_busy']:.1f}% |
| MFMA instructions (`SQ_INSTS_MFMA`) | {m['mfma']:.4g} |
| VALU instructions per MFMA (`SQ_INSTS_VALU` / `SQ_INSTS_MFMA`; the VALU count includes the MFMAs) | {m['valu_per_mfma']:.2f} |
| fp32 transcendental instructions per MFMA (`SQ_INSTS_VALU_TRANS_F32`) | {m['trans_per_mfma']:.3f} |
| LDS instructions per MFMA | {m['lds_per_mfma']:.3f} |
| waves per launch | {m['waves']:.0f} |

DATA {json.dumps(data)}
"""


def decode_span(out):
    from .profile_drivers import SPANS
    trace = _csv(os.path.join(out, "prof_span", "**", "*kernel_trace.csv"))
    ks = sorted((r for r in trace if "attn_decode" in r["Kernel_Name"]), key=lambda r: int(r["Start_Timestamp"]))
    dur = lambda r: (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    main_ = [r for r in ks if "combine" not in r["Kernel_Name"]]
    comb = [r for r in ks if "combine" in r["Kernel_Name"]]
    n = len(main_) // len(SPANS)
    lines, prev = [], None
    for i, L in enumerate(SPANS):
        m = sorted(dur(r) for r in main_[i * n:(i + 1) * n])[n // 2]
        c = sorted(dur(r) for r in comb[i * n:(i + 1) * n])[n // 2]
        byts = 2 * 32 * L * 2 * 128 * 2
        marg = "" if prev is None else f"{(byts - prev[1]) / ((m - prev[0]) * 1e-6) / 1e9:.0f}"
        lines.append(f"| {L} | {byts / 1e6:.1f} | {m:.1f} | {c:.1f} | {byts / (m * 1e-6) / 1e9:.0f} | {marg} |")
        prev = (m, byts)
    return f"""# Decode attention over growing key spans (rocprofv3 --kernel-trace)

Command (from /tmp with TMPDIR=/tmp; REPO = repository root), then the summary script:

```
rocprofv3 --kernel-trace --output-format csv -d $REPO/{_od(out)}/prof_span -o s -- python3 -m tensor_transformer_layer_05_amd.profile_drivers decode_attn_span
python3 -m tensor_transformer_layer_05_amd.profile_summary {_od(out)}
```

The TP=4 decode attention shard shape (32 sequences, 8 q / 2 KV heads of 128, bf16 cache), {n} calls per key
span on rotating cache copies; median kernel durations from the trace.

| keys | K+V MB | `attn_decode_kernel` us | combine us | GB/s (main kernel) | GB/s of the added bytes vs the previous span |
|---:|---:|---:|---:|---:|---:|
""" + "\n".join(lines) + """

The added bytes stream at 5-6 TB/s, but each launch carries a fixed cost of about 6 us (launch ramp,
first-tile latency, the partial write) and the combine kernel another 3-5 us: at 2048 keys these fixed costs
are about half of the attention time.
"""


def hbm_reference(out):
    from .profile_drivers import HBM_REF_BYTES, HBM_REF_CALLS
    trace = _csv(os.path.join(out, "prof_hbm", "**", "*kernel_trace.csv"))
    ks = sorted(trace, key=lambda r: int(r["Start_Timestamp"]))
    dur = lambda r: (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    med = lambda v: sorted(v)[len(v) // 2]
    copy = [dur(r) for r in ks if "copyBuffer" in r["Kernel_Name"]]    # the runtime's blit kernel
    red = [dur(r) for r in ks if "reduce_kernel" in r["Kernel_Name"]]
    gemv = [dur(r) for r in ks if "gemv_dot_kernel" in r["Kernel_Name"]]
    gemv_name = _short(next(r["Kernel_Name"] for r in ks if "gemv_dot_kernel" in r["Kernel_Name"]))
    wbytes = 7168 * 8192 * 2
    rows = [("device-to-device copy, 1 GiB read + 1 GiB written", copy, 2 * HBM_REF_BYTES),
            ("torch sum of a 1 GiB float32 tensor (read only)", red, HBM_REF_BYTES),
            (f"decode gate|up + SwiGLU, one token (`{gemv_name[:60]}`), weight read", gemv, wbytes)]
    lines = [f"| {what} | {len(v)} | {med(v):.1f} | {b / (med(v) * 1e-6) / 1e12:.2f} | "
             f"{b / (med(v) * 1e-6) / 8e12:.2f} |" for what, v, b in rows]
    return f"""# Plain streaming rates on this GPU next to the decode weight stream (rocprofv3 --kernel-trace)

Command (from /tmp with TMPDIR=/tmp; REPO = repository root), then the summary script:

```
rocprofv3 --kernel-trace --output-format csv -d $REPO/{_od(out)}/prof_hbm -o h -- python3 -m tensor_transformer_layer_05_amd.profile_drivers hbm_reference
python3 -m tensor_transformer_layer_05_amd.profile_summary {_od(out)}
```

{HBM_REF_CALLS} calls each; median kernel durations from the trace; the fraction is of the 8 TB/s HBM peak.

| kernel | calls | median us | TB/s | of 8 TB/s |
|---|---:|---:|---:|---:|
""" + "\n".join(lines) + "\n"


DECODE_SRCS = ["tensor_transformer_layer_05_amd/csrc/gemm_stream.hip",
               "tensor_transformer_layer_05_amd/csrc/gemm_stream_dma.hip",
               "tensor_transformer_layer_05_amd/csrc/gemv_dot.hip",
               "tensor_transformer_layer_05_amd/csrc/attention_decode.hip",
               "tensor_transformer_layer_05_amd/csrc/argmax.hip",
               "tensor_transformer_layer_05_amd/csrc/tplayer_api.hip",
               "tensor_transformer_layer_05_amd/csrc/common.h"]


def _short(name):
    name = name.replace("(anonymous namespace)::", "")
    return name.split("(")[0].replace("void ", "").replace("tpl::", "")[:90]


def decode_traffic(out):
    from .decode_workloads import DECODE_NAMES
    fetch, write = _counters(os.path.join(out, "pmc_dfetch")), _counters(os.path.join(out, "pmc_dwrite"))
    fk, wk = sorted(fetch), sorted(write)
    if [n for _, n in fk] != [n for _, n in wk]:
        raise ValueError("the FETCH_SIZE and WRITE_SIZE runs dispatched different kernels")
    cf = [fetch[k] for k in fk if "copyBuffer" in k[1]][0]
    cw = [write[k] for k in wk if "copyBuffer" in k[1]][0]
    fs, ws = 262144.0 / cf, 262144.0 / cw
    # markers come in pairs around each measured step; what lies between an
    # end marker and the next start marker is the next shard's setup
    segs, cur, nmark = [], None, 0
    for kf, kw in zip(fk, wk):
        if "stream_read_kernel" in kf[1]:
            nmark += 1
            cur = [] if nmark % 2 == 1 else None
            if cur is not None:
                segs.append(cur)
        elif cur is not None:
            cur.append((_short(kf[1]), fetch[kf], write[kw]))
    if len(segs) != len(DECODE_NAMES) or nmark != 2 * len(DECODE_NAMES):
        raise ValueError(f"{len(segs)} marked segments for {len(DECODE_NAMES)} decode shards")
    shards, rows = {}, []
    for name, seg in zip(DECODE_NAMES, segs):
        f = sum(v for _, v, _ in seg)
        w = sum(v for _, _, v in seg)
        byts = int((f * fs + w * ws) * 1024)
        shards[name] = {"fetch_kib": round(f, 1), "write_kib": round(w, 1), "bytes": byts,
                        "kernels": [k for k, _, _ in seg]}
        for i, (k, a, b) in enumerate(seg):
            rows.append(f"| {name if i == 0 else ''} | `{k}` | {a:.1f} | {b:.1f} |")
        rows.append(f"| **{name} total** | | **{f:.1f}** | **{w:.1f}** |  -> {byts / 1e6:.2f} MB |")
    h = hashlib.sha256()
    for fn in DECODE_SRCS:
        h.update(open(os.path.join(ROOT, fn), "rb").read())
    data = {"sources": DECODE_SRCS, "sources_sha256_16": h.hexdigest()[:16],
            "copy_fetch_kib": round(cf, 1), "copy_write_kib": round(cw, 1),
            "fetch_scale": round(fs, 4), "write_scale": round(ws, 4), "shards": shards}
    stream = ""
    tr = glob.glob(os.path.join(out, "prof_stream", "**", "*kernel_trace.csv"), recursive=True)
    if tr:
        t = [r for r in csv.DictReader(open(tr[0])) if "stream_read_kernel" in r["Kernel_Name"]]
        d = sorted((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in t)
        med = d[len(d) // 2]
        stream = f"""
## The read ceiling: the reference stream under the kernel trace

```
rocprofv3 --kernel-trace --output-format csv -d {_od(out)}/prof_stream -o s -- python3 -m tensor_transformer_layer_05_amd.profile_drivers stream_ref 512 8 8 1
```

{len(d)} reads of 1 GiB by `stream_read_kernel` with non-temporal loads (512 workgroups x 8 waves, 16-byte loads
per lane, 8 KB per wave per chunk with the next chunk in flight): median {med:.1f} us = {2 ** 30 / med / 1e3:.0f} GB/s
({2 ** 30 / med / 1e3 / 8000:.3f} of 8 TB/s); min {d[0]:.1f} us, max {d[-1]:.1f} us.
"""
        data["stream_ref_median_us"] = round(med, 2)
        data["stream_ref_gbps"] = round(2 ** 30 / med / 1e3, 1)
    return f"""# HBM bytes of each decode shard's step (rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE)

Commands (from the repository root):

```
rocprofv3 --pmc FETCH_SIZE --output-format csv -d {_od(out)}/pmc_dfetch -o f -- python3 -m tensor_transformer_layer_05_amd.profile_drivers decode_traffic
rocprofv3 --pmc WRITE_SIZE --output-format csv -d {_od(out)}/pmc_dwrite -o w -- python3 -m tensor_transformer_layer_05_amd.profile_drivers decode_traffic
python3 -m tensor_transformer_layer_05_amd.profile_summary {_od(out)}
```

The driver runs one plain 256 MiB copy (calibration: {cf:.1f} KiB fetched, {cw:.1f} KiB written for 262144 KiB
each way, so FETCH_SIZE is scaled by {fs:.4f} and WRITE_SIZE by {ws:.4f}), then for each decode shard of the
benchmark its setup, a 1 GiB read-only stream (evicts the caches, marks the step's start), one step of the
shard, and a 4 KiB read by the same kernel (marks its end); the table lists the dispatches between the markers.
FETCH_SIZE counts reads that leave an XCD's L2 (the Infinity Cache may still serve them): data read by
workgroups on several XCDs (the activations, the token rows) is counted once per XCD.

| shard | kernel | FETCH_SIZE KiB | WRITE_SIZE KiB |
|---|---|---:|---:|
{chr(10).join(rows)}

bench.py divides each shard's bytes by its measured step time (`counter_hbm_frac`) only while the decode
kernels' sources still have the hash below.
{stream}
DATA {json.dumps(data)}
"""


def main(argv=None):
    """``profile_summary <out_dir> [summary ...]``: write the named summaries
    (gate_up_gemm_traffic, bench_kernel_stats, decode_traffic,
    gate_up_gemm_counters, gate_up_vendor_counters, prefill_attention_counters, ffn_gemm_counters,
    decode_attention_span, hbm_reference; default: all
    whose raw outputs are present)."""
    argv = argv or sys.argv[1:]
    if not argv:
        raise SystemExit("usage: python3 -m tensor_transformer_layer_05_amd.profile_summary <out_dir> [summary ...]")
    out = argv[0]
    only = set(argv[1:])
    raw = lambda d, pat: glob.glob(os.path.join(out, d, "**", pat), recursive=True)
    has = lambda name, d, pat: (not only or name in only) and raw(d, pat)
    if has("gate_up_gemm_traffic", "pmc_fetch", "*counter_collection.csv") and \
            raw("pmc_write", "*counter_collection.csv"):
        open(os.path.join(ROOT, "profiles", "gate_up_gemm_traffic.md"), "w").write(traffic(out))
        print("wrote profiles/gate_up_gemm_traffic.md")
    if has("bench_kernel_stats", "prof_bench", "*kernel_stats.csv"):
        open(os.path.join(ROOT, "profiles", "bench_kernel_stats.md"), "w").write(kernel_stats(out))
        print("wrote profiles/bench_kernel_stats.md")
    if has("decode_traffic", "pmc_dfetch", "*counter_collection.csv") and \
            raw("pmc_dwrite", "*counter_collection.csv"):
        open(os.path.join(ROOT, "profiles", "decode_traffic.md"), "w").write(decode_traffic(out))
        print("wrote profiles/decode_traffic.md")
    if has("gate_up_gemm_counters", "pmc_mfma", "*counter_collection.csv"):
        open(os.path.join(ROOT, "profiles", "gate_up_gemm_counters.md"), "w").write(counters(out))
        print("wrote profiles/gate_up_gemm_counters.md")
    if has("gate_up_vendor_counters", "pmc_vendor1", "*counter_collection.csv") and \
            raw("pmc_vendor3", "*counter_collection.csv"):
        open(os.path.join(ROOT, "profiles", "gate_up_vendor_counters.md"), "w").write(vendor_counters(out))
        print("wrote profiles/gate_up_vendor_counters.md")
    if has("prefill_attention_counters", "pmc_attn", "*counter_collection.csv"):
        open(os.path.join(ROOT, "profiles", "prefill_attention_counters.md"), "w").write(attention_counters(out))
        print("wrote profiles/prefill_attention_counters.md")
    if has("ffn_gemm_counters", "pmc_ffn_sq", "*counter_collection.csv") and \
            raw("pmc_ffn_fetch", "*counter_collection.csv") and raw("pmc_ffn_write", "*counter_collection.csv"):
        open(os.path.join(ROOT, "profiles", "ffn_gemm_counters.md"), "w").write(ffn_counters(out))
        print("wrote profiles/ffn_gemm_counters.md")
    if has("decode_attention_span", "prof_span", "*kernel_trace.csv"):
        open(os.path.join(ROOT, "profiles", "decode_attention_span.md"), "w").write(decode_span(out))
        print("wrote profiles/decode_attention_span.md")
    if has("hbm_reference", "prof_hbm", "*kernel_trace.csv"):
        open(os.path.join(ROOT, "profiles", "hbm_reference.md"), "w").write(hbm_reference(out))
        print("wrote profiles/hbm_reference.md")


if __name__ == "__main__":
    main()
