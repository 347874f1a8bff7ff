"""Summaries of rocprofv3 runs of bench.py, written into profiles/.

Three modes, each reading the CSV output (``-o run --output-format csv``) of
the rocprofv3 commands it names in the summary it writes:

    python3 rocprof_summary.py trace   DIR LOG  # --kernel-trace --stats run of the default bench
    python3 rocprof_summary.py traffic BASE     # FETCH_SIZE / WRITE_SIZE passes (BASE/tr_*)
    python3 rocprof_summary.py util    BASE     # MFMA-busy passes (BASE/util_W)
    python3 rocprof_summary.py valu    BASE     # vector-unit passes (BASE/valu_W)

The raw runs (one MI355X, repository root, ``export TMPDIR=/tmp``; OUT is any
output directory):

    rocprofv3 --kernel-trace --stats -d OUT/kt -o run --output-format csv -- \\
        python3 bench.py --steps 50 --warmup 5 --no-cpu-baseline > OUT/kt.log
    rocprofv3 --pmc FETCH_SIZE -d OUT/tr_copy_FETCH_SIZE -o run --output-format csv -- \\
        python3 bench.py --copy-calibration 512          (and WRITE_SIZE)
    rocprofv3 --pmc FETCH_SIZE -d OUT/tr_FETCH_SIZE_W -o run --output-format csv -- \\
        python3 bench.py --workload W --steps 3 --warmup 1 --no-extra --no-cpu-baseline \\
        --no-backward --no-varlen --no-splitkv --no-fp8    (W = 1..5, and WRITE_SIZE)
    rocprofv3 --kernel-trace --pmc MfmaUtil SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES GRBM_GUI_ACTIVE \\
        -d OUT/util_W -o run --output-format csv -- python3 bench.py --workload W \\
        --steps 20 --warmup 2 --no-extra --no-cpu-baseline --no-backward --no-varlen \\
        --no-splitkv --no-fp8                              (W = 1..5)
    rocprofv3 --kernel-trace --pmc SQ_ACTIVE_INST_VALU SQ_INSTS_VALU SQ_INSTS_VALU_TRANS_F32 \\
        SQ_INSTS_MFMA SQ_INSTS_LDS SQ_ACTIVE_INST_LDS SQ_BUSY_CYCLES SQ_VALU_MFMA_BUSY_CYCLES \\
        -d OUT/valu_W -o run --output-format csv -- python3 bench.py --workload W --steps 20 \\
        --warmup 2 --no-extra --no-cpu-baseline --no-backward --no-varlen --no-splitkv --no-fp8  (W = 2..5)

This is measurement tooling: it reads CSV files and imports bench.py for the
workload definitions, algorithmic byte counts and the kernel source hash.
"""

import collections
import csv
import json
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import WORKLOADS  # noqa: E402

PROFILES = os.path.join(ROOT, "profiles")
BENCH_FLAGS = "--no-extra --no-cpu-baseline --no-backward --no-varlen --no-splitkv --no-fp8"
SIMDS = 1024   # 256 CUs x 4 SIMDs
SES = 32       # 8 XCDs x 4 shader engines (SQ_BUSY_CYCLES is summed over them)
XCDS = 8       # GRBM_GUI_ACTIVE is summed over the XCDs


def csv_in(base, name):
    """Path of rocprofv3's CSV `name` under the output directory `base` (directly in it, or in the
    host/process subdirectories rocprofv3 may add)."""
    direct = os.path.join(base, name)
    if os.path.exists(direct):
        return direct
    for root, _, files in os.walk(base):
        if name in files:
            return os.path.join(root, name)
    raise FileNotFoundError(f"{name} under {base}")


def short_name(kernel_name):
    n = kernel_name.replace("void attn::(anonymous namespace)::", "").replace("(attn::Params)", "")
    n = n.replace("(attn::(anonymous namespace)::BwdParams)", "").replace("(attn::BwdParams)", "")
    return n.split("(")[0]


def dispatches(path, kernel_filter="attn_fwd_bf16_kernel"):
    """{dispatch id: {counter: value}} plus durations (ns) from a counter CSV."""
    per = collections.defaultdict(dict)
    dur = {}
    for r in csv.DictReader(open(path)):
        if kernel_filter not in r["Kernel_Name"]:
            continue
        d = int(r["Dispatch_Id"])
        per[d][r["Counter_Name"]] = per[d].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        dur[d] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    return per, dur


def forward_kernel(w):
    """Name filter of the forward kernel that workload w launches."""
    return "attn_fwd_f32" if WORKLOADS[w].dtype == "f32" else "attn_fwd_bf16_kernel"


# --------------------------------------------------------------------------- trace

TRACE_LABELS = {
    ("attn_fwd_f32_split_kernel<64, false, 8>", 8): "forward, workload 1 (fp32): single-head B1 H1 N256 d64",
    ("attn_fwd_bf16_kernel<64, 4, false, 2, false, false>", 256): "forward, workload 2: mha B4 H8 N1024 d64",
    ("attn_fwd_bf16_kernel<64, 4, true, 2, true, false>", 256): "forward, workload 3: causal B2 H8 N4096 d64",
    ("attn_fwd_bf16_kernel<128, 8, true, 1, false, false>", 1024): "forward, workload 4: causal long B1 H16 N16384 d128",
    ("attn_fwd_bf16_kernel<128, 8, false, 1, false, false>", 2048):
        "forward, workload 5 (headline): gqa padded B2 Hq32 Hkv8 N8192 d128",
    ("attn_fwd_bf16_kernel<128, 4, true, 1, false, true>", 16384):
        "packed varlen: 8 sequences U{4096..8192}, Hq32 Hkv8 d128 causal",
    ("attn_fwd_bf16_kernel<128, 4, true, 1, false, true>", 2048):
        "split-KV, 16 ranges: Nq512 over Nk32768 Hq32 Hkv8 d128 causal",
    ("attn_fwd_bf16_kernel<128, 4, true, 2, true, true>", 128): "split-KV shape as one range (persistent)",
    ("attn_merge_kernel<true, unsigned short>", 2048): "merge of the 16 split-KV partials (bf16)",
    ("attn_fwd_fp8_kernel<128, true>", 2048): "fp8 forward, workload 4 shape",
    ("attn_fwd_fp8_kernel<128, false>", 4096): "fp8 forward, workload 5 shape",
}


def trace(base, log):
    cmd = (f"rocprofv3 --kernel-trace --stats -d {base} -o run --output-format csv -- "
           "python3 bench.py --steps 50 --warmup 5 --no-cpu-baseline")
    groups = collections.OrderedDict()
    for r in csv.DictReader(open(csv_in(base, "run_kernel_trace.csv"))):
        wg = int(r["Workgroup_Size_X"])
        key = (short_name(r["Kernel_Name"]), int(r["Grid_Size_X"]) // wg, wg)
        groups.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0)
    rows = []
    for (name, grid, wg), d in groups.items():
        label = TRACE_LABELS.get((name, grid), "")
        if not label and name.startswith("attn_bwd"):
            label = "backward"
        if not label:
            continue
        rest = d[1:] if len(d) > 1 else d
        rows.append((label, name, grid, wg, len(d), statistics.mean(d), statistics.mean(rest), statistics.median(d),
                     min(d), max(d)))
    result = None
    for line in open(log):
        if line.startswith('{"metric"'):
            result = json.loads(line)
    hdr = ("| kernel | what | workgroups x threads | calls | average us | average after first | median us | min us "
           "| max us |\n|---|---|---|---|---|---|---|---|---|\n")

    def table(sel):
        return hdr + "\n".join(f"| `{n}` | {lab} | {g} x {w} | {c} | {a:.2f} | {a2:.2f} | {m:.2f} | {mn:.2f} | {mx:.2f} |"
                               for (lab, n, g, w, c, a, a2, m, mn, mx) in sel) + "\n"

    fwd = sorted([r for r in rows if r[0].startswith("forward")], key=lambda r: r[0])
    md = f"""# rocprofv3 kernel-trace summary: the forward kernels, workloads 1 to 5 (5 is the headline)

Command (one MI355X, repository root), summarised by `python3 rocprof_summary.py trace`:

    {cmd}

Template arguments are attn_fwd_bf16_kernel <D, WAVES, CAUSAL, KSPLIT, PERSISTENT, GENERAL>
(WAVES: 32-row query slices per key-split group) and attn_fwd_f32_split_kernel <D, CAUSAL,
WAVES> (32 query rows, key tiles split over WAVES waves).
Durations in microseconds from run_kernel_trace.csv (the warm-up launches are included in the
plain average, not in the second).

{table(fwd)}
"""
    head = [r for r in fwd if "headline" in r[0]]
    if result and head:
        h = head[0]
        ev = result["ms_per_step"] * 1000
        md += (f"Headline workload: bench.py in the same profiled run timed {ev:.2f} us per launch with HIP events on "
               f"the launch stream over {result['steps']} back-to-back launches; rocprofv3 gives {h[6]:.2f} us per "
               f"launch averaged over the calls after the first (median {h[7]:.2f} us), "
               f"{abs(ev - h[6]) / h[6] * 100:.1f}% apart (the events also count the gaps between launches).\n")
    with open(os.path.join(PROFILES, "attn_fwd_workloads1-5_kernel_trace.md"), "w") as f:
        f.write(md)
    other = [r for r in rows if not r[0].startswith("forward")]
    md2 = f"""# rocprofv3 kernel-trace summary: packed varlen, split-KV + merge, fp8 forward, backward

Same run as attn_fwd_workloads1-5_kernel_trace.md:

    {cmd}

Template arguments: attn_fwd_bf16_kernel <D, WAVES, CAUSAL, KSPLIT, PERSISTENT, GENERAL>,
attn_fwd_fp8_kernel <D, CAUSAL>, attn_merge_kernel <bf16 output, partial type>, backward <D, CAUSAL>.
Durations in microseconds from run_kernel_trace.csv.

{table(other)}
"""
    with open(os.path.join(PROFILES, "next_rows_kernel_trace.md"), "w") as f:
        f.write(md2)
    print(md + "\n" + md2)


# --------------------------------------------------------------------------- traffic

def traffic(base):
    copy_mib = 512

    def med(path, filt):
        per, _ = dispatches(path, filt)
        vals = [sum(v.values()) for _, v in sorted(per.items())]
        return statistics.median(vals)

    f_copy = med(csv_in(os.path.join(base, "tr_copy_FETCH_SIZE"), "run_counter_collection.csv"), "copyBuffer")
    w_copy = med(csv_in(os.path.join(base, "tr_copy_WRITE_SIZE"), "run_counter_collection.csv"), "copyBuffer")
    f_factor = copy_mib * 1024 / f_copy
    w_factor = copy_mib * 1024 / w_copy
    out = {"kernel_source_hash": bench.kernel_source_hash(),
           "calibration": {"copy_bytes": copy_mib << 20, "fetch_kib_read": f_copy, "write_kib_read": w_copy,
                           "fetch_factor": round(f_factor, 4), "write_factor": round(w_factor, 4)},
           "workloads": {}}
    lines = []
    for w in (1, 2, 3, 4, 5):
        fk = med(csv_in(os.path.join(base, f"tr_FETCH_SIZE_{w}"), "run_counter_collection.csv"), forward_kernel(w))
        wk = med(csv_in(os.path.join(base, f"tr_WRITE_SIZE_{w}"), "run_counter_collection.csv"), forward_kernel(w))
        b = fk * 1024 * f_factor + wk * 1024 * w_factor
        alg = bench.algorithmic_bytes(WORKLOADS[w])
        out["workloads"][str(w)] = {"fetch_kib": fk, "write_kib": wk, "bytes_per_launch": int(b),
                                    "algorithmic_bytes": alg, "ratio": round(b / alg, 3)}
        lines.append(f"| {w} | {WORKLOADS[w].name} | {fk:.0f} | {wk:.0f} | {b / 2**20:.1f} | {alg / 2**20:.1f} "
                     f"| {b / alg:.2f} |")
    with open(os.path.join(PROFILES, "hbm_traffic.json"), "w") as f:
        json.dump(out, f, indent=1)
    md = f"""# HBM traffic of the forward kernel per launch, workloads 1 to 5 (rocprofv3 counters)

Commands (one MI355X, repository root; one counter per pass), summarised by
`python3 rocprof_summary.py traffic {base}`:

    rocprofv3 --pmc FETCH_SIZE -d {base}/tr_copy_FETCH_SIZE -o run --output-format csv -- python3 bench.py --copy-calibration 512
    rocprofv3 --pmc WRITE_SIZE -d {base}/tr_copy_WRITE_SIZE -o run --output-format csv -- python3 bench.py --copy-calibration 512
    rocprofv3 --pmc FETCH_SIZE -d {base}/tr_FETCH_SIZE_W -o run --output-format csv -- python3 bench.py --workload W --steps 3 --warmup 1 {BENCH_FLAGS}
    rocprofv3 --pmc WRITE_SIZE -d {base}/tr_WRITE_SIZE_W -o run --output-format csv -- python3 bench.py --workload W --steps 3 --warmup 1 {BENCH_FLAGS}

Calibration: a device-to-device copy of 512 MiB (`__amd_rocclr_copyBuffer`) reads
FETCH_SIZE = {f_copy:.0f} KiB and WRITE_SIZE = {w_copy:.0f} KiB, so FETCH_SIZE is scaled by
{f_factor:.3f} and WRITE_SIZE by {w_factor:.3f}.  Values are medians over the profiled launches;
the counters are summed over all agents' blocks per dispatch.

Kernel source hash (bench.kernel_source_hash): `{out['kernel_source_hash']}`.

| workload | name | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled MiB | algorithmic MiB | ratio |
|---|---|---|---|---|---|---|
""" + "\n".join(lines) + "\n"
    with open(os.path.join(PROFILES, "attn_fwd_workloads1-5_hbm_traffic.md"), "w") as f:
        f.write(md)
    print(md)


# --------------------------------------------------------------------------- MFMA utilisation

def util(base):
    out = {"kernel_source_hash": bench.kernel_source_hash(), "workloads": {}}
    lines = []
    for w in (1, 2, 3, 4, 5):
        per, dur = dispatches(csv_in(os.path.join(base, f"util_{w}"), "run_counter_collection.csv"), forward_kernel(w))
        recs = []
        for d, c in sorted(per.items()):
            ns = dur[d]
            busy = c["SQ_VALU_MFMA_BUSY_CYCLES"] / SIMDS             # MFMA-busy cycles per SIMD
            clk = c["SQ_BUSY_CYCLES"] / SES / ns                     # GHz: cycles with waves present / time
            recs.append({"us": ns / 1000.0, "clock_ghz": clk, "mfma_busy": busy / (c["SQ_BUSY_CYCLES"] / SES),
                         "rocprof_MfmaUtil": c.get("MfmaUtil", float("nan")) / 100.0})
        recs = recs[1:] if len(recs) > 2 else recs                   # drop the first (cold) launch
        med = {k: statistics.median(r[k] for r in recs) for k in recs[0]}
        out["workloads"][str(w)] = {k: round(v, 4) for k, v in med.items()}
        out["workloads"][str(w)]["launches"] = len(recs)
        lines.append(f"| {w} | {WORKLOADS[w].name} | {len(recs)} | {med['us']:.1f} | {med['clock_ghz']:.2f} | "
                     f"{100 * med['mfma_busy']:.1f}% | {100 * med['rocprof_MfmaUtil']:.1f}% |")
    with open(os.path.join(PROFILES, "mfma_util.json"), "w") as f:
        json.dump(out, f, indent=1)
    md = f"""# MFMA utilisation and shader clock of the forward kernel, workloads 1 to 5 (rocprofv3 counters)

Command per workload W (one MI355X, repository root), summarised by
`python3 rocprof_summary.py util {base}`:

    rocprofv3 --kernel-trace --pmc MfmaUtil SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES GRBM_GUI_ACTIVE -d {base}/util_W -o run --output-format csv -- python3 bench.py --workload W --steps 20 --warmup 2 {BENCH_FLAGS}

Per launch: `SQ_VALU_MFMA_BUSY_CYCLES` (summed over the 1024 SIMDs; 32 per 32x32x16 bf16 MFMA,
64 per 32x32x2 fp32 MFMA of workload 1)
/ 1024 is the matrix-core busy time of one SIMD; `SQ_BUSY_CYCLES` (summed over the 32 shader
engines) / 32 is the number of shader-clock cycles with waves present, and divided by the
launch's duration it gives the effective shader clock.  "MFMA busy" is the ratio of the two;
"rocprof MfmaUtil" is rocprofv3's derived metric (busy cycles over GUI-active cycles, which for
short launches also count time outside the kernel).  Medians over the launches after the first.

The bf16 peak of 2.5 PFLOP/s assumes a 2.4 GHz clock: achieved TFLOP/s ≈ 2500 × (clock / 2.4)
× MFMA busy × (algorithmic / executed MFMA flops) (workload 1: 157.3 in place of 2500).

Workload 1 launches eight workgroups: the shader engines without waves count no busy cycles, so
its "clock" (cycles with waves present, averaged over all 32 engines) and "MFMA busy" are not
utilisation figures of the chip; it is launch-latency bound.

Kernel source hash (bench.kernel_source_hash): `{out['kernel_source_hash']}`.

| workload | name | launches | us | shader clock GHz | MFMA busy | rocprof MfmaUtil |
|---|---|---|---|---|---|---|
""" + "\n".join(lines) + "\n"
    with open(os.path.join(PROFILES, "attn_fwd_workloads1-5_mfma_util.md"), "w") as f:
        f.write(md)
    print(md)


# --------------------------------------------------------------------------- vector unit

VALU_COUNTERS = ("SQ_ACTIVE_INST_VALU SQ_INSTS_VALU SQ_INSTS_VALU_TRANS_F32 SQ_INSTS_MFMA SQ_INSTS_LDS "
                 "SQ_ACTIVE_INST_LDS SQ_BUSY_CYCLES SQ_VALU_MFMA_BUSY_CYCLES")


def valu(base):
    lines = []
    out = {"kernel_source_hash": bench.kernel_source_hash(), "workloads": {}}
    for w in (2, 3, 4, 5):
        per, dur = dispatches(csv_in(os.path.join(base, f"valu_{w}"), "run_counter_collection.csv"), forward_kernel(w))
        recs = []
        for d, c in sorted(per.items()):
            cycles = c["SQ_BUSY_CYCLES"] / SES                      # shader cycles with waves present
            mfma_n = c["SQ_INSTS_MFMA"]
            recs.append({
                "valu_per_mfma": c["SQ_INSTS_VALU"] / mfma_n if mfma_n else float("nan"),
                "trans_per_mfma": c["SQ_INSTS_VALU_TRANS_F32"] / mfma_n if mfma_n else float("nan"),
                "lds_per_mfma": c["SQ_INSTS_LDS"] / mfma_n if mfma_n else float("nan"),
                # SQ_ACTIVE_INST_* count quad-cycles per wave, summed over the waves of each SIMD
                "valu_busy": 4 * c["SQ_ACTIVE_INST_VALU"] / SIMDS / cycles,
                "lds_busy": 4 * c["SQ_ACTIVE_INST_LDS"] / SIMDS / cycles,
                "mfma_busy": c["SQ_VALU_MFMA_BUSY_CYCLES"] / SIMDS / cycles,
            })
        recs = recs[1:] if len(recs) > 2 else recs
        med = {k: statistics.median(r[k] for r in recs) for k in recs[0]}
        out["workloads"][str(w)] = {k: round(v, 4) for k, v in med.items()}
        lines.append(f"| {w} | {WORKLOADS[w].name} | {med['valu_per_mfma']:.2f} | {med['trans_per_mfma']:.2f} | "
                     f"{med['lds_per_mfma']:.2f} | {100 * med['valu_busy']:.1f}% | {100 * med['mfma_busy']:.1f}% | "
                     f"{100 * med['lds_busy']:.1f}% |")
    md = f"""# Vector-unit activity of attn_fwd_bf16_kernel beside its MFMA activity (rocprofv3 counters)

Command per workload W (one MI355X, repository root), summarised by
`python3 rocprof_summary.py valu {base}`:

    rocprofv3 --kernel-trace --pmc {VALU_COUNTERS} -d {base}/valu_W -o run --output-format csv -- python3 bench.py --workload W --steps 20 --warmup 2 {BENCH_FLAGS}

Per launch (medians over the launches after the first): instructions per MFMA instruction from
`SQ_INSTS_VALU` (every vector instruction, MFMAs included), `SQ_INSTS_VALU_TRANS_F32` (the
exponentials) and `SQ_INSTS_LDS`; busy fractions of one SIMD from `SQ_ACTIVE_INST_VALU` and
`SQ_ACTIVE_INST_LDS` (quad-cycles a wave spends on such instructions, summed over the SIMD's waves,
so a fraction above the unit's share means waves overlap) and `SQ_VALU_MFMA_BUSY_CYCLES`, each over
`SQ_BUSY_CYCLES` / 32 (shader cycles with waves present) and 1024 SIMDs.  `SQ_INSTS_VALU` counts the
MFMAs too, so "VALU instr per MFMA" is one more than the vector instructions issued per MFMA; a
32x32x16 bf16 MFMA holds the matrix core 32 cycles, about what six or seven plain vector
instructions take to issue.

Kernel source hash (bench.kernel_source_hash): `{out['kernel_source_hash']}`.

| workload | name | VALU instr per MFMA | exp per MFMA | LDS instr per MFMA | VALU-active | MFMA busy | LDS-active |
|---|---|---|---|---|---|---|---|
""" + "\n".join(lines) + "\n"
    with open(os.path.join(PROFILES, "attn_fwd_workloads2-5_valu.md"), "w") as f:
        f.write(md)
    print(md)


if __name__ == "__main__":
    mode = sys.argv[1] if len(sys.argv) > 1 else ""
    if mode == "trace" and len(sys.argv) == 4:
        trace(sys.argv[2], sys.argv[3])
    elif mode == "traffic" and len(sys.argv) == 3:
        traffic(sys.argv[2])
    elif mode == "util" and len(sys.argv) == 3:
        util(sys.argv[2])
    elif mode == "valu" and len(sys.argv) == 3:
        valu(sys.argv[2])
    else:
        sys.exit(__doc__)
