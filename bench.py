#!/usr/bin/env python3
"""Attention fwd+bwd throughput of the 8-layer SSSL stack on one MI355X.

One step = the whole hot path over one batch: the forward of all 8 layers
(sa_attn_fwd, each layer on its own seeded inputs) followed by the backward of
all 8 layers in reverse order (sa_attn_bwd_ex, which reads the normed k rows
back from the workspace its layer's forward kept, as a trainer keeps a
layer's saved tensors). Inputs, outputs and workspaces are resident in HBM
before the timed region starts.

Work is counted on the band only: a (query, key) pair is counted when key j is
visible to query i (0 <= i - j <= W, or j <= i for a full causal layer), at
4*D FLOP per pair for the forward (Q K^T and P V) and 10*D for the backward
(S recompute, dV, dP, dK, dQ). Masked halves of edge tiles and skipped tiles
count nothing.

Output: one JSON line (see the contract in the repository's documentation),
with a "roofline" object for the dominant kernel timed with HIP events
around each of its launches inside the timed region, and a "cpu_baseline"
object: the fp64 oracle timed on the host cores on a bounded sample of the
same workload.

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--workload 4] [--rope] [--ve]
       python bench.py --summarize-pmc FETCH_DIR WRITE_DIR   (CPU only: turns two
       rocprofv3 --pmc runs of this script into profiles/traffic_<workload>.json)
"""

from __future__ import annotations

import argparse
import csv
import ctypes
import glob
import hashlib
import json
import os
import sys
import time

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA (published)
PEAK_HBM_GBS = 8000.0
ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "qk_normed_sliding_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")
COPY_PROBE_BYTES = 1 << 30  # bytes read (and written) by the copy probe: 4x the 256 MB last-level cache

# The kernel behind each timed slot with QK-norm (the workloads here, any
# query-to-KV head ratio), and the source files its code comes from.
KERNELS = {
    "fwd": ("attn_fwd_pp_kernel", ("attn_fwd_pp.hip", "sa_common.h")),
    "bwd_dq": ("attn_bwd_dq_pp_kernel", ("attn_bwd_dq_pp.hip", "sa_common.h")),
    "bwd_dkdv": ("attn_bwd_dkdv_pp_kernel", ("attn_bwd_dkdv_pp.hip", "sa_common.h")),
    "knorm": ("qknorm_kernel", ("qknorm.hip", "sa_common.h", "ve_common.h")),
}
# the MFMA-bound attention kernels and the HBM-bound pass that norms the key rows (the
# forward's; the backward reads its output back from the forward's workspace)
MFMA_KINDS = ("fwd", "bwd_dq", "bwd_dkdv")
HBM_KINDS = ("knorm",)


def source_hash(files) -> str:
    """sha256 over a kernel's source files: identifies the code that counters were taken on."""
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def band_pairs(T: int, W: int) -> int:
    """Visible (query, key) pairs of one head: rows i >= W see W+1 keys, rows i < W see i+1."""
    if W < 0 or W >= T - 1:
        return T * (T + 1) // 2
    return (W + 1) * (T - W) + W * (W + 1) // 2


def variant_tag(args) -> str:
    """Suffix of the profile files of a run with rotary tables and/or value embeddings."""
    return ("_rope" if args.rope else "") + ("_ve" if args.ve else "")


def traffic_file(workload: str) -> str:
    return os.path.join(PROFILES, f"traffic_{workload}.json")


def traffic_bytes(workload: str, kernel: str, files):
    """HBM bytes per launch (FETCH + WRITE, scaled by the copy probe) of `kernel`
    from the committed counter summary, or None if there is none or the
    kernel's source has changed since the counters were taken."""
    try:
        with open(traffic_file(workload)) as fh:
            rec = json.load(fh)["kernels"][kernel]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source") != source_hash(files):
        return None
    return rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]


def _pmc_rows(d):
    """Per-dispatch counter values of one rocprofv3 --pmc output directory."""
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    if not rows:
        raise SystemExit(f"no *counter_collection.csv under {d}")
    return rows


def _per_dispatch(rows, counter):
    """{kernel name: [value of `counter` per dispatch]} (values summed over a dispatch's rows)."""
    acc = {}
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        key = (r["Kernel_Name"], r["Dispatch_Id"])
        acc[key] = acc.get(key, 0.0) + float(r["Counter_Value"])
    out = {}
    for (name, _), v in acc.items():
        out.setdefault(name, []).append(v)
    return out


def summarize_pmc(fetch_dir, write_dir, workload, extra=""):
    """Scale FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the attention kernels by
    what the same counters read for the copy probe (COPY_PROBE_BYTES in, same out),
    and write profiles/traffic_<workload>.json."""
    fetch = _per_dispatch(_pmc_rows(fetch_dir), "FETCH_SIZE")
    write = _per_dispatch(_pmc_rows(write_dir), "WRITE_SIZE")

    def find(table, needle):
        hits = [k for k in table if needle in k]
        if len(hits) != 1:
            raise SystemExit(f"expected one kernel matching {needle!r}, found {hits}")
        return table[hits[0]]

    probe_f = find(fetch, "neg_kernel")
    probe_w = find(write, "neg_kernel")
    f_scale = COPY_PROBE_BYTES / (sum(probe_f) / len(probe_f) * 1024.0)
    w_scale = COPY_PROBE_BYTES / (sum(probe_w) / len(probe_w) * 1024.0)
    kernels = {}
    for slot, (name, files) in KERNELS.items():
        vf, vw = find(fetch, f"{name}<"), find(write, f"{name}<")
        kernels[name] = {
            "source": source_hash(files),
            "launches_averaged": len(vf),
            "fetch_kib_per_launch_raw": sum(vf) / len(vf),
            "write_kib_per_launch_raw": sum(vw) / len(vw),
            "fetch_bytes_per_launch": sum(vf) / len(vf) * 1024.0 * f_scale,
            "write_bytes_per_launch": sum(vw) / len(vw) * 1024.0 * w_scale,
        }
    rec = {
        "workload": workload,
        "copy_probe": {"bytes_each_way": COPY_PROBE_BYTES,
                       "fetch_kib_raw": sum(probe_f) / len(probe_f), "write_kib_raw": sum(probe_w) / len(probe_w),
                       "fetch_scale": f_scale, "write_scale": w_scale},
        "kernels": kernels,
        "commands": [
            f"rocprofv3 --pmc FETCH_SIZE -f csv -d {fetch_dir} -o pmc -- python -u bench.py --steps 2 "
            f"--warmup 1 --cpu-seconds 0 --no-kernel-events --no-graph --copy-probe{extra}",
            f"rocprofv3 --pmc WRITE_SIZE -f csv -d {write_dir} -o pmc -- python -u bench.py --steps 2 "
            f"--warmup 1 --cpu-seconds 0 --no-kernel-events --no-graph --copy-probe{extra}",
            f"python bench.py --summarize-pmc {fetch_dir} {write_dir}{extra}",
        ],
    }
    os.makedirs(PROFILES, exist_ok=True)
    with open(traffic_file(workload), "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    print(json.dumps(rec, indent=1))


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=4, choices=[2, 3, 4, 5, 6])
    ap.add_argument("--rope", action="store_true",
                    help="fuse the rotary embedding of q and k (tables for ten sequence lengths)")
    ap.add_argument("--ve", action="store_true",
                    help="mix value embeddings into the layers that carry them in the trainer (1, 3, 5, 7)")
    ap.add_argument("--polar", action="store_true",
                    help="time Muon's polar-express orthogonalisation of the trainer's weight groups instead "
                         "of the attention step (its own JSON line)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="wall-clock budget of the oracle sample (0 disables the CPU baseline)")
    ap.add_argument("--no-graph", action="store_true",
                    help="launch the headline pass's steps one call at a time instead of replaying a captured "
                         "HIP graph of the step")
    ap.add_argument("--recompute-k", action="store_true",
                    help="run each backward without the forward's workspace (it norms the k rows again) instead "
                         "of reading back the normed rows the layer's forward kept")
    ap.add_argument("--no-kernel-events", action="store_true",
                    help="do not bracket the main kernels with HIP events")
    ap.add_argument("--copy-probe", action="store_true",
                    help="after the timed steps, run a plain 1 GiB device copy (bf16 negation) three times: "
                         "the reference that scales FETCH_SIZE / WRITE_SIZE counters to bytes")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarize two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of "
                         "`bench.py --copy-probe` into profiles/ and exit (no GPU needed)")
    ap.add_argument("--summarize-sq", nargs=2, metavar=("PASS0_DIR", "PASS1_DIR"),
                    help="summarize the two rocprofv3 --pmc SQ counter passes of this script into profiles/ "
                         "and exit (no GPU needed)")
    ap.add_argument("--summarize-polar-trace", nargs=3, metavar=("TRACE_DIR", "BENCH_JSON", "COMMAND"),
                    help="summarize a rocprofv3 --kernel-trace run of `bench.py --polar` into profiles/ and exit")
    ap.add_argument("--summarize-trace", nargs=4, metavar=("TRACE_DIR", "TRACE_JSON", "PLAIN_JSON", "COMMAND"),
                    help="summarize a rocprofv3 --kernel-trace run of this script (its JSON line in TRACE_JSON) "
                         "over the dispatches that the run's HIP events timed, beside the events of that run "
                         "and of a run without the profiler (its JSON line in PLAIN_JSON); COMMAND is the "
                         "command line that made them. Writes profiles/ and exits (no GPU needed)")
    return ap.parse_args()


class Hip:
    """Minimal HIP event API from the runtime torch already loaded."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so.7")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        h = ctypes.c_void_p()
        if self.lib.hipEventCreate(ctypes.byref(h)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return h.value

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        if self.lib.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def destroy(self, h):
        self.lib.hipEventDestroy(ctypes.c_void_p(h))


def hbm_bytes_per_launch(kind, w, gated=False):
    """Algorithmic HBM bytes of one launch of an HBM-bound pass: every element it must read,
    read once, and every element it must write, written once. The k-norm pass reads the bf16
    k rows and writes the bf16 normed rows and an fp32 1/rms per row. On a layer with the
    value-embedding gate the same launch also reads v, the gathered embedding rows, the ids
    and the first 32 channels of x, and writes v' and the fp32 gate."""
    rows = w.B * w.T * w.Hkv
    if kind == "knorm":
        nbytes = rows * w.D * 2 * 2 + rows * 4
        if gated:
            nbytes += rows * w.D * 2 * 3 + rows * 4 + w.B * w.T * (4 + 64)
        return nbytes
    raise ValueError(kind)


def _json_line(path):
    with open(path) as fh:
        return json.loads([ln for ln in fh if ln.lstrip().startswith("{")][-1])


def summarize_trace(trace_dir, trace_json, plain_json, command):
    """Per-kernel durations of a rocprofv3 --kernel-trace run of this script, averaged over the
    dispatches of its per-kernel pass (the last steps x layers launches of each kernel: the ones
    its HIP events bracketed), beside the event figures of the same run and of a run without the
    profiler; writes profiles/attn_kernels_<workload>_trace.md."""
    import synth

    rec = _json_line(trace_json)
    plain = _json_line(plain_json)
    cfg = rec["config"]
    w = [x for x in synth.WORKLOADS.values() if x.name == cfg["workload"]][0]
    n_last = rec["steps"] * w.n_layer
    rows = []
    for f in glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True):
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    if not rows:
        raise SystemExit(f"no *kernel_trace.csv under {trace_dir}")
    by = {}
    for r in rows:
        by.setdefault(r["Kernel_Name"], []).append(r)
    tag = ("_rope" if cfg.get("rope") else "") + ("_ve" if cfg.get("value_embeddings") else "")
    out = [f"# Kernel trace: {cfg['workload']}{' with rotary tables' if cfg.get('rope') else ''}"
           f"{' and value embeddings' if cfg.get('value_embeddings') else ''}", "",
           f"B={w.B}, T={w.T}, Hq={w.Hq}, Hkv={w.Hkv}, D={w.D}, windows {list(w.windows)}.", "",
           "Command (run from the repository root on one MI355X):", "", "```", command, "```", "",
           f"Averages over the last {n_last} dispatches of each kernel ({rec['steps']} steps x {w.n_layer} layers: "
           "the per-kernel pass, whose launches the script's HIP events bracket). Beside them: those events "
           "(same process, under the profiler, which adds a few microseconds to every event pair), and the "
           f"events of a run without the profiler ({plain['steps']} steps), which the JSON line's roofline "
           "comes from. The headline pass before the per-kernel pass replays a HIP graph of the step.", "",
           "| kernel | dispatches in run | avg us (trace) | min us | max us | avg us (events, profiled run) | "
           "avg us (events, plain run) | trace / plain events |",
           "|---|---|---|---|---|---|---|---|"]
    ev = rec.get("kernels") or {}
    ev_plain = plain.get("kernels") or {}
    shapes = []
    summary = {}
    for slot, (name, _) in KERNELS.items():
        hits = [k for k in by if k.startswith(name + "<") or k == name]
        if not hits:
            continue
        disp = sorted((r for k in hits for r in by[k]), key=lambda r: int(r["Start_Timestamp"]))
        last = disp[-n_last:]
        d = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3 for r in last]
        avg = sum(d) / len(d)
        e_ms, p_ms = ev.get(f"{slot}_ms_per_step"), ev_plain.get(f"{slot}_ms_per_step")
        e_us = e_ms * 1e3 / w.n_layer if e_ms is not None else None
        p_us = p_ms * 1e3 / w.n_layer if p_ms is not None else None
        summary[slot] = avg
        out.append(f"| {name} | {len(disp)} | {avg:.1f} | {min(d):.1f} | {max(d):.1f} | "
                   f"{'%.1f' % e_us if e_us else '-'} | {'%.1f' % p_us if p_us else '-'} | "
                   f"{'%.3f' % (avg / p_us) if p_us else '-'} |")
        r0 = last[-1]
        shapes.append(f"- {name}: grid {r0['Grid_Size_X']}x{r0['Grid_Size_Y']}, wg {r0['Workgroup_Size_X']}, "
                      f"LDS {r0['LDS_Block_Size']}, VGPR {r0['VGPR_Count']}, AGPR {r0['Accum_VGPR_Count']}, "
                      f"scratch {r0['Scratch_Size']}")
    known = [k for k in by if any(k.startswith(n + "<") or k == n for n, _ in KERNELS.values())]
    others = sorted((k for k in by if k not in known and not k.startswith("__amd")),
                    key=lambda k: -sum(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in by[k]))
    if others:
        out += ["", "Other kernels in the run (all dispatches, warm-up included):", "",
                "| kernel | dispatches | avg us | min us | max us |", "|---|---|---|---|---|"]
        for k in others:
            d = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3 for r in by[k]]
            out.append(f"| {k} | {len(d)} | {sum(d) / len(d):.1f} | {min(d):.1f} | {max(d):.1f} |")
    out += ["", "Launch shape (grid threads, workgroup threads, LDS bytes, VGPR/AGPR as reported, scratch):", ""]
    out += shapes
    rf = plain.get("roofline")
    if rf:
        slot = [s for s, (n, _) in KERNELS.items() if n == rf["kernel"]][0]
        tr = rf["algorithmic_flop_per_launch"] / (summary[slot] * 1e-6) / 1e12
        out += ["", f"Roofline of the dominant kernel ({rf['kernel']}): {rf['algorithmic_flop_per_launch']:.4g} "
                    f"algorithmic FLOP per launch ({rf['flop_per_visible_pair']} per visible pair). From the trace "
                    f"average: {tr:.0f} TFLOP/s = {tr / PEAK_BF16_TFLOPS:.4f} of {PEAK_BF16_TFLOPS:g}; from the "
                    f"plain run's events (its JSON line's roofline): {rf['achieved']:.0f} TFLOP/s = "
                    f"{rf['frac']:.4f}.", ""]
    for slot in HBM_KINDS:
        if slot in summary:
            gb = ev_plain.get(f"{slot}_algorithmic_bytes")
            if gb:
                out.append(f"- {KERNELS[slot][0]}: {gb / 1e6:.1f} MB algorithmic per launch; "
                           f"{gb / (summary[slot] * 1e-6) / 1e9:.0f} GB/s from the trace average, "
                           f"{ev_plain.get(f'{slot}_gbs', 0):.0f} GB/s from the plain run's events "
                           f"(peak {PEAK_HBM_GBS:g}).")
    out += ["", f"Headlines: {rec['ms_per_step']:.3f} ms per step under the profiler, {plain['ms_per_step']:.3f} "
                f"ms per step ({plain['value']:.1f} TFLOP/s, {plain['pct_bf16_peak']:.2f}% of bf16 peak) in the "
                f"plain run; {plain['config'].get('launch')}."]
    path = os.path.join(PROFILES, f"attn_kernels_{cfg['workload']}{tag}_trace.md")
    os.makedirs(PROFILES, exist_ok=True)
    with open(path, "w") as fh:
        fh.write("\n".join(out) + "\n")
    print("\n".join(out))
    print(f"wrote {path}", file=sys.stderr)


SQ_PASSES = (
    "SQ_BUSY_CYCLES SQ_VALU_MFMA_BUSY_CYCLES SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS SQ_WAIT_INST_LDS "
    "SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_INSTS_LDS GRBM_GUI_ACTIVE",
    "SQ_WAVE_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_ACTIVE_INST_ANY SQ_INSTS_MFMA SQ_INSTS_VALU "
    "SQ_VALU_MFMA_COEXEC_CYCLES SQ_INSTS_SALU GRBM_GUI_ACTIVE",
)


def summarize_sq(dir_a, dir_b, workload, extra=""):
    """Utilisation ratios of each kernel from two rocprofv3 --pmc passes (SQ_PASSES) of this
    script; writes profiles/sq_counters_<workload>.md. GRBM_GUI_ACTIVE is summed over the 8 XCDs
    in the counter output (and present in both passes), so one XCD's busy cycles per dispatch is
    its per-kernel sum / dispatches / 2 / 8; a SIMD-cycle budget is that times 1024 SIMDs."""
    agg, disp = {}, {}
    for d in (dir_a, dir_b):
        for r in _pmc_rows(d):
            k = r["Kernel_Name"].split("(")[0].replace("void ", "").replace("sa::", "")
            c = agg.setdefault(k, {})
            c[r["Counter_Name"]] = c.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
            disp.setdefault(k, set()).add((d, r["Dispatch_Id"]))
    lines = []
    for slot, (name, _) in KERNELS.items():
        for k, c in agg.items():
            if not k.startswith(name + "<"):
                continue
            nd = len(disp[k]) / 2

            def f(x):
                return c.get(x, 0.0) / nd

            g = c["GRBM_GUI_ACTIVE"] / nd / 2 / 8
            simd, cu = g * 1024, g * 256
            wave = max(1.0, f("SQ_WAVE_CYCLES"))
            lines.append(
                f"{k[:40]:40s} GRBM/xcd {g:8.0f}  MFMA-busy {f('SQ_VALU_MFMA_BUSY_CYCLES') / simd:6.1%}  "
                f"VALU-active {4 * f('SQ_ACTIVE_INST_VALU') / simd:6.1%}  coexec "
                f"{f('SQ_VALU_MFMA_COEXEC_CYCLES') / simd:6.1%}  LDS-active {f('SQ_LDS_IDX_ACTIVE') / cu:6.1%}  "
                f"bank-confl {f('SQ_LDS_BANK_CONFLICT') / max(1.0, f('SQ_LDS_IDX_ACTIVE')):6.1%}  "
                f"wait-LDS {f('SQ_WAIT_INST_LDS') / wave:6.1%}  wait-any {f('SQ_WAIT_ANY') / wave:6.1%}  "
                f"wait-inst {f('SQ_WAIT_INST_ANY') / wave:6.1%}  MFMA/VALU insts "
                f"{f('SQ_INSTS_MFMA') / max(1.0, f('SQ_INSTS_VALU')):.3f}")
    base = f"python -u bench.py --steps 2 --warmup 1 --cpu-seconds 0 --no-kernel-events --no-graph{extra}"
    cmds = [f"timeout -s KILL 120 rocprofv3 --pmc {SQ_PASSES[i]} -f csv -d {d} -o pmc -- {base}"
            for i, d in enumerate((dir_a, dir_b))]
    cmds.append(f"python bench.py --summarize-sq {dir_a} {dir_b}{extra}")
    out = [f"# SQ counters: {workload}", "",
           "Commands (two counter passes, each its own run, then the summary; from the repository root):", "",
           "```", *cmds, "```", "",
           "Per dispatch, averaged over each kernel's dispatches. GRBM/xcd = GRBM_GUI_ACTIVE per XCD (the counter "
           "sums the 8 XCDs); SIMD cycles = GRBM/xcd x 1024 SIMDs, CU cycles = GRBM/xcd x 256.",
           "MFMA-busy = SQ_VALU_MFMA_BUSY_CYCLES / SIMD cycles; VALU-active = 4 x SQ_ACTIVE_INST_VALU (quad-cycles) "
           "/ SIMD cycles; coexec = SQ_VALU_MFMA_COEXEC_CYCLES / SIMD cycles; LDS-active = SQ_LDS_IDX_ACTIVE / CU "
           "cycles; bank-confl = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE; wait-LDS, wait-any, wait-inst = "
           "SQ_WAIT_INST_LDS, SQ_WAIT_ANY, SQ_WAIT_INST_ANY over SQ_WAVE_CYCLES.", "",
           "```", *lines, "```"]
    path = os.path.join(PROFILES, f"sq_counters_{workload}.md")
    os.makedirs(PROFILES, exist_ok=True)
    with open(path, "w") as fh:
        fh.write("\n".join(out) + "\n")
    print("\n".join(out))


def summarize_polar_trace(trace_dir, bench_json, command):
    """Per-kernel statistics over every dispatch of a rocprofv3 --kernel-trace run of
    `bench.py --polar`, beside that run's JSON line; writes
    profiles/polar_express_muon_groups_n768_trace.md."""
    rec = _json_line(bench_json)
    rows = []
    for f in glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True):
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    if not rows:
        raise SystemExit(f"no *kernel_trace.csv under {trace_dir}")
    by = {}
    for r in rows:
        name = r["Kernel_Name"].split("<")[0]
        if name.startswith(("gemm", "sumsq", "transpose")):
            by.setdefault(name, []).append(r)
    tot = sum((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3 for v in by.values() for r in v)
    out = [f"# Kernel trace: {rec['config']['workload']} (Muon polar express, 5 steps)", "",
           "Command (run from the repository root on one MI355X):", "", "```", command, "```", "",
           "| kernel | dispatches | total us | avg us | min us | max us | % |", "|---|---|---|---|---|---|---|"]
    shapes = []
    for name, v in sorted(by.items(), key=lambda kv: -len(kv[1])):
        d = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3 for r in v]
        out.append(f"| {name} | {len(d)} | {sum(d):.1f} | {sum(d) / len(d):.1f} | {min(d):.1f} | {max(d):.1f} | "
                   f"{100 * sum(d) / tot:.2f} |")
        seen = set()
        for r in v:
            key = (r["Grid_Size_X"], r["Grid_Size_Y"])
            if key not in seen:
                seen.add(key)
                shapes.append(f"- {name}: grid {r['Grid_Size_X']}x{r['Grid_Size_Y']}, wg {r['Workgroup_Size_X']}, "
                              f"LDS {r['LDS_Block_Size']}, VGPR {r['VGPR_Count']}, AGPR {r['Accum_VGPR_Count']}")
    out += ["", "Launch shapes:", ""] + shapes
    out += ["", f"The same run's JSON line: {rec['value']:.1f} TFLOP/s, {rec['ms_per_step']:.3f} ms per optimizer step "
                f"({rec['steps']} timed steps after {rec['warmup']} warm-up; the trace counts the warm-up too)."]
    path = os.path.join(PROFILES, "polar_express_muon_groups_n768_trace.md")
    with open(path, "w") as fh:
        fh.write("\n".join(out) + "\n")
    print("\n".join(out))


def cpu_model() -> str:
    """The host CPU as lscpu names it: model name, family and model numbers, from /proc/cpuinfo
    (a virtual machine may report a short model name; the numbers still identify the part)."""
    info = {}
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if ":" in line:
                    key, val = (x.strip() for x in line.split(":", 1))
                    info.setdefault(key, val)
                if not line.strip() and info:
                    break
    except OSError:
        return "unknown"
    name = info.get("model name", "unknown")
    return f"{name} (family {info.get('cpu family', '?')}, model {info.get('model', '?')}, " \
           f"stepping {info.get('stepping', '?')})"


def cpu_baseline(w, budget_s):
    """Time the fp64 oracle (as it stands) on whole (batch, KV-group) slices of
    one sliding-window layer and one full-causal layer of the workload,
    alternating, until the budget is used; report band FLOP/s."""
    import torch

    import oracle
    import synth

    torch.set_num_threads(max(1, os.cpu_count() or 1))
    G = w.Hq // w.Hkv
    local = next(i for i, W in enumerate(w.windows) if W >= 0)
    full = next(i for i, W in enumerate(w.windows) if W < 0) if -1 in w.windows else local
    picked = sorted({local, full})
    inputs = {layer: synth.layer_inputs(w, layer) for layer in picked}
    flops = spent = 0.0
    n = {layer: 0 for layer in picked}
    i = 0
    while spent < budget_s and i < len(picked) * w.B * w.Hkv:
        layer = picked[i % len(picked)]
        b = (i // len(picked)) % w.B
        g = (i // (len(picked) * w.B)) % w.Hkv
        q, k, v, do = inputs[layer]
        hs = slice(g * G, (g + 1) * G)
        qs, ks, vs, ds = q[b:b + 1, :, hs], k[b:b + 1, :, g:g + 1], v[b:b + 1, :, g:g + 1], do[b:b + 1, :, hs]
        W = w.windows[layer]
        t0 = time.perf_counter()
        oracle.attn_forward(qs, ks, vs, W, w.scale, eps=w.eps)
        oracle.attn_backward(qs, ks, vs, ds, W, w.scale, eps=w.eps)
        spent += time.perf_counter() - t0
        flops += 14.0 * w.D * G * band_pairs(w.T, W)
        n[layer] += 1
        i += 1
    parts = ", ".join(f"{n[layer]} of layer {layer} (window {w.windows[layer]})" for layer in picked)
    return {
        "value": flops / spent / 1e12,
        "unit": "TFLOP/s",
        "cores": torch.get_num_threads(),
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": (f"fp64 oracle forward+backward on whole (batch, KV-group) slices ({G} query heads, "
                   f"T={w.T}) of the same workload: {parts}; {spent:.1f} s of oracle time; "
                   f"band FLOPs counted as on the GPU"),
    }


# The trainer's Muon groups at n_embd 768, 8 layers, multi-head attention (the
# pages' default n_kv_head = n_head): per layer the q, k, v and output
# projections (768 x 768) and the MLP's two matrices ([out, in] = 3072 x 768
# and 768 x 3072), stacked by shape.
POLAR_GROUPS = ((32, 768, 768), (8, 3072, 768), (8, 768, 3072))


def polar_flops(batch, rows, cols, steps=5):
    """MFMA FLOP of the iteration: per step A = X X^T (2 m^2 n), A A (2 m^3), B X (2 m^2 n), m <= n."""
    m, n = min(rows, cols), max(rows, cols)
    return float(batch) * steps * (4.0 * m * m * n + 2.0 * m ** 3)


def bench_polar(args):
    import torch

    import qk_normed_sliding_amd as sa

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    gen = torch.Generator().manual_seed(4242)
    groups = []
    for batch, rows, cols in POLAR_GROUPS:
        g = torch.randn((batch, rows, cols), generator=gen, dtype=torch.float32).to(torch.bfloat16).to(dev)
        ws = torch.empty(sa.sa_polar_express_workspace_bytes(batch, rows, cols), dtype=torch.uint8, device=dev)
        groups.append((g, torch.empty_like(g), ws))
    flop = sum(polar_flops(*x) for x in POLAR_GROUPS)
    # MFMA FLOP the library actually executes: its symmetric products (X X^T, A A) compute the
    # tiles on and above the diagonal only
    flop_exec = sum(sa.sa_polar_express_executed_flops(b, r, c, 5) for b, r, c in POLAR_GROUPS)

    def step():
        for g, out, ws in groups:
            sa.sa_polar_express(g, out=out, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(args.steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    tflops = flop / (ms * 1e-3) / 1e12

    cpu = None
    if args.cpu_seconds > 0:
        import oracle

        torch.set_num_threads(max(1, os.cpu_count() or 1))
        done = spent = 0.0
        samples = 0
        while spent < args.cpu_seconds:
            batch, rows, cols = POLAR_GROUPS[samples % len(POLAR_GROUPS)]
            g = groups[samples % len(POLAR_GROUPS)][0][0:1].cpu()
            t = time.perf_counter()
            oracle.polar_express(g)
            spent += time.perf_counter() - t
            done += polar_flops(1, rows, cols)
            samples += 1
        cpu = {"value": done / spent / 1e12, "unit": "TFLOP/s", "cores": torch.get_num_threads(),
               "cpu_model": cpu_model(), "kind": "oracle",
               "sample": f"{samples} single matrices cycling through the three groups (fp64 iteration), "
                         f"{spent:.1f} s"}

    out = {
        "metric": "Muon polar-express TFLOP/s (5 steps, the trainer's weight groups at n_embd 768)",
        "value": tflops, "unit": "TFLOP/s", "pct_bf16_peak": 100.0 * tflops / PEAK_BF16_TFLOPS,
        "executed_tflops": flop_exec / (ms * 1e-3) / 1e12,
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 gradients of the weight shapes)",
        "config": {"workload": "muon_polar_express_n768_8layers_mha", "groups": [list(x) for x in POLAR_GROUPS],
                   "flop_count": "per matrix 5 x (4 m^2 n + 2 m^3), m <= n (full products; value and "
                                 "pct_bf16_peak are effective throughput on this count, executed_tflops counts "
                                 "the MFMA work run: the symmetric products compute their upper tiles only)",
                   "flop_per_step": flop, "executed_flop_per_step": flop_exec,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "kernel": "gemm_kernel (with the norm and transpose passes)",
                     "achieved": tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / PEAK_BF16_TFLOPS, "traffic": None},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.polar and args.gpus == 1:
        bench_polar(args)
        return
    if args.summarize_pmc:
        import synth

        extra = (f" --workload {args.workload}" if args.workload != 4 else "") + \
            (" --rope" if args.rope else "") + (" --ve" if args.ve else "")
        summarize_pmc(*args.summarize_pmc, synth.WORKLOADS[args.workload].name + variant_tag(args), extra)
        return
    if args.summarize_sq:
        import synth

        extra = (f" --workload {args.workload}" if args.workload != 4 else "") + \
            (" --rope" if args.rope else "") + (" --ve" if args.ve else "")
        summarize_sq(*args.summarize_sq, synth.WORKLOADS[args.workload].name + variant_tag(args), extra)
        return
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace)
        return
    if args.summarize_polar_trace:
        summarize_polar_trace(*args.summarize_polar_trace)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build runs on a single MI355X and has no multi-GPU path "
              f"(--gpus {args.gpus} requested). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import qk_normed_sliding_amd as sa
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = synth.WORKLOADS[args.workload]

    layers = []
    for layer in range(w.n_layer):
        q, k, v, do = (x.to(dev) for x in synth.layer_inputs(w, layer))
        ve = None
        if args.ve and layer in sa.ve_layers(w.n_layer):
            ve = tuple(t.to(dev) for t in synth.ve_inputs(w, layer))
        print(f"inputs of layer {layer} resident", file=sys.stderr, flush=True)
        # each layer keeps its forward's workspace (normed k rows and their 1/rms; v' and the
        # gate on gated layers) for its backward, as a trainer keeps a layer's saved tensors
        layers.append(dict(
            W=w.windows[layer], q=q, k=k, v=v, do=do,
            o=torch.empty_like(q), lse=torch.empty((w.B, w.Hq, w.T), dtype=torch.float32, device=dev),
            dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v), ve=ve,
            wsf=torch.empty(sa.sa_attn_fwd_workspace_bytes(w.B, w.T, w.Hq, w.Hkv, w.D), dtype=torch.uint8,
                            device=dev)))
    ws = torch.empty(sa.sa_attn_bwd_workspace_bytes(w.B, w.T, w.Hq, w.Hkv, w.D), dtype=torch.uint8, device=dev)
    rope = sa.rope_tables(10 * w.T, w.D, device=dev) if args.rope else None
    ws_ve = (torch.empty(sa.sa_attn_ve_workspace_bytes(w.B, w.T, w.Hkv, w.D), dtype=torch.uint8, device=dev)
             if args.ve else None)
    torch.cuda.synchronize()

    def fwd(L):
        if L["ve"] is not None:
            sa.sa_attn_fwd_ex(L["q"], L["k"], L["v"], window=L["W"], softmax_scale=w.scale, eps=w.eps, o=L["o"],
                              lse=L["lse"], workspace=L["wsf"], rope=rope, ve=L["ve"])
            return
        sa.sa_attn_fwd(L["q"], L["k"], L["v"], window=L["W"], softmax_scale=w.scale, eps=w.eps, o=L["o"], lse=L["lse"],
                       workspace=L["wsf"], rope=rope)

    def bwd(L):
        sa.sa_attn_bwd_ex(L["q"], L["k"], L["v"], L["o"], L["lse"], L["do"], window=L["W"], softmax_scale=w.scale,
                          eps=w.eps, dq=L["dq"], dk=L["dk"], dv=L["dv"], workspace=ws, rope=rope, ve=L["ve"],
                          ve_workspace=ws_ve if L["ve"] is not None else None,
                          fwd_workspace=None if args.recompute_k else L["wsf"])

    hip = Hip()
    use_ev = not args.no_kernel_events
    # one event pair per launch of each main kernel in the timed region
    n_ev = args.steps * w.n_layer
    # (with --recompute-k the backward's own k-norm pass too: the same kernel)
    hbm_kinds = HBM_KINDS + (("bwd_knorm",) if args.recompute_k else ())
    kinds = MFMA_KINDS + hbm_kinds
    hook = {"fwd": sa.SA_KERNEL_FWD, "bwd_dq": sa.SA_KERNEL_BWD_DQ, "bwd_dkdv": sa.SA_KERNEL_BWD_DKDV,
            "knorm": sa.SA_KERNEL_FWD_KNORM, "bwd_knorm": sa.SA_KERNEL_BWD_KNORM}
    ev = {k: [(hip.event(), hip.event()) for _ in range(n_ev)] if use_ev else [] for k in kinds}

    def step(s=None):
        for li, L in enumerate(layers):
            if s is not None and use_ev:
                sa.sa_set_timing_events(hook["fwd"], *ev["fwd"][s * w.n_layer + li])
                sa.sa_set_timing_events(hook["knorm"], *ev["knorm"][s * w.n_layer + li])
            fwd(L)
        for li in reversed(range(w.n_layer)):
            if s is not None and use_ev:
                sa.sa_set_timing_events(hook["bwd_dq"], *ev["bwd_dq"][s * w.n_layer + li])
                sa.sa_set_timing_events(hook["bwd_dkdv"], *ev["bwd_dkdv"][s * w.n_layer + li])
                if args.recompute_k:
                    sa.sa_set_timing_events(hook["bwd_knorm"], *ev["bwd_knorm"][s * w.n_layer + li])
            bwd(layers[li])
        if use_ev:
            for k in kinds:
                sa.sa_set_timing_events(hook[k], None, None)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # Pass 1, the headline: exactly `steps` steps with no per-launch events in the timed region.
    # By default the step's launches (8 forwards, 8 backwards: 40 kernels) are captured once
    # in a HIP graph and the graph is replayed per step, as a trainer replays its step graph;
    # the library records nothing but kernel launches, so the graph holds kernel nodes only.
    graph = None
    if not args.no_graph:
        graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            with torch.cuda.graph(graph, stream=cap):
                step()
        torch.cuda.current_stream().wait_stream(cap)
        for _ in range(2):
            graph.replay()
        torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record()
    for _ in range(args.steps):
        if graph is not None:
            graph.replay()
        else:
            step()
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = t0.elapsed_time(t1)
    ms_step = ms_total / args.steps
    # Pass 2, the per-kernel split: the same steps again, with HIP events around each main kernel's launches.
    ms_step_events = None
    if use_ev:
        t0.record()
        for s in range(args.steps):
            step(s)
        t1.record()
        torch.cuda.synchronize()
        ms_step_events = t0.elapsed_time(t1) / args.steps

    pairs = [w.B * w.Hq * band_pairs(w.T, L["W"]) for L in layers]
    flop_fwd = sum(4.0 * w.D * p for p in pairs)
    flop_bwd = sum(10.0 * w.D * p for p in pairs)
    flop_step = flop_fwd + flop_bwd
    tflops = flop_step / (ms_step * 1e-3) / 1e12

    kern = {}
    roofline = None
    if use_ev:
        # MFMA FLOP each kernel executes per visible pair: the forward 4 D (Q K^T, P V);
        # the dQ kernel 6 D (S recompute, dP, dQ); the dK/dV kernel 8 D (S recompute,
        # dP, dV, dK). The headline value counts 4 D + 10 D per pair, so the
        # backward's duplicated S and dP earn nothing there.
        per_pair = {"fwd": 4.0, "bwd_dq": 6.0, "bwd_dkdv": 8.0}
        ms = {k: sum(hip.elapsed_ms(a, b) for a, b in ev[k]) / args.steps for k in kinds}
        for k in MFMA_KINDS:
            kern[f"{k}_ms_per_step"] = ms[k]
            kern[f"{k}_tflops"] = per_pair[k] * w.D * sum(pairs) / (ms[k] * 1e-3) / 1e12
        for k in hbm_kinds:
            # (the backward's own pass, run only without the forward's workspace, mixes v' too)
            step_bytes = sum(hbm_bytes_per_launch("knorm", w, gated=L["ve"] is not None) for L in layers)
            kern[f"{k}_ms_per_step"] = ms[k]
            kern[f"{k}_algorithmic_bytes"] = step_bytes / w.n_layer
            kern[f"{k}_gbs"] = step_bytes / (ms[k] * 1e-3) / 1e9
            kern[f"{k}_traffic"] = traffic_bytes(w.name + variant_tag(args), *KERNELS["knorm"])
        kern["ms_per_step_with_events"] = ms_step_events
        kern["other_ms_per_step"] = ms_step_events - sum(ms.values())
        # the headline pass (no events; graph replay unless --no-graph) less the same kernels' own
        # durations: the launch gaps of the step as timed
        kern["other_ms_per_step_headline"] = ms_step - sum(ms.values())
        dom = max(MFMA_KINDS, key=lambda k: ms[k])
        flop_launch = per_pair[dom] * w.D * sum(pairs) / w.n_layer
        avg_ms = ms[dom] / w.n_layer
        achieved = flop_launch / (avg_ms * 1e-3) / 1e12
        name, files = KERNELS[dom]
        roofline = {"bound": "mfma", "kernel": name, "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                    "traffic": traffic_bytes(w.name + variant_tag(args), name, files),
                    "avg_launch_ms": avg_ms, "algorithmic_flop_per_launch": flop_launch,
                    "flop_per_visible_pair": f"{per_pair[dom]:g} D"}
        for k in kinds:
            for a, b in ev[k]:
                hip.destroy(a)
                hip.destroy(b)

    if args.copy_probe:
        # plain device copy of known size: one read and one write of COPY_PROBE_BYTES per launch
        src = torch.ones(COPY_PROBE_BYTES // 2, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(w, args.cpu_seconds)

    out = {
        "metric": "attention fwd+bwd TFLOP/s (band-counted), SSSL 8-layer T=2048; % bf16 MFMA peak",
        "value": tflops,
        "unit": "TFLOP/s",
        "pct_bf16_peak": 100.0 * tflops / PEAK_BF16_TFLOPS,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 q/k/v/dO of the model shape; no dataset or trained weights)",
        "config": {
            "workload": w.name,
            "B": w.B, "T": w.T, "Hq": w.Hq, "Hkv": w.Hkv, "head_dim": w.D,
            "windows": list(w.windows), "qk_norm": True, "eps": w.eps, "softmax_scale": w.scale,
            "rope": bool(args.rope), "value_embeddings": bool(args.ve),
            "flop_count": "band pairs x (4D fwd + 10D bwd)",
            "flop_per_step": flop_step,
            "launch": "HIP graph of the step, replayed" if graph is not None else "one call per layer",
            "backward_k_rows": "recomputed" if args.recompute_k else "read back from the layer's forward workspace",
            "parallelism": "single GPU",
        },
        "wall_s_timed": wall,
        "kernels": kern,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
