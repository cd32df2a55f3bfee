"""Helpers around rocprofv3 output: kernel-time tables, HBM traffic records, copy calibration.

    python -m scaled_dot_product_tiled_amd.profiling copy [--mib N] [--reps R]
        runs a plain device-to-device copy of N MiB R times, the reference for scaling the
        FETCH_SIZE / WRITE_SIZE counters (a copy of N MiB fetches and writes exactly N MiB);
    python -m scaled_dot_product_tiled_amd.profiling stats DIR
        prints the per-kernel table of a `rocprofv3 --kernel-trace --stats` output directory;
    python -m scaled_dot_product_tiled_amd.profiling traffic --kernel NAME --source FILE
            --fetch DIR --write DIR --copy-fetch DIR --copy-write DIR [--copy-mib N]
        prints a traffic record for kernel NAME from four `rocprofv3 --pmc` output
        directories: the kernel's FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each scaled
        by the copy run's bytes per counter unit, with the sha256 of the kernel's source file.

    python -m scaled_dot_product_tiled_amd.profiling summaries OUT
        writes the profiles/ summaries of every workload W with a directory OUT/W holding the
        rocprofv3 passes of `bench.py --workload W` (stats, fetch, write, sq; the copy
        calibration in OUT/cfetch, OUT/cwrite); each summary lists the commands that made it.

bench.py reads such records back (read_traffic) and reports the traffic only while the
source file still has the recorded hash.
"""
import argparse
import csv
import glob
import hashlib
import os
import sys
from typing import Dict, List, Optional

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _csvs(d: str, suffix: str) -> List[str]:
    found = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not found:
        raise FileNotFoundError(f"no *{suffix} under {d}")
    return found


def counter_per_dispatch(d: str, counter: str) -> Dict[str, List[float]]:
    """{kernel name: [value per dispatch]} of one counter in a rocprofv3 --pmc csv output."""
    out: Dict[str, List[float]] = {}
    for f in _csvs(d, "_counter_collection.csv"):
        with open(f) as fh:
            for row in csv.DictReader(fh):
                if row["Counter_Name"] == counter:
                    out.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
    return out


def _pick(values: Dict[str, List[float]], kernel: str) -> List[float]:
    """The values of the one kernel whose name contains `kernel` (spaces ignored, so that a
    template argument list can be written without them)."""
    key = kernel.replace(" ", "")
    names = [n for n in values if key in n.replace(" ", "")]
    if len(names) != 1:
        raise KeyError(f"{kernel!r} matches {names}")
    return values[names[0]]


def sha256(path: str) -> str:
    with open(path, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()


def copy_factor(d: str, counter: str, nbytes: int) -> float:
    """Bytes per counter unit: the largest dispatch of the copy run moved nbytes (the
    counters report KiB, but FETCH_SIZE reads half the fetched bytes here, so the scale is
    measured rather than assumed)."""
    vals = [max(v) for v in counter_per_dispatch(d, counter).values()]
    return nbytes / max(vals)


def traffic_record(kernel: str, source: str, fetch: str, write: str, copy_fetch: str, copy_write: str,
                   copy_mib: int) -> str:
    nbytes = copy_mib << 20
    ff = copy_factor(copy_fetch, "FETCH_SIZE", nbytes)
    fw = copy_factor(copy_write, "WRITE_SIZE", nbytes)
    fv = _pick(counter_per_dispatch(fetch, "FETCH_SIZE"), kernel)
    wv = _pick(counter_per_dispatch(write, "WRITE_SIZE"), kernel)
    fkib, wkib = sum(fv) / len(fv), sum(wv) / len(wv)
    rel = os.path.relpath(os.path.abspath(source), ROOT)
    return (f"record: kernel={kernel} fetch_count={fkib:.1f} write_count={wkib:.1f} fetch_scale={ff:.4f} "
            f"write_scale={fw:.4f} fetch_bytes={fkib * ff:.0f} write_bytes={wkib * fw:.0f} "
            f"dispatches={len(fv)},{len(wv)} source={rel} sha256={sha256(source)}")


def read_traffic(path: str, kernel: str) -> Optional[dict]:
    """The traffic record of `kernel` in a profiles/ summary, or None if it is missing or
    the kernel's source has changed since it was taken."""
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        for line in fh:
            line = line.strip()
            if not line.startswith("record:"):
                continue
            kv = dict(t.split("=", 1) for t in line[len("record:"):].split())
            if kv.get("kernel") != kernel:
                continue
            src = os.path.join(ROOT, kv["source"])
            if not os.path.exists(src) or sha256(src) != kv["sha256"]:
                return None
            fetch = float(kv["fetch_count"]) * float(kv["fetch_scale"])
            write = float(kv["write_count"]) * float(kv["write_scale"])
            return {"fetch_bytes": fetch, "write_bytes": write, "bytes": fetch + write}
    return None


def trace_durations(d: str) -> Dict[str, List[float]]:
    """{kernel name: [duration ns per dispatch, in dispatch order]} of a --kernel-trace csv output."""
    out: Dict[str, List[float]] = {}
    try:
        files = _csvs(d, "_kernel_trace.csv")
    except FileNotFoundError:
        return out
    rows = []
    for f in files:
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    for r in rows:
        out.setdefault(r["Kernel_Name"], []).append(float(r["End_Timestamp"]) - float(r["Start_Timestamp"]))
    return out


def stats_table(d: str) -> str:
    """Per-kernel table of a --kernel-trace --stats output: calls, mean, median (from the trace),
    min, max and share of the total time, for the library's kernels (the run's other kernels,
    torch's input generation and copies, are summed in one line)."""
    rows = []
    for f in _csvs(d, "_kernel_stats.csv"):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    dur = trace_durations(d)
    lines = [f"{'calls':>6} {'avg_us':>10} {'med_us':>10} {'min_us':>10} {'max_us':>10} {'pct':>6}  kernel"]
    other = [r for r in rows if "attn::" not in r["Name"]]
    rows = [r for r in rows if "attn::" in r["Name"]]
    for r in rows:
        med = float(np.median(dur[r["Name"]])) / 1e3 if r["Name"] in dur else float("nan")
        lines.append(f"{int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.2f} {med:10.2f} "
                     f"{float(r['MinNs']) / 1e3:10.2f} {float(r['MaxNs']) / 1e3:10.2f} {float(r['Percentage']):6.2f}  "
                     f"{r['Name']}")
    if other:
        lines.append(f"{sum(int(r['Calls']) for r in other):6d} launches of {len(other)} other kernels (input "
                     f"generation, copies): {sum(float(r['Percentage']) for r in other):.2f}% of the time")
    return "\n".join(lines)


WORKLOADS = {
    "tiny_d512": "tiny causal GQA, B=1 S=128 Hq=2 Hkv=1 D=512 (forward + backward)",
    "full_d512": "causal GQA, B=2 S=4096 Hq=32 Hkv=4 D=512 (forward + backward; the bench.py step)",
    "window_d256": "causal sliding window 1024, B=2 S=4096 Hq=32 Hkv=16 D=256, Q/K std 3 (forward + backward)",
    "varlen_d512": "padded varlen causal GQA, B=8 lengths U{512..8192} padded to 8192, Hq=32 Hkv=4 D=512 "
                   "(forward + backward)",
    "decode_d128": "paged decode, B=64 Hq=32 Hkv=8 D=128, 16-token pages, contexts U{512..4096} (two pools)",
    "paged_prefill_d512": "paged forward, a 2048-token chunk after 6144 cached tokens, Hq=32 Hkv=4 D=512, 16-token "
                          "pages (append + attn_fwd_paged; then append + gather + chunk-pair forward)",
    "mixed_step_d512": "paged forward, a 1024-token chunk after 3072 cached plus 31 decode rows of 512..4096 tokens, "
                       "Hq=32 Hkv=4 D=512 (append + attn_fwd_paged_split: rank, forward, merge; then "
                       "attn_fwd_paged alone)",
}

SQ_COUNTERS = ("SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_LDS_DATA_FIFO_FULL", "SQ_VALU_MFMA_BUSY_CYCLES",
               "SQ_BUSY_CU_CYCLES", "SQ_WAIT_INST_LDS", "SQ_INSTS_LDS_LOAD_BANDWIDTH", "SQ_LDS_ADDR_CONFLICT",
               "GRBM_GUI_ACTIVE")
N_XCD, N_CU, N_SIMD = 8, 256, 1024

# source file of each kernel family (for the sha256 a traffic record carries)
SOURCES = (("fwd_kernel<", "attn_fwd.hip"), ("fwd_merge_kernel<", "attn_fwd.hip"), ("fwd_paged_kernel<", "attn_fwd.hip"),
           ("fwd_split_merge", "attn_fwd.hip"), ("paged_rank", "varlen_prep.hip"), ("bwd_", "attn_bwd.hip"),
           ("decode_", "attn_decode.hip"), ("varlen_", "varlen_prep.hip"), ("ds_seq_base", "varlen_prep.hip"),
           ("lse_merge", "attn_merge.hip"), ("paged_kv", "paged_kv.hip"))


def commands(wl: str) -> str:
    steps = "--steps 10 --warmup 3" if wl != "decode_d128" else "--steps 50 --warmup 4"
    few = "--steps 2 --warmup 1" if wl != "decode_d128" else "--steps 4 --warmup 2"
    b = f"python3 $R/bench.py --workload {wl}"
    return f"""Commands (cd /tmp && export TMPDIR=/tmp first; R = repository root, OUT = an output directory):
  rocprofv3 --kernel-trace --stats -d $OUT/{wl}/stats --output-format csv -- {b} {steps}
  rocprofv3 --pmc FETCH_SIZE -d $OUT/{wl}/fetch --output-format csv -- {b} {few}
  rocprofv3 --pmc WRITE_SIZE -d $OUT/{wl}/write --output-format csv -- {b} {few}
  rocprofv3 --pmc {' '.join(SQ_COUNTERS)} -d $OUT/{wl}/sq --output-format csv -- {b} {few}
  rocprofv3 --pmc FETCH_SIZE -d $OUT/cfetch --output-format csv -- python3 $R/scaled_dot_product_tiled_amd/profiling.py copy --mib 1024
  rocprofv3 --pmc WRITE_SIZE -d $OUT/cwrite --output-format csv -- python3 $R/scaled_dot_product_tiled_amd/profiling.py copy --mib 1024
  python3 -m scaled_dot_product_tiled_amd.profiling summaries $OUT
"""


def _short(name: str) -> str:
    """'void attn::fwd_kernel<512, 32, false, false, false>(attn::AttnArgs)' -> 'fwd_kernel<512,32,false,false,false>'"""
    n = name.replace("void ", "").replace("attn::", "").replace(" ", "")
    return n.split("(")[0]


def sq_table(d: str) -> str:
    """Matrix-core and LDS use per kernel from one pass of SQ_COUNTERS.  GRBM_GUI_ACTIVE is summed
    over the 8 XCDs, so one XCD's active cycles (the kernel's duration in shader clocks) are an
    eighth of it; SQ_VALU_MFMA_BUSY_CYCLES is summed over the 1024 SIMDs, SQ_INSTS_LDS_LOAD_BANDWIDTH
    counts 64-byte units, SQ_WAIT_INST_LDS counts wave-cycles in units of 4."""
    vals = {c: counter_per_dispatch(d, c) for c in SQ_COUNTERS}
    rows = [f"{'kernel':42s} {'cycles':>9s} {'MFMA busy':>9s} {'LDS B/clk/CU':>12s} {'bank confl.':>11s} "
            f"{'LDS fifo full':>13s} {'wait LDS issue':>14s}"]
    names = sorted(vals["GRBM_GUI_ACTIVE"], key=lambda n: -sum(vals["GRBM_GUI_ACTIVE"][n]))
    for k in names:
        if not any(k.replace(" ", "").startswith(p) or ("attn::" + p) in k.replace(" ", "") for p, _ in SOURCES):
            continue
        m = {c: sum(vals[c].get(k, [0.0])) / max(len(vals[c].get(k, [1.0])), 1) for c in SQ_COUNTERS}
        cyc = m["GRBM_GUI_ACTIVE"] / N_XCD
        if cyc <= 0:
            continue
        busy = m["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * N_SIMD)
        lds = m["SQ_INSTS_LDS_LOAD_BANDWIDTH"] * 64 / (cyc * N_CU)
        conf = m["SQ_LDS_BANK_CONFLICT"] / max(m["SQ_LDS_IDX_ACTIVE"], 1.0)
        fifo = m["SQ_LDS_DATA_FIFO_FULL"] / max(m["SQ_BUSY_CU_CYCLES"], 1.0)
        wait = 4 * m["SQ_WAIT_INST_LDS"] / max(4 * cyc * N_CU, 1.0)   # per wave slot: 4 waves per CU
        rows.append(f"{_short(k):42s} {cyc:9.0f} {100 * busy:8.1f}% {lds:12.1f} {100 * conf:10.2f}% "
                    f"{100 * fifo:12.2f}% {100 * wait:13.1f}%")
    return "\n".join(rows)


def traffic_records(d: str, out: str) -> List[str]:
    """One traffic record per attention kernel of a workload's fetch / write passes."""
    fetch = counter_per_dispatch(os.path.join(d, "fetch"), "FETCH_SIZE")
    recs = []
    for name in sorted(fetch, key=lambda n: -sum(fetch[n]) / len(fetch[n])):
        short = _short(name)
        src = next((f for p, f in SOURCES if short.startswith(p)), None)
        if src is None:
            continue
        recs.append(traffic_record(short, os.path.join(ROOT, "scaled_dot_product_tiled_amd", "csrc", src),
                                   os.path.join(d, "fetch"), os.path.join(d, "write"), os.path.join(out, "cfetch"),
                                   os.path.join(out, "cwrite"), 1024))
    return recs


def _bench_line(d: str) -> Optional[dict]:
    import json
    line = None
    for f in glob.glob(os.path.join(d, "*.log")):
        for ln in open(f):
            if ln.startswith("{"):
                try:
                    line = json.loads(ln)
                except ValueError:
                    pass
    return line


def write_summaries(out: str, pdir: str) -> None:
    """profiles/<workload>_kernel_stats.txt, _traffic.txt and _sq.txt for every workload directory
    OUT/<workload> that holds the rocprofv3 passes of commands(workload)."""
    os.makedirs(pdir, exist_ok=True)
    for wl, what in WORKLOADS.items():
        d = os.path.join(out, wl)
        if not os.path.isdir(os.path.join(d, "stats")):
            continue
        cmds = commands(wl)
        txt = f"Kernel times on one MI355X, rocprofv3 kernel trace: {what}.\n\n{cmds}\n{stats_table(os.path.join(d, 'stats'))}\n"
        line = _bench_line(d)
        if line is not None and "kernels" in line:
            txt += "\nbench.py --workload's own HIP-event timings of the same run (ms per launch):\n"
            for n, v in line["kernels"].items():
                txt += f"  {n:14s} {v['ms_avg']:.4f}\n"
        with open(os.path.join(pdir, f"{wl}_kernel_stats.txt"), "w") as fh:
            fh.write(txt)
        if os.path.isdir(os.path.join(d, "fetch")) and os.path.isdir(os.path.join(d, "write")):
            recs = traffic_records(d, out)
            txt = (f"HBM traffic per dispatch on one MI355X: {what}.\n\n"
                   "rocprofv3 counters FETCH_SIZE and WRITE_SIZE (one pass each, averaged over the dispatches of each\n"
                   "kernel), scaled by what the same counters read for a plain 1 GiB device copy (bytes per counter\n"
                   "unit: fetch_scale, write_scale).  FETCH_SIZE counts every L2 miss sent to the fabric, part of\n"
                   "which the 256 MB last-level cache serves.\n\n")
            for r in recs:
                kv = dict(t.split("=", 1) for t in r[len("record:"):].split())
                txt += (f"  {kv['kernel']:42s} fetched {int(kv['fetch_bytes']) / 1e9:8.4f} GB   written "
                        f"{int(kv['write_bytes']) / 1e9:8.4f} GB\n")
            txt += (f"\n{cmds}\nbench.py reads the record lines below for its roofline \"traffic\" fields, as long as\n"
                    "each kernel's source still has the recorded sha256.\n\n" + "\n".join(recs) + "\n")
            with open(os.path.join(pdir, f"{wl}_traffic.txt"), "w") as fh:
                fh.write(txt)
        if os.path.isdir(os.path.join(d, "sq")):
            txt = (f"Matrix-core and LDS use on one MI355X: {what}; one rocprofv3 pass of SQ counters,\n"
                   "averaged over each kernel's dispatches.\n\n"
                   "  cycles          shader clocks the kernel was active on one XCD (GRBM_GUI_ACTIVE / 8)\n"
                   "  MFMA busy       SQ_VALU_MFMA_BUSY_CYCLES / (cycles x 1024 SIMDs)\n"
                   "  LDS B/clk/CU    bytes read from LDS (SQ_INSTS_LDS_LOAD_BANDWIDTH x 64) / (cycles x 256 CUs)\n"
                   "  bank confl.     SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE\n"
                   "  LDS fifo full   SQ_LDS_DATA_FIFO_FULL / SQ_BUSY_CU_CYCLES\n"
                   "  wait LDS issue  wave-cycles waiting to issue an LDS instruction / wave-cycles of 4 waves per CU\n\n"
                   f"{cmds}\n{sq_table(os.path.join(d, 'sq'))}\n")
            with open(os.path.join(pdir, f"{wl}_sq.txt"), "w") as fh:
                fh.write(txt)


def run_copy(mib: int, reps: int) -> None:
    import torch
    a = torch.ones(mib << 20, dtype=torch.uint8, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(f"copied {mib} MiB x {reps}", flush=True)


def main(argv=None) -> int:
    p = argparse.ArgumentParser(prog="python -m scaled_dot_product_tiled_amd.profiling")
    sub = p.add_subparsers(dest="cmd", required=True)
    c = sub.add_parser("copy")
    c.add_argument("--mib", type=int, default=1024)
    c.add_argument("--reps", type=int, default=3)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    t = sub.add_parser("traffic")
    for name in ("kernel", "source", "fetch", "write", "copy-fetch", "copy-write"):
        t.add_argument("--" + name, required=True)
    t.add_argument("--copy-mib", type=int, default=1024)
    w = sub.add_parser("summaries")
    w.add_argument("out")
    w.add_argument("--profiles", default=os.path.join(ROOT, "profiles"))
    a = p.parse_args(argv)
    if a.cmd == "copy":
        run_copy(a.mib, a.reps)
    elif a.cmd == "stats":
        print(stats_table(a.dir))
    elif a.cmd == "summaries":
        write_summaries(a.out, a.profiles)
    else:
        print(traffic_record(a.kernel, a.source, a.fetch, a.write, a.copy_fetch, a.copy_write, a.copy_mib))
    return 0


if __name__ == "__main__":
    sys.exit(main())
