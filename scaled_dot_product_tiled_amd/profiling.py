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
        writes the profiles/ summaries of the bench.py workloads from OUT/{stats,fetch,write,
        cfetch,cwrite} and, if present, OUT/sq (the rocprofv3 runs listed in each summary).

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


def stats_table(d: str) -> str:
    rows = []
    for f in _csvs(d, "_kernel_stats.csv"):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    lines = [f"{'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'pct':>6}  kernel"]
    for r in rows:
        lines.append(f"{int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.2f} {float(r['MinNs']) / 1e3:10.2f} "
                     f"{float(r['MaxNs']) / 1e3:10.2f} {float(r['Percentage']):6.2f}  {r['Name']}")
    return "\n".join(lines)


COMMANDS = """Commands (cd /tmp && export TMPDIR=/tmp first; R = repository root, OUT = an output directory):
  rocprofv3 --kernel-trace --stats -d $OUT/stats --output-format csv -- python3 $R/bench.py --steps 10 --warmup 3 --no-cpu-baseline --no-other
  rocprofv3 --pmc FETCH_SIZE -d $OUT/fetch --output-format csv -- python3 $R/bench.py --steps 2 --warmup 1 --decode-steps 4 --no-cpu-baseline --no-other
  rocprofv3 --pmc WRITE_SIZE -d $OUT/write --output-format csv -- python3 $R/bench.py --steps 2 --warmup 1 --decode-steps 4 --no-cpu-baseline --no-other
  rocprofv3 --pmc FETCH_SIZE -d $OUT/cfetch --output-format csv -- python3 $R/scaled_dot_product_tiled_amd/profiling.py copy --mib 1024
  rocprofv3 --pmc WRITE_SIZE -d $OUT/cwrite --output-format csv -- python3 $R/scaled_dot_product_tiled_amd/profiling.py copy --mib 1024
  rocprofv3 --pmc SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_LDS_DATA_FIFO_FULL SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES SQ_WAIT_INST_LDS SQ_INSTS_LDS_LOAD_BANDWIDTH SQ_LDS_ADDR_CONFLICT GRBM_GUI_ACTIVE -d $OUT/sq --output-format csv -- python3 $R/bench.py --steps 2 --warmup 1 --decode-steps 4 --no-cpu-baseline --no-other
  python3 -m scaled_dot_product_tiled_amd.profiling summaries $OUT
"""

SQ_COUNTERS = ("SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_LDS_DATA_FIFO_FULL", "SQ_VALU_MFMA_BUSY_CYCLES",
               "SQ_BUSY_CU_CYCLES", "SQ_WAIT_INST_LDS", "SQ_INSTS_LDS_LOAD_BANDWIDTH", "SQ_LDS_ADDR_CONFLICT",
               "GRBM_GUI_ACTIVE")
SQ_KERNELS = (("attn_fwd", "fwd_kernel<512,32,false,false,false>"), ("bwd_dkdv", "bwd_dkdv_kernel<512,false,false>"),
              ("bwd_dq", "bwd_dq_kernel<256,4,2,false>"), ("decode_split", "decode_split_kernel<4,false,false>"))
N_XCD, N_CU, N_SIMD = 8, 256, 1024


def sq_table(d: str) -> str:
    """Matrix-core and LDS use per kernel from one pass of SQ_COUNTERS.  GRBM_GUI_ACTIVE is summed
    over the 8 XCDs, so one XCD's active cycles (the kernel's duration in shader clocks) are an
    eighth of it; SQ_VALU_MFMA_BUSY_CYCLES is summed over the 1024 SIMDs, SQ_INSTS_LDS_LOAD_BANDWIDTH
    counts 64-byte units, SQ_WAIT_INST_LDS counts wave-cycles in units of 4."""
    vals = {c: counter_per_dispatch(d, c) for c in SQ_COUNTERS}
    rows = [f"{'kernel':14s} {'cycles':>9s} {'MFMA busy':>9s} {'LDS B/clk/CU':>12s} {'bank confl.':>11s} "
            f"{'LDS fifo full':>13s} {'wait LDS issue':>14s}"]
    for label, k in SQ_KERNELS:
        m = {c: sum(_pick(vals[c], k)) / len(_pick(vals[c], k)) for c in SQ_COUNTERS}
        cyc = m["GRBM_GUI_ACTIVE"] / N_XCD
        busy = m["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * N_SIMD)
        lds = m["SQ_INSTS_LDS_LOAD_BANDWIDTH"] * 64 / (cyc * N_CU)
        conf = m["SQ_LDS_BANK_CONFLICT"] / max(m["SQ_LDS_IDX_ACTIVE"], 1.0)
        fifo = m["SQ_LDS_DATA_FIFO_FULL"] / max(m["SQ_BUSY_CU_CYCLES"], 1.0)
        wait = 4 * m["SQ_WAIT_INST_LDS"] / max(4 * cyc * N_CU, 1.0)   # per wave slot: 4 waves per CU
        rows.append(f"{label:14s} {cyc:9.0f} {100 * busy:8.1f}% {lds:12.1f} {100 * conf:10.2f}% {100 * fifo:12.2f}% "
                    f"{100 * wait:13.1f}%")
    return "\n".join(rows)

# (file, kernel name, source, what, algorithmic bytes) of each traffic summary
TRAFFIC_SUMMARIES = [
    ("attn_fwd_d512_B2_S4096_traffic.txt", "fwd_kernel<512,32,false,false,false>", "scaled_dot_product_tiled_amd/csrc/attn_fwd.hip",
     "forward kernel, causal GQA B=2 S=4096 Hq=32 Hkv=4 D=512 (bench.py workload)",
     "Algorithmic bytes: Q, K, V read once (268 + 33.5 + 33.5 MB) and O, LSE written once (268 + 1 MB).  "
     "The fetch figure counts every L2 miss sent to the fabric (the 256 MB last-level cache can serve part "
     "of it); above the algorithmic reads it is the K/V re-reads of the query-row tiles of each head group."),
    ("bwd_dkdv_d512_B2_S4096_traffic.txt", "bwd_dkdv_kernel<512,false,false>", "scaled_dot_product_tiled_amd/csrc/attn_bwd.hip",
     "dK/dV kernel of the backward, causal GQA B=2 S=4096 Hq=32 Hkv=4 D=512 (bench.py workload)",
     "Algorithmic bytes: Q, dO read once (268 MB each), K, V (33.5 MB each), LSE and delta (1 MB each); "
     "writes dK, dV (33.5 MB each) and the stored dS blocks (1.107 GB).  Fetch above the algorithmic reads "
     "is the Q / dO re-reads of the 64 key tiles of each head group that miss in L2."),
    ("bwd_dq_d512_B2_S4096_traffic.txt", "bwd_dq_kernel<256,4,2,false>", "scaled_dot_product_tiled_amd/csrc/attn_bwd.hip",
     "dQ kernel of the backward (dQ = scale dS K over the stored dS blocks, two head_dim halves), same workload",
     "Algorithmic bytes: dS blocks read once (1.107 GB), K (33.5 MB); dQ written once (268 MB).  Each dS "
     "block is read by both head_dim halves; the second read is meant to hit in L2."),
    ("decode_split_d128_B64_traffic.txt", "decode_split_kernel<4,false,false>", "scaled_dot_product_tiled_amd/csrc/attn_decode.hip",
     "paged decode split kernel, B=64 Hq=32 Hkv=8 D=128, 16-token pages, contexts U{512..4096} "
     "(bench.py decode workload)",
     "Algorithmic bytes: K and V of every context token once (619.6 MB per launch, the bench's "
     "bytes_per_launch); writes the chunk partials (about 5.5 MB)."),
]


def write_summaries(out: str, pdir: str) -> None:
    import json
    for fn, k, src, what, note in TRAFFIC_SUMMARIES:
        rec = traffic_record(k, os.path.join(ROOT, src), os.path.join(out, "fetch"), os.path.join(out, "write"),
                             os.path.join(out, "cfetch"), os.path.join(out, "cwrite"), 1024)
        kv = dict(t.split("=", 1) for t in rec[len("record:"):].split())
        txt = (f"HBM traffic per dispatch: {what}\n\n"
               "rocprofv3 counters FETCH_SIZE and WRITE_SIZE (one pass each, averaged over the dispatches of the\n"
               "kernel), scaled by the same counters read for a plain 1 GiB device copy: bytes per counter unit\n"
               f"{kv['fetch_scale']} (FETCH_SIZE) and {kv['write_scale']} (WRITE_SIZE).\n\n"
               f"  fetched {int(kv['fetch_bytes']) / 1e9:.3f} GB   written {int(kv['write_bytes']) / 1e9:.3f} GB   "
               "per dispatch\n\n"
               f"{note}\n\n{COMMANDS}\n"
               "bench.py reads the record line below for its roofline \"traffic\" field, as long as the kernel\n"
               f"source still has the recorded sha256.\n\n{rec}\n")
        with open(os.path.join(pdir, fn), "w") as fh:
            fh.write(txt)
    line = None
    for f in glob.glob(os.path.join(out, "**", "*.log"), recursive=True) + [os.path.join(out, "bench_stats.log")]:
        if os.path.exists(f):
            for ln in open(f):
                if ln.startswith('{"metric"'):
                    line = json.loads(ln)
    txt = ("Kernel times of bench.py on one MI355X: causal GQA forward + backward, B=2 S=4096 Hq=32 Hkv=4\n"
           "D=512 (10 timed + 3 warm-up steps, plus the per-call and per-kernel passes) and the paged decode\n"
           "B=64 Hq=32 Hkv=8 D=128.\n\n"
           f"{COMMANDS}\n{stats_table(os.path.join(out, 'stats'))}\n")
    if line is not None:
        txt += "\nbench.py's own HIP-event timings of the same run (ms per launch):\n"
        for n, v in list(line["kernels"].items()) + list(line["decode"]["kernels"].items()):
            txt += f"  {n:14s} {v['ms_avg']:.4f}\n"
        txt += f"\nbench.py line: value {line['value']} TFLOP/s, ms_per_step {line['ms_per_step']}\n"
    with open(os.path.join(pdir, "bench_d512_B2_S4096_kernel_stats.txt"), "w") as fh:
        fh.write(txt)
    if os.path.isdir(os.path.join(out, "sq")):
        txt = ("Matrix-core and LDS use of the bench.py kernels on one MI355X (causal GQA B=2 S=4096 Hq=32 Hkv=4\n"
               "D=512 forward and backward; paged decode B=64 Hq=32 Hkv=8 D=128), one rocprofv3 pass of SQ\n"
               "counters, averaged over each kernel's dispatches.\n\n"
               "  cycles          shader clocks the kernel was active on one XCD (GRBM_GUI_ACTIVE / 8)\n"
               "  MFMA busy       SQ_VALU_MFMA_BUSY_CYCLES / (cycles x 1024 SIMDs)\n"
               "  LDS B/clk/CU    bytes read from LDS (SQ_INSTS_LDS_LOAD_BANDWIDTH x 64) / (cycles x 256 CUs)\n"
               "  bank confl.     SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE\n"
               "  LDS fifo full   SQ_LDS_DATA_FIFO_FULL / SQ_BUSY_CU_CYCLES\n"
               "  wait LDS issue  wave-cycles waiting to issue an LDS instruction / wave-cycles of 4 waves per CU\n\n"
               f"{COMMANDS}\n{sq_table(os.path.join(out, 'sq'))}\n")
        with open(os.path.join(pdir, "sq_mfma_lds_d512_B2_S4096.txt"), "w") as fh:
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
