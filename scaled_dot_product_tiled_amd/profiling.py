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
    names = [n for n in values if kernel in n]
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
    a = p.parse_args(argv)
    if a.cmd == "copy":
        run_copy(a.mib, a.reps)
    elif a.cmd == "stats":
        print(stats_table(a.dir))
    else:
        print(traffic_record(a.kernel, a.source, a.fetch, a.write, a.copy_fetch, a.copy_write, a.copy_mib))
    return 0


if __name__ == "__main__":
    sys.exit(main())
