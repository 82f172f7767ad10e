"""Condense rocprofv3 CSV output into the short text summaries kept in profiles/.

    python -m spherical_block_sparse_amd.rocprof_summary stats  <kernel_stats.csv>
    python -m spherical_block_sparse_amd.rocprof_summary counters <counter_collection.csv> [--kernel REGEX]
    python -m spherical_block_sparse_amd.rocprof_summary traffic --fetch F.csv --write W.csv \
        --copy-fetch CF.csv --copy-write CW.csv --copy-mib N --kernel REGEX --source FILE
    python -m spherical_block_sparse_amd.rocprof_summary duration <kernel_stats.csv> --kernel REGEX --source FILE

`stats` lists name, calls, average / min / max duration of every kernel.
`counters` sums each counter over the dispatches of the matching kernels and
prints the per-dispatch mean (FETCH_SIZE and WRITE_SIZE are in KiB).
`traffic` turns one FETCH_SIZE pass and one WRITE_SIZE pass of a kernel into
HBM bytes per dispatch, each scaled by the ratio of the known bytes of a
plain N MiB copy to what the same counter reported for it, and records the
SHA-256 of the kernel source so a later reader can tell whether the kernel
has changed since.
`duration` records the mean duration of the one kernel matching REGEX in a
--kernel-trace --stats run, with the same source hash.  With --update
FILE --key NAME either record is merged into that JSON file under NAME.
"""

from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import re
import sys


def short(name: str) -> str:
    name = name.replace("(anonymous namespace)::", "").replace("void ", "", 1)
    name = re.sub(r"\(.*", "", name)          # drop the argument list
    return name[:90]


def stats(path: str) -> str:
    rows = list(csv.DictReader(open(path)))
    out = [f"{'kernel':<70} {'calls':>6} {'avg ms':>10} {'min ms':>10} {'max ms':>10} {'%':>6}"]
    for r in rows:
        out.append(f"{short(r['Name']):<70} {int(r['Calls']):>6} {float(r['AverageNs']) / 1e6:>10.3f} "
                   f"{float(r['MinNs']) / 1e6:>10.3f} {float(r['MaxNs']) / 1e6:>10.3f} {float(r['Percentage']):>6.2f}")
    return "\n".join(out)


def counters(path: str, kernel: str | None) -> str:
    rows = list(csv.DictReader(open(path)))
    if kernel:
        rows = [r for r in rows if re.search(kernel, r["Kernel_Name"])]
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    names = {}
    for r in rows:
        per[r["Dispatch_Id"]][r["Counter_Name"]] += float(r["Counter_Value"])
        names[r["Dispatch_Id"]] = short(r["Kernel_Name"])
    out = []
    keys = sorted({c for d in per.values() for c in d})
    out.append(f"{'dispatch':>8} {'kernel':<50} " + " ".join(f"{k:>22}" for k in keys))
    for did in sorted(per, key=lambda x: int(x)):
        out.append(f"{did:>8} {names[did]:<50} " + " ".join(f"{per[did][k]:>22.6g}" for k in keys))
    n = max(1, len(per))
    out.append(f"{'mean':>8} {'':<50} " + " ".join(f"{sum(d[k] for d in per.values()) / n:>22.6g}" for k in keys))
    return "\n".join(out)


def mean_counter(path: str, kernel: str, counter: str) -> float:
    rows = [r for r in csv.DictReader(open(path))
            if re.search(kernel, r["Kernel_Name"]) and r["Counter_Name"] == counter]
    per = collections.defaultdict(float)
    for r in rows:
        per[r["Dispatch_Id"]] += float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"no {counter} rows for /{kernel}/ in {path}")
    return sum(per.values()) / len(per)


def traffic(a) -> dict:
    known_kib = a.copy_mib * 1024.0
    rf = known_kib / mean_counter(a.copy_fetch, "copy", "FETCH_SIZE")
    wf = known_kib / mean_counter(a.copy_write, "copy", "WRITE_SIZE")
    fetch = mean_counter(a.fetch, a.kernel, "FETCH_SIZE")
    write = mean_counter(a.write, a.kernel, "WRITE_SIZE")
    return {
        "kernel_regex": a.kernel,
        "source": a.source,
        "source_sha256": hashlib.sha256(open(a.source, "rb").read()).hexdigest(),
        "fetch_kib_per_dispatch": fetch, "write_kib_per_dispatch": write,
        "copy_mib": a.copy_mib, "read_factor": rf, "write_factor": wf,
        "hbm_read_bytes": fetch * rf * 1024.0, "hbm_write_bytes": write * wf * 1024.0,
        "hbm_bytes": (fetch * rf + write * wf) * 1024.0,
    }


def duration(a) -> dict:
    rows = [r for r in csv.DictReader(open(a.csv)) if re.search(a.kernel, r["Name"])]
    if len(rows) != 1:
        raise SystemExit(f"/{a.kernel}/ matches {len(rows)} kernels in {a.csv}")
    r = rows[0]
    return {
        "kernel_regex": a.kernel,
        "source": a.source,
        "source_sha256": hashlib.sha256(open(a.source, "rb").read()).hexdigest(),
        "calls": int(r["Calls"]), "avg_ms": float(r["AverageNs"]) / 1e6,
        "min_ms": float(r["MinNs"]) / 1e6, "max_ms": float(r["MaxNs"]) / 1e6,
    }


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("mode", choices=["stats", "counters", "traffic", "duration"])
    ap.add_argument("csv", nargs="?")
    ap.add_argument("--kernel", default=None)
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--copy-fetch")
    ap.add_argument("--copy-write")
    ap.add_argument("--copy-mib", type=int, default=0)
    ap.add_argument("--source")
    ap.add_argument("--update", help="JSON file to merge the record into")
    ap.add_argument("--key", help="name of the record in --update")
    a = ap.parse_args()
    if a.mode == "stats":
        print(stats(a.csv))
        return 0
    if a.mode == "counters":
        print(counters(a.csv, a.kernel))
        return 0
    rec = traffic(a) if a.mode == "traffic" else duration(a)
    print(json.dumps(rec, indent=1))
    if a.update:
        try:
            allrec = json.load(open(a.update))
        except FileNotFoundError:
            allrec = {}
        allrec[a.key] = rec
        with open(a.update, "w") as f:
            json.dump(allrec, f, indent=1, sort_keys=True)
            f.write("\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())
