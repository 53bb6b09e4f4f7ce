"""Summarise rocprofv3 CSV output for one kernel.

    python -m joint_video_audio_amd.counter_summary <csv> <kernel-substring> [copy-bytes]
        [--every N --nth K]

<csv> is a --pmc run's counter_collection.csv or a --kernel-trace run's
kernel_trace.csv. For counters it prints, per counter, the average value per
dispatch of the kernel whose name contains <kernel-substring>; with
copy-bytes, also the value per dispatch of the largest torch copy kernel and
the factor known-bytes / (counter KiB * 1024) that scales the kernel's
counter to bytes. For a kernel trace it prints the average duration.

A kernel-substring that starts with "=" matches the whole name (a kernel
trace names kernels without template arguments, so "k_gemm_bf16" would also
match "k_gemm_bf16_half").

--every N --nth K keeps, of the matching dispatches in dispatch order, those
whose index i has i % N == K: launches of one kernel with different roles
(the output and down projections share a kernel) split by launch order.
"""
import argparse
import collections
import csv


def matching(rows, needle, every=1, nth=0):
    """Dispatch ids of the kernel, in dispatch order, thinned to index % every == nth."""
    if needle.startswith("="):
        hit = lambda name: name == needle[1:]
    else:
        hit = lambda name: needle in name
    ids = sorted({int(r["Dispatch_Id"]) for r in rows if hit(r["Kernel_Name"])})
    return {d for i, d in enumerate(ids) if i % every == nth}


def per_dispatch(path, needle, every=1, nth=0):
    rows = list(csv.DictReader(open(path)))
    keep = matching(rows, needle, every, nth)
    acc = collections.defaultdict(lambda: collections.defaultdict(float))
    for r in rows:
        if int(r["Dispatch_Id"]) in keep:
            acc[r["Counter_Name"]][r["Dispatch_Id"]] += float(r["Counter_Value"])
    return {c: sum(d.values()) / len(d) for c, d in acc.items()}, rows


def mean_duration_ns(path, needle, every=1, nth=0):
    rows = list(csv.DictReader(open(path)))
    keep = matching(rows, needle, every, nth)
    t = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in rows if int(r["Dispatch_Id"]) in keep]
    return sum(t) / len(t), len(t)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("csv")
    ap.add_argument("kernel")
    ap.add_argument("copy_bytes", nargs="?", type=int, default=0)
    ap.add_argument("--every", type=int, default=1)
    ap.add_argument("--nth", type=int, default=0)
    a = ap.parse_args()
    if not 0 <= a.nth < a.every:
        raise SystemExit("need 0 <= nth < every")
    with open(a.csv) as f:
        header = f.readline()
    if "Counter_Name" not in header:
        ns, n = mean_duration_ns(a.csv, a.kernel, a.every, a.nth)
        print(f"{a.kernel}: {n} dispatches, average duration {ns:.0f} ns")
        return
    vals, rows = per_dispatch(a.csv, a.kernel, a.every, a.nth)
    for c, v in sorted(vals.items()):
        print(f"{a.kernel}: {c} = {v:.6e} per dispatch")
    if a.copy_bytes:
        acc = collections.defaultdict(lambda: collections.defaultdict(float))
        for r in rows:
            name = r["Kernel_Name"]
            if "copy" in name.lower() or "elementwise" in name.lower():
                acc[r["Counter_Name"]][(name, r["Dispatch_Id"])] += float(r["Counter_Value"])
        for c, d in sorted(acc.items()):
            v = max(d.values())
            print(f"copy({a.copy_bytes} B): {c} = {v:.6e} per dispatch; "
                  f"bytes/(KiB*1024) = {a.copy_bytes / (v * 1024):.4f}")


if __name__ == "__main__":
    main()
