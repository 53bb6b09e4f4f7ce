"""Summarise rocprofv3 --pmc CSV output for one kernel.

    python -m joint_video_audio_amd.counter_summary <counter_collection.csv> <kernel-substring> [copy-bytes]

Prints, per counter, the average value per dispatch of the kernel whose name
contains <kernel-substring>; with copy-bytes, also the value per dispatch of
the largest torch copy kernel and the factor known-bytes / (counter KiB *
1024) that scales the kernel's counter to bytes.
"""
import collections
import csv
import sys


def per_dispatch(path, needle):
    rows = list(csv.DictReader(open(path)))
    acc = collections.defaultdict(lambda: collections.defaultdict(float))
    for r in rows:
        if needle in r["Kernel_Name"]:
            acc[r["Counter_Name"]][r["Dispatch_Id"]] += float(r["Counter_Value"])
    return {c: sum(d.values()) / len(d) for c, d in acc.items()}, rows


def main():
    path, needle = sys.argv[1], sys.argv[2]
    copy_bytes = int(sys.argv[3]) if len(sys.argv) > 3 else 0
    vals, rows = per_dispatch(path, needle)
    for c, v in sorted(vals.items()):
        print(f"{needle}: {c} = {v:.6e} per dispatch")
    if copy_bytes:
        acc = collections.defaultdict(lambda: collections.defaultdict(float))
        for r in rows:
            name = r["Kernel_Name"]
            if "copy" in name.lower() or "elementwise" in name.lower():
                acc[r["Counter_Name"]][(name, r["Dispatch_Id"])] += float(r["Counter_Value"])
        for c, d in sorted(acc.items()):
            v = max(d.values())
            print(f"copy({copy_bytes} B): {c} = {v:.6e} per dispatch; bytes/(KiB*1024) = {copy_bytes / (v * 1024):.4f}")


if __name__ == "__main__":
    main()
