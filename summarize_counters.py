"""HBM traffic per kernel launch from rocprofv3 counter runs of msa_counters.

Reads the counter_collection CSVs of four runs -- FETCH_SIZE and WRITE_SIZE
of the workload (msa_counters scan|decode), FETCH_SIZE and WRITE_SIZE of the
calibration copy (msa_counters copy <MiB>) -- and writes one JSON file: for
each library kernel the mean counter values per launch, scaled into bytes by
the factor that makes the copy kernel's counters equal the bytes it moves,
plus a hash of the kernel's sources so a reader can tell whether the figures
still describe the code.

    python summarize_counters.py --spec S --fetch F.csv --write W.csv \\
        --copy-fetch CF.csv --copy-write CW.csv --copy-mib 1024 --out OUT.json

With --table and a list of counter_collection CSVs it prints instead a
markdown table of every counter's mean value per launch, per kernel.
"""
import argparse
import collections
import csv
import hashlib
import json
import os
import re
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "block_sparse_attention_10_amd", "csrc")

# kernel family -> the sources that define it
SOURCES = {
    "index_scan": ["index_scan.hip", "msa_device.h"],
    "select": ["topk.hip", "select_device.h", "msa_device.h"],
    "sparse_attn": ["attention.hip", "msa_device.h", "select_device.h"],
    "union_attn": ["attention.hip", "msa_device.h", "select_device.h"],
    "lse_merge": ["attention.hip", "msa_device.h"],
}


def source_hash(family):
    h = hashlib.sha256()
    for f in SOURCES[family]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def family_of(name):
    for fam in SOURCES:
        # index_scan_kernel, index_scan_q4_kernel, sparse_attn_kernel, ...
        if re.search(r"\b" + fam + r"(_q4)?(_kernel)?\b", name):
            return fam
    return None


def per_launch(path, pick):
    """Mean Counter_Value per dispatch of the kernels `pick` accepts, keyed by
    the kernel's family (or name)."""
    vals = collections.defaultdict(list)
    names = {}
    with open(path) as fh:
        for r in csv.DictReader(fh):
            key = pick(r["Kernel_Name"])
            if key is None:
                continue
            vals[key].append(float(r["Counter_Value"]))
            names[key] = r["Kernel_Name"]
    return {k: (sum(v) / len(v), len(v), names[k]) for k, v in vals.items()}


def read_spec(path):
    with open(path) as fh:
        head = fh.readline().split()
        ctx = [int(x) for x in fh.readline().split()]
    B, T, Hq, Hkv, Hidx, MAXB, NB = (int(x) for x in head[:7])
    return dict(B=B, T=T, Hq=Hq, Hkv=Hkv, Hidx=Hidx, MAXB=MAXB, NB=NB, kv=head[7],
                idx=head[8], topk=int(head[9]), ctx=ctx)


def index_key_bytes(spec):
    """Bytes of the index keys of every causal block: the scan's input."""
    per_tok = {"bf16": 128, "fp8": 64, "nvfp4": 36}[spec["idx"]]  # bytes per token and head
    blocks = sum((L + 127) // 128 for L in spec["ctx"])
    return blocks * spec["Hidx"] * 128 * per_tok


def counter_table(paths):
    """Markdown table: mean value per launch of every counter in the given
    counter_collection CSVs, one row per library kernel."""
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    for path in paths:
        with open(path) as fh:
            for r in csv.DictReader(fh):
                fam = family_of(r["Kernel_Name"])
                if fam is None:
                    continue
                name = re.sub(r"\(.*", "", r["Kernel_Name"].replace("(anonymous namespace)::", ""))
                vals[name.replace("void ", "")][r["Counter_Name"]].append(float(r["Counter_Value"]))
    counters = sorted({c for k in vals.values() for c in k})
    lines = ["| kernel | " + " | ".join(counters) + " |",
             "|---|" + "---|" * len(counters)]
    for name, cs in vals.items():
        cells = [f"{sum(cs[c]) / len(cs[c]):,.0f}" if c in cs else "" for c in counters]
        lines.append(f"| {name} | " + " | ".join(cells) + " |")
    return "\n".join(lines)


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--table":
        print(counter_table(sys.argv[2:]))
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("--spec", required=True)
    ap.add_argument("--workload", required=True)
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--copy-fetch", required=True)
    ap.add_argument("--copy-write", required=True)
    ap.add_argument("--copy-mib", type=int, required=True)
    ap.add_argument("--out", required=True)
    a = ap.parse_args()

    copy_bytes = a.copy_mib << 20
    is_copy = lambda n: "copy16" if "copy16" in n else None
    cf = per_launch(a.copy_fetch, is_copy)["copy16"][0]
    cw = per_launch(a.copy_write, is_copy)["copy16"][0]
    # the copy reads and writes copy_bytes; counters are in KiB
    f_factor = copy_bytes / (cf * 1024)
    w_factor = copy_bytes / (cw * 1024)

    fetch = per_launch(a.fetch, family_of)
    write = per_launch(a.write, family_of)
    spec = read_spec(a.spec)
    kernels = {}
    for fam in sorted(fetch):
        fk, n, name = fetch[fam]
        wk = write.get(fam, (0.0, 0, name))[0]
        rd = fk * 1024 * f_factor
        wr = wk * 1024 * w_factor
        kernels[fam] = {
            "kernel": re.sub(r"\(.*", "", name.replace("(anonymous namespace)::", "")),
            "launches": n,
            "fetch_size_kib_per_launch": fk,
            "write_size_kib_per_launch": wk,
            "hbm_read_bytes_per_launch": int(rd),
            "hbm_write_bytes_per_launch": int(wr),
            "hbm_bytes_per_launch": int(rd + wr),
            "kernel_source_sha256_16": source_hash(fam),
        }
    if "index_scan" in kernels:
        alg = index_key_bytes(spec)
        kernels["index_scan"]["algorithmic_bytes_per_launch"] = alg
        kernels["index_scan"]["traffic_over_algorithmic"] = (
            kernels["index_scan"]["hbm_bytes_per_launch"] / alg)
    out = {
        "workload": a.workload,
        "copy_calibration": {
            "bytes_per_launch": copy_bytes,
            "fetch_size_kib": cf,
            "write_size_kib": cw,
            "fetch_factor": f_factor,
            "write_factor": w_factor,
        },
        "kernels": kernels,
    }
    with open(a.out, "w") as fh:
        json.dump(out, fh, indent=1)
    for fam, k in kernels.items():
        print(f"{fam:12s} {k['kernel']:45s} read {k['hbm_read_bytes_per_launch']:>14,d} "
              f"write {k['hbm_write_bytes_per_launch']:>12,d}")


if __name__ == "__main__":
    main()
