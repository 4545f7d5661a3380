"""The counter summariser behind roofline.traffic (summarize_counters.py):
every library kernel that msa_decode launches maps to a source family, and
the bytes it reports follow from the counter files and the copy calibration.
CPU only; the counter files are written here, not taken from a GPU run."""
import csv
import glob
import json
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import summarize_counters as sc  # noqa: E402

CSRC = os.path.join(ROOT, "block_sparse_attention_10_amd", "csrc")
# kernels that msa_decode never launches, so no counter run measures them
UNMEASURED = {"insert_kernel", "input_check_kernel", "page_table_kernel", "selftest_kernel"}


def kernel_names():
    names = set()
    for path in glob.glob(os.path.join(CSRC, "*.hip")):
        src = open(path).read()
        names |= set(re.findall(r"__global__[^;{]*?\bvoid\s+(\w+)\s*\(", src, re.S))
    return names


def test_every_decode_kernel_has_a_family():
    names = kernel_names()
    assert {"index_scan_kernel", "index_scan_q4_kernel", "sparse_attn_kernel",
            "union_attn_kernel", "lse_merge_kernel", "select_kernel"} <= names
    for n in sorted(names - UNMEASURED):
        # as rocprofv3 names a template instance
        full = f"void msa::(anonymous namespace)::{n}<1, 8>(int const*, float*)"
        fam = sc.family_of(full)
        assert fam is not None, n
        assert n.startswith(fam), (n, fam)
    assert sc.family_of("copy16(u32x4 const*, u32x4*, unsigned long)") is None


def test_source_hash_covers_the_family_sources():
    for fam, files in sc.SOURCES.items():
        for f in files:
            assert os.path.exists(os.path.join(CSRC, f)), (fam, f)
        assert re.fullmatch(r"[0-9a-f]{16}", sc.source_hash(fam))


def write_counters(path, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, counter, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_bytes_per_launch_from_counters(tmp_path):
    # a 2-request spec: contexts 300 and 128 tokens -> 3 + 1 causal blocks
    spec = tmp_path / "w.spec"
    spec.write_text("2 1 8 1 2 4 16 bf16 bf16 16\n300 128\n")
    scan = "void msa::(anonymous namespace)::index_scan_q4_kernel<0>(unsigned short const*)"
    attn = "void msa::(anonymous namespace)::sparse_attn_kernel<0, 8, true>(unsigned short const*)"
    copy = "copy16(u32x4 const*, u32x4*, unsigned long)"
    # the copy moves 1 MiB: FETCH_SIZE reads half of it in KiB (factor 2),
    # WRITE_SIZE all of it (factor 1)
    write_counters(tmp_path / "cf.csv", [(copy, "FETCH_SIZE", 512.0)] * 3)
    write_counters(tmp_path / "cw.csv", [(copy, "WRITE_SIZE", 1024.0)] * 3)
    write_counters(tmp_path / "f.csv", [(scan, "FETCH_SIZE", 30.0), (scan, "FETCH_SIZE", 34.0),
                                        (attn, "FETCH_SIZE", 100.0)])
    write_counters(tmp_path / "w.csv", [(scan, "WRITE_SIZE", 1.0), (scan, "WRITE_SIZE", 1.0),
                                        (attn, "WRITE_SIZE", 4.0)])
    out = tmp_path / "out.json"
    subprocess.run([sys.executable, os.path.join(ROOT, "summarize_counters.py"),
                    "--spec", str(spec), "--workload", "w",
                    "--fetch", str(tmp_path / "f.csv"), "--write", str(tmp_path / "w.csv"),
                    "--copy-fetch", str(tmp_path / "cf.csv"),
                    "--copy-write", str(tmp_path / "cw.csv"),
                    "--copy-mib", "1", "--out", str(out)], check=True, capture_output=True)
    r = json.loads(out.read_text())
    assert r["copy_calibration"]["fetch_factor"] == 2.0
    assert r["copy_calibration"]["write_factor"] == 1.0
    k = r["kernels"]["index_scan"]
    assert k["kernel"] == "void msa::index_scan_q4_kernel<0>"
    assert k["launches"] == 2
    assert k["hbm_read_bytes_per_launch"] == 32 * 1024 * 2
    assert k["hbm_write_bytes_per_launch"] == 1024
    # 4 causal blocks x 2 index heads x 128 tokens x 128 B (bf16 keys)
    assert k["algorithmic_bytes_per_launch"] == 4 * 2 * 128 * 128
    assert k["traffic_over_algorithmic"] == pytest.approx((65536 + 1024) / 131072)
    a = r["kernels"]["sparse_attn"]
    assert a["hbm_read_bytes_per_launch"] == 100 * 1024 * 2
    assert a["hbm_write_bytes_per_launch"] == 4 * 1024
    assert a["kernel_source_sha256_16"] == sc.source_hash("sparse_attn")
