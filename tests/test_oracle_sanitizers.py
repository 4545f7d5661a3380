"""The C oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

The oracle's C source is compiled a second time with gcc's address and
undefined-behaviour sanitizers (every report fatal) and a subset of the
oracle pins runs against that build in a child interpreter with the ASan
runtime preloaded.  The subset reaches every exported function: the three
decoders and two encoders, index scores, selection, page table, attention
(plain, masked and with a custom scale), the write path, and one planted
end-to-end run.  An out-of-bounds read or write, a signed overflow or a bad
shift in the oracle ends the child with a report and fails this test.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "msa_oracle.c")

# fast pins that together call every function of the C oracle
SUBSET = " or ".join([
    "decoder", "encoder", "test_block_scores_brute_force", "closed_form",
    "test_selection_ties_go_to_lower_block", "test_dense_equality_up_to_2048_keys and kw0",
    "test_masked_dense_brute_force and kw1", "test_custom_softmax_scale",
    "test_insert_writes", "test_decode_after_insert", "test_planted_blocks_recovered and tiny",
])


def _asan_runtime():
    if shutil.which("gcc") is None:
        return None
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_pins_pass_under_address_and_ub_sanitizers(tmp_path):
    runtime = _asan_runtime()
    if runtime is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    so = str(tmp_path / "libmsa_oracle_san.so")
    subprocess.check_call([
        "gcc", "-O1", "-g", "-std=c99", "-fopenmp", "-fPIC", "-shared",
        "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
        "-fno-omit-frame-pointer", "-o", so, SRC, "-lm"])
    env = dict(os.environ)
    env.update(
        LD_PRELOAD=runtime,
        ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
        UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
        MSA_ORACLE_LIB=so,
        OMP_NUM_THREADS="4",
    )
    which = "from oracle import oracle as o; print(o.lib()._name)"
    probe = subprocess.run([sys.executable, "-c", which], cwd=ROOT, env=env,
                           capture_output=True, text=True, timeout=300)
    assert probe.returncode == 0 and probe.stdout.strip() == so, probe.stdout + probe.stderr
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider",
           os.path.join(ROOT, "tests", "test_oracle_pins.py"), "-k", SUBSET]
    res = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (res.stdout + res.stderr)[-4000:]
    assert res.returncode == 0, tail
    assert " passed" in res.stdout and "deselected" in res.stdout, tail
