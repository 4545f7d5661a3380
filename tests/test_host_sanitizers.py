"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

libmsa.so is rebuilt with the sanitizers on its host side only (device code
is compiled as usual and never runs here), and the boundary tests -- which
drive every entry point's argument validation, workspace sizing, status
strings and the exported-symbol checks without a GPU -- run against it in
a child interpreter with clang's ASan runtime preloaded and Python's own
allocations routed through malloc, so an overrun of a caller's buffer is
seen too.  Any report ends the child and fails this test.
"""
import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_attention_10_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN = ["-Xarch_host", "-fsanitize=address,undefined",
       "-Xarch_host", "-fno-sanitize-recover=all",
       "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-shared-libasan"]
FLAGS = ["-O1", "-g", "-std=c++17", "--offload-arch=gfx950", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found and os.path.exists(HIPCC) else None


def _compile(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr


def test_boundary_tests_pass_against_a_host_sanitized_library(tmp_path):
    runtime = _asan_runtime()
    if runtime is None:
        pytest.skip("hipcc or clang's AddressSanitizer runtime is not installed")
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [str(tmp_path / (os.path.basename(s)[:-4] + ".o")) for s in srcs]
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        list(ex.map(_compile, [[HIPCC, *FLAGS, *SAN, "-c", s, "-o", o]
                               for s, o in zip(srcs, objs)]))
    so = str(tmp_path / "libmsa.so")
    _compile([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *SAN, "-o", so, *objs])

    env = dict(os.environ)
    env.update(
        LD_PRELOAD=runtime,
        PYTHONMALLOC="malloc",
        ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
        UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
        MSA_LIBRARY=so,
    )
    which = "import block_sparse_attention_10_amd as m; print(m.library_path())"
    probe = subprocess.run([sys.executable, "-c", which], cwd=ROOT, env=env,
                           capture_output=True, text=True, timeout=300)
    assert probe.returncode == 0 and probe.stdout.strip() == so, probe.stdout + probe.stderr
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider",
           os.path.join(ROOT, "tests", "test_boundary.py")]
    res = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (res.stdout + res.stderr)[-4000:]
    assert res.returncode == 0, tail
    assert " passed" in res.stdout, tail
