"""AddressSanitizer + UndefinedBehaviorSanitizer builds, run on the CPU.

* The oracle (plain C) is built with gcc -fsanitize=address,undefined and
  driven by tests/sanitize/oracle_driver.c over every entry point, ragged
  shapes with empty sequences, all cache storage types, row subsets and the
  rejected configurations, with closed-form checks on the results.
* The library's host code (validation, planning, workspace sizing, the C ABI)
  is built with the same sanitizers (host only: -Xarch_host) and driven by
  tests/sanitize/abi_driver.c through calls that the host answers before any
  device call.

Any sanitizer report aborts the driver (-fno-sanitize-recover=all) and fails
the test.  (mlxd PR #99 ran its suites under ASan and UBSan; the same
discipline for the parts here that run on the host.)
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def run(cmd, env=None, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, env=env, **kw)
    assert res.returncode == 0, f"{' '.join(cmd)}\n{res.stdout}\n{res.stderr[-4000:]}"
    return res


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_is_clean_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", *SAN, "-I", os.path.join(ROOT, "oracle"),
         os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"), os.path.join(ROOT, "oracle", "qsa_oracle.c"),
         "-lm", "-o", exe])
    env = dict(os.environ, OMP_NUM_THREADS="4", ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    out = run([exe], env=env).stdout
    assert "clean" in out


HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="needs hipcc")
def test_c_abi_host_code_is_clean_under_asan_and_ubsan(tmp_path):
    from gated_gqa_attention_amd import build as B

    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all"]
    flags = [f for f in B.FLAGS if f != "-O3"] + ["-O1", "-g", "-Wno-inline-asm"]

    def compile_one(src):
        obj = str(tmp_path / (os.path.splitext(src)[0] + ".o"))
        run([HIPCC, *flags, *host_san, "-c", os.path.join(B.CSRC, src), "-o", obj])
        return obj

    with ThreadPoolExecutor(max_workers=len(B.SOURCES)) as ex:
        objs = list(ex.map(compile_one, B.SOURCES))
    exe = str(tmp_path / "abi_driver")
    run([HIPCC, f"--offload-arch={B.ARCH}", *host_san, "-I", os.path.join(ROOT, "include"),
         "-x", "c", os.path.join(ROOT, "tests", "sanitize", "abi_driver.c"), "-x", "none", *objs, "-o", exe])
    # the HIP runtime keeps allocations until exit, so leak reports are off here
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    out = run([exe], env=env).stdout
    assert "clean" in out
