"""AddressSanitizer and UndefinedBehaviorSanitizer builds of the host code
(CPU only, no GPU needed):

* the CPU oracle (oracle/moe_oracle.c, gcc) driven through every entry point
  on small problems by tests/sanitize/oracle_check.c;
* libmoe's host code, i.e. every source compiled by hipcc with the
  sanitizers on the host side only (device code is built as usual but never
  run), driven by tests/sanitize/abi_host_check.c through the C ABI's
  validation and size queries, which return before anything reaches a
  device.

A sanitizer report or a failed check makes that program exit non-zero."""

import concurrent.futures as cf
import glob
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "dropless_grouped_gemm_router_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

pytestmark = pytest.mark.slow

SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _run(cmd, env=None):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_check")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-ffp-contract=off",
          os.path.join(ROOT, "oracle", "moe_oracle.c"),
          os.path.join(ROOT, "tests", "sanitize", "oracle_check.c"), "-o", exe, "-lm"])
    r = _run([exe], env=dict(SAN_ENV, ASAN_OPTIONS="detect_leaks=1"))
    assert "clean" in r.stdout


def test_abi_host_code_under_asan_ubsan(tmp_path):
    # host-side sanitizers only: each flag follows -Xarch_host
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
    common = ["-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-w", "-I", INCLUDE,
              "-I", CSRC, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        _run([HIPCC] + common + san + lang + ["-c", src, "-o", obj])
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, srcs))
    exe = str(tmp_path / "abi_host_check")
    _run([HIPCC, "--offload-arch=gfx950"] + san + objs +
         ["-x", "c", os.path.join(ROOT, "tests", "sanitize", "abi_host_check.c"), "-I", INCLUDE,
          "-o", exe])
    r = _run([exe], env=SAN_ENV)
    assert "clean" in r.stdout
