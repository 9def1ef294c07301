"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The float64 oracle (oracle/ssd_oracle.c) built with gcc -fsanitize=address,
  undefined and driven on small shapes through every path of its forward and
  backward (tests/sanitize/oracle_driver.c).
* The oracle's own pin tests (tests/test_oracle.py, tests/test_oracle_state.py)
  run in a child Python process against a sanitized build of the oracle
  library, with the sanitizer runtimes preloaded.
* libssd's C-ABI host code -- argument checks, workspace layout, the entry
  points' rejection paths -- built from the library's sources with the
  sanitizers on the host side only (hipcc -Xarch_host), and driven with no
  GPU: no call in tests/sanitize/abi_driver.cpp gets past the checks.

Any sanitizer report fails the run (-fno-sanitize-recover / halt_on_error).
"""
import concurrent.futures as cf
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "state_space_model_mamba2_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
GCC_SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
HIP_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all"]


def _run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    return r.returncode, r.stdout, r.stderr


def _clean(rc, out, err, what):
    assert rc == 0, f"{what} failed (rc {rc}):\n{out[-3000:]}\n{err[-3000:]}"
    for bad in ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer"):
        assert bad not in err and bad not in out, f"{what}: sanitizer report\n{err[-3000:]}"


@pytest.fixture(scope="module")
def build_dir(tmp_path_factory):
    return tmp_path_factory.mktemp("sanitize")


def test_oracle_driver_under_asan_ubsan(build_dir):
    exe = str(build_dir / "oracle_driver")
    rc, out, err = _run(["gcc", "-O1", "-g", "-std=c99", "-fopenmp", "-ffp-contract=off", *GCC_SAN,
                         os.path.join(SAN, "oracle_driver.c"), os.path.join(ROOT, "oracle", "ssd_oracle.c"),
                         "-o", exe, "-lm"])
    _clean(rc, out, err, "gcc")
    rc, out, err = _run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1"))
    _clean(rc, out, err, "oracle driver")
    assert "oracle sanitizer driver: ok" in out


def test_oracle_pins_against_sanitized_oracle(build_dir):
    lib = str(build_dir / "libssd_oracle_asan.so")
    rc, out, err = _run(["gcc", "-O1", "-g", "-std=c99", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
                         *GCC_SAN, os.path.join(ROOT, "oracle", "ssd_oracle.c"), "-o", lib, "-lm"])
    _clean(rc, out, err, "gcc")
    runtimes = [subprocess.run(["gcc", f"-print-file-name={n}"], capture_output=True, text=True).stdout.strip()
                for n in ("libasan.so", "libubsan.so")]
    env = dict(os.environ, SSD_ORACLE_LIB=lib, LD_PRELOAD=":".join(runtimes),
               ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    rc, out, err = _run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                         os.path.join(ROOT, "tests", "test_oracle.py"),
                         os.path.join(ROOT, "tests", "test_oracle_state.py")], env=env, timeout=900)
    _clean(rc, out, err, "oracle pin tests")
    assert " passed" in out


def test_abi_host_code_under_asan_ubsan(build_dir):
    common = ["-O1", "-g", "-std=c++17", f"--offload-arch=gfx950", "-I", os.path.join(ROOT, "include"),
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument",
              *HIP_SAN]
    srcs = ["fwd.hip", "bwd.hip", "pad.hip", "conv.hip", "api.cpp"]

    def compile_one(src):
        obj = str(build_dir / (os.path.basename(src) + ".o"))
        cmd = [HIPCC, *common, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        return obj, _run(cmd)

    with cf.ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        results = list(ex.map(compile_one, srcs))
    objs = []
    for obj, (rc, out, err) in results:
        _clean(rc, out, err, f"hipcc {obj}")
        objs.append(obj)
    drv = str(build_dir / "abi_driver.o")
    rc, out, err = _run([HIPCC, "-O1", "-g", "-std=c++17", "-I", os.path.join(ROOT, "include"), *HIP_SAN,
                         "-c", os.path.join(SAN, "abi_driver.cpp"), "-o", drv])
    _clean(rc, out, err, "hipcc driver")
    exe = str(build_dir / "abi_driver")
    rc, out, err = _run([HIPCC, f"--offload-arch=gfx950", *HIP_SAN, *objs, drv, "-o", exe])
    _clean(rc, out, err, "link")
    # the HIP runtime keeps allocations to process exit; leak checks are off
    rc, out, err = _run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=0"))
    _clean(rc, out, err, "abi driver")
    assert "abi sanitizer driver: ok" in out
