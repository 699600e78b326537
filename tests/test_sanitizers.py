"""Host AddressSanitizer + UndefinedBehaviorSanitizer runs (CPU, no GPU).

* The fp64 oracle (oracle/gdn_oracle.c) built with the sanitizers and driven
  on small inputs that reach all of its branches (tests/san/oracle_driver.c).
* The C ABI front end (csrc/gdn_api.cpp and csrc/host_layout.cpp: every
  argument check that runs before a launch) built with the sanitizers against
  a launcher stub and driven through every entry point with valid and invalid
  arguments, sizes at the accepted limits included (tests/san/abi_driver.c).
Any invalid access, leak or undefined operation aborts the driver."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1",
           OMP_NUM_THREADS="2")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", *SAN, "-ffp-contract=off", "-fopenmp", os.path.join(ROOT, "tests", "san", "oracle_driver.c"),
          os.path.join(ROOT, "oracle", "gdn_oracle.c"), "-lm", "-o", exe])
    r = _run([exe], env=ENV, timeout=120)
    assert "oracle driver: ok" in r.stdout


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="g++ or the ROCm headers not available")
def test_c_abi_front_end_under_asan_ubsan(tmp_path):
    csrc = os.path.join(ROOT, "gateddeltanet_chunked_delta_amd", "csrc")
    inc = ["-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include")]
    objs = []
    for src in (os.path.join(csrc, "gdn_api.cpp"), os.path.join(csrc, "host_layout.cpp"),
                os.path.join(ROOT, "tests", "san", "stub_launch.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run(["g++", "-std=c++17", *SAN, *inc, "-c", src, "-o", obj])
        objs.append(obj)
    drv = str(tmp_path / "abi_driver.o")
    _run(["gcc", "-std=c11", *SAN, "-I" + os.path.join(ROOT, "include"), "-c",
          os.path.join(ROOT, "tests", "san", "abi_driver.c"), "-o", drv])
    exe = str(tmp_path / "abi_san")
    _run(["g++", *SAN, drv, *objs, "-o", exe])
    r = _run([exe], env=ENV, timeout=120)
    assert "abi driver: ok" in r.stdout
