"""Host sanitizer runs (no GPU): the fp64 oracle and the C-ABI validation
code built with AddressSanitizer and UndefinedBehaviorSanitizer, driven by
small C/C++ programs under tests/sanitize/. The kernels themselves are not
instrumented (GPU sanitizers are not used here); the C-ABI driver only makes
calls that are rejected, are no-ops or are size queries, so no HIP call runs.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(map(str, cmd))}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_address_and_ub_sanitizers(tmp_path):
    exe = tmp_path / "oracle_driver"
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
    run(["gcc", "-std=c11", "-O1", "-g", *san, "-pthread", "-I", os.path.join(ROOT, "oracle"),
         os.path.join(SAN, "oracle_driver.c"), os.path.join(ROOT, "oracle", "kda_oracle.c"),
         "-o", str(exe), "-lm"])
    r = run([str(exe)], env=dict(ENV, ASAN_OPTIONS="detect_leaks=1"), timeout=120)
    assert "MISMATCH" not in r.stdout and r.stdout.count(": ok") == 5, r.stdout


HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="needs hipcc")
def test_abi_validation_under_address_and_ub_sanitizers(tmp_path):
    from gated_delta_rule_22_amd import _build
    objs = [os.path.join(_build.BUILD, s.rsplit(".", 1)[0] + ".o") for s in _build.SOURCES
            if s != "kda_api.cpp"]
    if not all(os.path.exists(o) for o in objs):
        _build.build()
    # host-side instrumentation only: each sanitizer flag goes to the host pass
    host_san = []
    for flag in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all"):
        host_san += ["-Xarch_host", flag]
    common = [f"--offload-arch={_build.ARCH}", "-O1", "-g", "-std=c++17", "-fPIC",
              "-I", os.path.join(ROOT, "include"), "-I", _build.CSRC, *host_san]
    api = tmp_path / "kda_api_san.o"
    drv = tmp_path / "abi_driver.o"
    exe = tmp_path / "abi_driver"
    run([HIPCC, *common, "-x", "hip", "-c", os.path.join(_build.CSRC, "kda_api.cpp"), "-o", str(api)])
    run([HIPCC, *common, "-c", os.path.join(SAN, "abi_driver.cpp"), "-o", str(drv)])
    run([HIPCC, f"--offload-arch={_build.ARCH}", *host_san, str(drv), str(api), *objs, "-o", str(exe)])
    r = run([str(exe)], env=ENV, timeout=120)
    assert "0 failures" in r.stdout, r.stdout
