"""The fp64 oracle (plain C) and the C ABI's host code, built with
AddressSanitizer and UndefinedBehaviorSanitizer and driven on the CPU:
tests/sanitize/oracle_driver.c runs every oracle entry point on drawn
inputs (-inf gates, one-token sequences, d_k != d_v, recompute blocks);
tests/sanitize/abi_driver.cpp calls every exported function with valid and
invalid arguments, its kernel launchers replaced by stubs (no GPU code runs;
the sanitizers apply to host code only)."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    return r.returncode, r.stdout + r.stderr


@pytest.fixture(scope="module")
def tmp():
    d = tempfile.mkdtemp(prefix="kda_san_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


def test_oracle_clean_under_asan_ubsan(tmp):
    exe = os.path.join(tmp, "oracle_san")
    rc, out = _run(["gcc", "-O1", "-g", "-std=c11", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-fno-fast-math",
                    "-ffp-contract=off", "-I", os.path.join(ROOT, "oracle"),
                    os.path.join(SAN, "oracle_driver.c"),
                    os.path.join(ROOT, "oracle", "kda_oracle.c"), "-lm",
                    "-o", exe])
    assert rc == 0, out
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    rc, out = _run([exe], env=env, timeout=300)
    assert rc == 0 and "clean" in out, out


@pytest.mark.skipif(shutil.which("hipcc") is None and
                    not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_c_abi_clean_under_asan_ubsan(tmp):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    exe = os.path.join(tmp, "abi_san")
    csrc = os.path.join(ROOT, "gated_delta_rule_74_amd", "csrc")
    # sanitizers on host code only (-Xarch_host before each -fsanitize)
    rc, out = _run([hipcc, "-O1", "-g", "-std=c++17",
                    "--offload-arch=gfx950", "-fno-omit-frame-pointer",
                    "-Xarch_host", "-fsanitize=address",
                    "-Xarch_host", "-fsanitize=undefined",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                    "-I", os.path.join(ROOT, "include"), "-I", csrc,
                    os.path.join(csrc, "kda_api.hip"),
                    os.path.join(SAN, "abi_driver.cpp"), "-o", exe],
                   timeout=600)
    assert rc == 0, out
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    rc, out = _run([exe], env=env, timeout=300)
    assert rc == 0 and "0 mismatches" in out, out
