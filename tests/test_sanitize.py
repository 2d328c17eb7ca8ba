"""The C oracle and the host side of the C ABI built with AddressSanitizer and UBSan (host
code only) and driven over their edge cases and argument checks: any sanitizer report or
wrong status fails.  CPU only."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1")


def _run(exe):
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=120)
    report = r.stdout + r.stderr
    assert r.returncode == 0, report
    assert "runtime error" not in report and "AddressSanitizer" not in report, report
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_asan")
    subprocess.run(["gcc", "-std=c99", "-O1", "-g", "-ffp-contract=off", *SAN,
                    os.path.join(HERE, "oracle_driver.c"), "-lm", "-o", exe], check=True)
    assert "checksum" in _run(exe)


HIPCC = "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not (os.path.exists(HIPCC) and shutil.which("g++")), reason="needs hipcc and g++")
def test_host_abi_under_sanitizers(tmp_path):
    """api.hip's host code instrumented (each sanitizer flag only for the host pass), linked
    with g++ against the kernels' objects of the regular build."""
    from bit_diffusion_amd import build as B
    objs = [os.path.join(B.OBJ_DIR, os.path.splitext(s)[0] + ".o") for s in B.SOURCES if s != "api.hip"]
    if not all(os.path.exists(o) for o in objs):
        B.build()
    api_o = str(tmp_path / "api_san.o")
    flags = [f for f in B.FLAGS]
    subprocess.run([HIPCC, *flags, "-Xarch_host", "-fsanitize=address,undefined",
                    "-Xarch_host", "-fno-sanitize-recover=all", "-c", os.path.join(B.CSRC, "api.hip"),
                    "-o", api_o], check=True, capture_output=True)
    exe = str(tmp_path / "host_asan")
    subprocess.run(["g++", "-std=c++17", "-g", *SAN, os.path.join(HERE, "host_driver.cpp"), api_o, *objs,
                    "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe],
                   check=True, capture_output=True)
    out = _run(exe)
    assert "0 failures" in out, out
