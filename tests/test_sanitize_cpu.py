"""AddressSanitizer / UndefinedBehaviorSanitizer builds, on the CPU:

  * the oracle (plain C), driven on small seeded inputs and edge cases by
    tests/sanitize/oracle_drive.c;
  * the library's host code (argument checks, error text, workspace sizing of
    every entry point), with the HIP sources compiled for gfx950 and the host
    half instrumented, driven by tests/sanitize/abi_drive.cpp with valid and
    invalid arguments (no call reaches a kernel launch).
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "sparse_attention_dim_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, cwd, timeout=600):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True, timeout=timeout, env=ENV)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout[-3000:], r.stderr[-3000:])
    return r


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_drive")
    _run(["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-mfma", *SAN, "-o", exe,
          os.path.join(HERE, "oracle_drive.c"), os.path.join(ROOT, "oracle", "rtp_oracle.c"), "-lm"], str(tmp_path))
    r = _run([exe], str(tmp_path))
    assert "oracle drive ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr


@pytest.mark.skipif(not os.path.exists("/opt/rocm/bin/hipcc"), reason="needs hipcc")
def test_abi_host_code_under_sanitizers(tmp_path):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    objs = []
    # device code for gfx950 as usual; only the host half is instrumented
    host_san = [x for f in SAN for x in ("-Xarch_host", f)]
    for src in sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp"))):
        o = str(tmp_path / (src + ".o"))
        _run([hipcc, "--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-std=c++17", *host_san,
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-x", "hip", "-c",
              os.path.join(CSRC, src), "-o", o], str(tmp_path))
        objs.append(o)
    drv = str(tmp_path / "abi_drive.o")
    _run(["g++", "-O1", "-g", "-std=c++17", *SAN, "-c", os.path.join(HERE, "abi_drive.cpp"), "-o", drv],
         str(tmp_path))
    exe = str(tmp_path / "abi_drive")
    _run(["g++", *SAN, "-o", exe, drv, *objs, "-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64"],
         str(tmp_path))
    r = _run([exe], str(tmp_path))
    assert "abi drive ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
