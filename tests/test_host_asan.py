"""The host library under AddressSanitizer, on the CPU: clef_head.cpp is
compiled with ASan on its host code (device code stays unsanitised), linked
with the library's kernel objects and the C driver tests/host/abi_checks.cpp,
which runs batch validation and planning, every error path, the weight
enumeration and create's early failure paths.  Any invalid access or leak in
that code fails the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_host_library_under_asan(tmp_path):
    from structured_decision_head_amd import build as B
    B.build()
    objs = [os.path.join(B.BUILD, os.path.splitext(s)[0] + ".o") for s in B.SOURCES if s != "clef_head.cpp"]
    host = str(tmp_path / "clef_head_asan.o")
    inc = ["-I", B.INCLUDE, "-I", B.CSRC]
    flags = ["-O1", "-g", "-std=c++17", "-fPIC", f"--offload-arch={B.ARCH}", "-fno-omit-frame-pointer",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Xarch_host", "-fsanitize=address"]
    subprocess.run([HIPCC, *flags, *inc, "-x", "hip", "-c", os.path.join(B.CSRC, "clef_head.cpp"), "-o", host],
                   check=True, capture_output=True, text=True)
    drv = str(tmp_path / "abi_checks.o")
    subprocess.run([HIPCC, "-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer", "-Xarch_host", "-fsanitize=address",
                    *inc, "-c", os.path.join(ROOT, "tests", "host", "abi_checks.cpp"), "-o", drv],
                   check=True, capture_output=True, text=True)
    exe = str(tmp_path / "abi_checks")
    subprocess.run([HIPCC, f"--offload-arch={B.ARCH}", "-fsanitize=address", "-fno-gpu-sanitize", "-o", exe, drv, host,
                    *objs], check=True, capture_output=True, text=True)
    supp = tmp_path / "lsan.supp"
    # allocations the ROCm runtime libraries keep for the process's lifetime
    supp.write_text("leak:libamdhip64\nleak:libhsa-runtime64\nleak:libamd_comgr\nleak:libdrm\nleak:libnuma\n")
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=23",
               LSAN_OPTIONS=f"suppressions={supp}", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    print(out[-4000:])
    assert "ERROR: AddressSanitizer" not in out and "ERROR: LeakSanitizer" not in out, out[-4000:]
    assert r.returncode == 0 and "OK: 0 failures" in r.stdout, out[-4000:]
