"""The library's host code under AddressSanitizer and LeakSanitizer (CPU
only): every source compiled with the sanitizer on its host pass, linked
with tests/asan/host_checks.c, which drives the C ABI's argument checks, its
status strings, the two-wave rule, and a workspace creation that, without a
GPU, fails at its first HIP call and must release what it had built.  The
GPU code is not instrumented (no sanitizer runs on the device here)."""
import concurrent.futures as cf
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mixture_experts_layer_device_amd", "csrc")
SOURCES = ["api.hip", "schedule.hip", "route.hip", "rows.hip", "router_bwd.hip", "gemm_bf16.hip", "gemm_mxfp8.hip"]
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
# the sanitizer applies to the host pass only
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{err}"


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm toolchain not found")
def test_host_code_under_address_sanitizer(tmp_path):
    inc = os.path.join(ROOT, "include")
    objs = [str(tmp_path / (os.path.splitext(src)[0] + ".o")) for src in SOURCES]
    # (device code is built as for the library, the host pass with the sanitizer)
    dev = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    with cf.ThreadPoolExecutor(max_workers=4) as ex:
        list(ex.map(lambda so: _run([HIPCC, *dev, "-O1", "-g", "-std=c++17", "-fPIC", *SAN, "-I", inc, "-c",
                                     os.path.join(CSRC, so[0]), "-o", so[1]]), zip(SOURCES, objs)))
    drv = str(tmp_path / "host_checks.o")
    _run([CLANG, "-O1", "-g", "-fsanitize=address", "-fno-omit-frame-pointer", "-I", inc, "-c",
          os.path.join(ROOT, "tests", "asan", "host_checks.c"), "-o", drv])
    exe = str(tmp_path / "host_checks")
    _run([HIPCC, "--offload-arch=gfx950", *SAN, *objs, drv, "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert "AddressSanitizer" not in r.stderr and "LeakSanitizer" not in r.stderr, r.stderr[-4000:]
    assert r.returncode == 0, r.stdout + r.stderr[-4000:]
    assert "host checks ok" in r.stdout
