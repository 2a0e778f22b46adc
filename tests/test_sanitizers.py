"""AddressSanitizer / UndefinedBehaviorSanitizer builds, CPU only.

* The FP64 oracle (plain C) is built with gcc under both sanitizers and run
  over small seeded shapes (tests/sanitize/oracle_harness.c).
* The library is built with its host code under both sanitizers (device code
  unchanged) and linked into tests/sanitize/capi_harness.cpp, which drives
  every C-ABI entry point through its validation and size arithmetic,
  including extreme shapes.  It runs in a child process that sees no GPU:
  calls that pass validation then fail at their first launch, so the made-up
  device addresses are never touched (the harness refuses to run if a device
  is visible).
"""
import concurrent.futures as cf
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "linear_recurrence_sequence_amd", "csrc")
SAN = os.path.join(ROOT, "tests", "sanitize")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
SOURCES = ["capi.cpp", "prefix.hip", "samu_fwd.hip", "samu_bwd.hip", "samu_decode.hip", "rglru.hip",
           "baseline.hip", "gate_proj.hip", "noalloc.hip"]
# host-side sanitizer flags: each one behind -Xarch_host, so device code is built as usual
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _env():
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    env.update(HIP_VISIBLE_DEVICES="", ROCR_VISIBLE_DEVICES="", CUDA_VISIBLE_DEVICES="")
    return env


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_harness")
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fopenmp", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-o", exe, os.path.join(SAN, "oracle_harness.c"),
           os.path.join(ROOT, "oracle", "oracle.c"), "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([exe], capture_output=True, text=True, env=_env(), timeout=600)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "all outputs finite" in r.stdout


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_capi_validation_under_asan_ubsan(tmp_path):
    common = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Xclang", "-target-feature",
              "-Xclang", "-packed-fp32-ops", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"] + HOST_SAN

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        r = subprocess.run([HIPCC, "-x", "hip", "-c", src, "-o", obj] + common, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return obj

    srcs = [os.path.join(CSRC, s) for s in SOURCES] + [os.path.join(SAN, "capi_harness.cpp")]
    with cf.ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, srcs))
    exe = str(tmp_path / "capi_harness")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-o", exe] + objs + HOST_SAN[:4], capture_output=True,
                       text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([exe], capture_output=True, text=True, env=_env(), timeout=600)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "checks passed" in r.stdout
