"""The library's host code built with AddressSanitizer and UndefinedBehaviorSanitizer and
driven through the C ABI on the CPU (tests/sanitize/host_checks.cpp): argument checks of
every entry point, empty plans, workspace-size arithmetic over extreme sizes.  Only the
host side of each source is compiled; each translation unit's reference to its device
image is met by an empty offload bundle, so the HIP runtime registers no kernels and
nothing launches.  A sanitizer report fails the run (no recovery), leaks included."""
import concurrent.futures
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "spatial_sparse_attention_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["ssa_plan.hip", "ssa_forward.hip", "ssa_backward.hip", "ssa_api.hip", "ssa_producer.hip",
           "ssa_conv.hip"]
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all"]
FLAGS = ["--offload-host-only", "-O1", "-g", "-fPIC", "-std=c++17", "-I" + os.path.join(ROOT, "include"),
         "-I" + CSRC] + SAN

LIBS = ["-L/opt/rocm/lib", "-lrocprofiler-sdk-roctx", "-Wl,-rpath,/opt/rocm/lib"]

pytestmark = pytest.mark.skipif(not (os.path.exists(HIPCC) and shutil.which("g++")),
                                reason="needs hipcc and g++")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stderr[-4000:]}"


def test_host_code_under_sanitizers(tmp_path):
    jobs = [(os.path.join(CSRC, s), str(tmp_path / s.replace(".hip", ".o"))) for s in SOURCES]
    jobs.append((os.path.join(ROOT, "tests", "sanitize", "host_checks.cpp"), str(tmp_path / "host_checks.o")))
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        list(ex.map(lambda j: _run([HIPCC] + FLAGS + ["-c", j[0], "-o", j[1]]), jobs))
    objs = [j[1] for j in jobs]
    nm = subprocess.run(["nm"] + objs, capture_output=True, text=True, check=True).stdout
    syms = sorted(set(re.findall(r" U (__hip_fatbin_\w+)", nm)))
    bundle = ",".join(str(b) for b in b"__CLANG_OFFLOAD_BUNDLE__" + bytes(8))   # no entries
    stub = tmp_path / "images.cpp"
    stub.write_text("".join(f'extern "C" __attribute__((aligned(4096))) const unsigned char {s}[32] = {{{bundle}}};\n'
                            for s in syms))
    _run(["g++", "-c", str(stub), "-o", str(tmp_path / "images.o")])
    exe = str(tmp_path / "host_checks")
    _run([HIPCC, "--offload-host-only"] + SAN + ["-o", exe]
         + objs + [str(tmp_path / "images.o")] + LIBS)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-6000:]
    assert "host checks passed" in r.stdout
