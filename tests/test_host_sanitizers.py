"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

capi.hip and timing.hip (argument validation, size queries, workspace carving, the timing
table) are compiled with the sanitizers on their host side, linked with the kernel objects of
the regular build into a separate library, and driven by tests/host_sanitizer_driver.cpp,
itself built with the sanitizers: tens of thousands of calls with extreme and inconsistent
sizes, NULL, misaligned and overlapping pointers and undersized workspaces. The driver runs
where no GPU is visible, so every call stops at validation or at the device check; any
out-of-bounds access, signed overflow or other undefined behaviour aborts it with a report.
"""
import os
import shutil
import subprocess

import pytest
import torch

from linear_cross_entropy_masked_amd import build as lce_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "linear_cross_entropy_masked_amd", "csrc")
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd, sanitized_program=False):
    env = None
    if sanitized_program:  # the driver: no leak check (the HIP runtime keeps its allocations)
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, env=env,
                       timeout=600)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}"
    return r.stdout


@pytest.mark.timeout(900)
def test_c_abi_host_code_under_asan_and_ubsan(tmp_path):
    if torch.cuda.is_available():
        pytest.skip("runs where no GPU is visible (valid calls would reach the kernels)")
    hipcc = lce_build.hipcc()
    clangxx = os.path.join(os.path.dirname(os.path.realpath(hipcc)), "..", "llvm", "bin", "clang++")
    if not os.path.exists(clangxx):
        clangxx = shutil.which("clang++") or "/opt/rocm/llvm/bin/clang++"
    # kernel objects of the regular build (built if missing); host code rebuilt with sanitizers
    objs = {s: os.path.join(lce_build.BUILD_DIR, s.replace(".hip", ".o")) for s in lce_build.SOURCES}
    if not all(os.path.exists(o) for o in objs.values()):
        lce_build.build()
    common = [f"--offload-arch={lce_build.ARCH}", "-O1", "-std=c++17", "-fPIC", "-g",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    san_objs = []
    for src in ("capi.hip", "timing.hip"):
        out = str(tmp_path / src.replace(".hip", "_san.o"))
        _run([hipcc, *common, *HOST_SAN, "-c", os.path.join(CSRC, src), "-o", out])
        san_objs.append(out)
    kernels = [objs[s] for s in lce_build.SOURCES if s not in ("capi.hip", "timing.hip")]
    lib = str(tmp_path / "liblce_masked_san.so")
    _run([hipcc, f"--offload-arch={lce_build.ARCH}", "-shared", "-fPIC", *san_objs, *kernels,
          *HOST_SAN, "-o", lib])
    exe = str(tmp_path / "host_sanitizer_driver")
    rocm_lib = os.path.join(os.path.dirname(os.path.realpath(hipcc)), "..", "lib")
    _run([clangxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
          "-I", os.path.join(ROOT, "include"),
          os.path.join(ROOT, "tests", "host_sanitizer_driver.cpp"), lib,
          f"-Wl,-rpath,{tmp_path}", f"-L{rocm_lib}", "-lamdhip64", f"-Wl,-rpath,{rocm_lib}",
          "-o", exe])
    out = _run([exe], sanitized_program=True)
    print(out.strip().splitlines()[-1])
    assert "0 failures" in out or "skipped" in out
