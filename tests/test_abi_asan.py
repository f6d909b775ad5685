"""The C ABI's host-side argument checks under AddressSanitizer.

Builds the library with its host code instrumented (hipcc, the sanitizer on
the host side only; device code is compiled as usual) into _build/asan/,
links tests/asan/abi_checks.c against it with the sanitizer runtime, and runs
it: every status code must be the expected one, and no invalid host access
may occur (ASan aborts the process).  No GPU is needed: no case reaches a HIP
call."""
import concurrent.futures as cf
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "latent_flow_matching_flux3_amd", "csrc")
OUT = os.path.join(ROOT, "_build", "asan")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
HOST_ASAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}{r.stderr}"


@pytest.mark.timeout(900)
def test_abi_argument_checks_under_asan():
    if not os.path.exists(CLANG) or not os.path.exists(HIPCC):
        pytest.skip("ROCm clang/hipcc not installed")
    os.makedirs(OUT, exist_ok=True)
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Xclang", "-target-feature",
             "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), *HOST_ASAN]
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))

    def compile_one(f):
        obj = os.path.join(OUT, f[:-4] + ".o")
        _run([HIPCC, *flags, "-c", os.path.join(CSRC, f), "-o", obj])
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 4)) as ex:
        objs = list(ex.map(compile_one, srcs))
    lib = os.path.join(OUT, "libflux3_dit_asan.so")
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *HOST_ASAN, "-o", lib, *objs])
    exe = os.path.join(OUT, "abi_checks")
    _run([CLANG, "-fsanitize=address", "-fno-omit-frame-pointer", "-g", "-I", os.path.join(ROOT, "include"),
          "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include", os.path.join(ROOT, "tests", "asan", "abi_checks.c"),
          lib, f"-Wl,-rpath,{OUT}", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and "all passed" in r.stdout, r.stdout + r.stderr
    assert "AddressSanitizer" not in r.stderr, r.stderr
