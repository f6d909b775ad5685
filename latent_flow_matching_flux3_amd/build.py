"""Build libflux3_dit.so (gfx950) in-tree with hipcc.

    python -m latent_flow_matching_flux3_amd.build [--jobs N] [--verbose]

Every .hip file under csrc/ is compiled to an object in _build/ (parallel
hipcc processes), then linked into latent_flow_matching_flux3_amd/libflux3_dit.so;
probe/probe.hip (the measurement harness's peak probes) becomes
latent_flow_matching_flux3_amd/libflux3_probe.so.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libflux3_dit.so")
ARCH = "gfx950"

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # packed fp32 VALU forms stay off; ordinary float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


# Per-file code-generation options.  attention.hip keeps every MFMA
# accumulator in ordinary VGPRs (its softmax reads the score accumulators
# with VALU instructions; with AGPR accumulators the compiler shuttles them
# through v_accvgpr_read/write on every tile).
FILE_FLAGS = {
    "attention.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *COMMON_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    if out and verbose:
        print(out, flush=True)
    return obj


PROBE_SRC = os.path.join(PKG, "probe", "probe.hip")
PROBE_LIB = os.path.join(PKG, "libflux3_probe.so")


def build_probe(verbose: bool = False) -> str:
    """The peak probes of the measurement harness (MFMA and HBM copy), a
    library of their own next to libflux3_dit.so."""
    tmp = PROBE_LIB + ".tmp"
    cmd = [HIPCC, *COMMON_FLAGS, "-shared", PROBE_SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {PROBE_SRC}:\n{r.stdout}{r.stderr}")
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


def build(jobs: int | None = None, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), os.cpu_count() or 4, 16)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        probe = ex.submit(build_probe, verbose)
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
        probe.result()
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--verbose", action="store_true")
    a = ap.parse_args(argv)
    print(build(a.jobs, a.verbose))


if __name__ == "__main__":
    sys.exit(main())
