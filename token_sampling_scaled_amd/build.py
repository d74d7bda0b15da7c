"""Build libtssample.so and libtsprobe.so (gfx950) in-tree with hipcc.

    python -m token_sampling_scaled_amd.build          # compile every source
    python -m token_sampling_scaled_amd.build --stage-marks
        # also libtssample_marks.so: the sampler with stage marks in the
        # register-resident kernel (token_sampling_scaled_amd.stage_times)

Every HIP source is compiled for gfx950 only, with packed-fp32 instruction
generation switched off.  csrc/ (kernels and the C-ABI host code) links into
libtssample.so, the sampler; csrc_probe/ links into libtsprobe.so, the measurement
probes that the benchmark and the GPU tests use beside it.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
PROBE = os.path.join(PKG, "csrc_probe")
LIB = os.path.join(PKG, "libtssample.so")
PROBE_LIB = os.path.join(PKG, "libtsprobe.so")
MARKS_LIB = os.path.join(PKG, "libtssample_marks.so")

ARCH = "gfx950"
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libtssample.so")


def sources(folder: str = CSRC):
    return sorted(os.path.join(folder, f) for f in os.listdir(folder) if f.endswith((".hip", ".cpp")))


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile both libraries (every call compiles every source); returns the sampler's path."""
    _build_lib(sources(CSRC), LIB, verbose, jobs)
    _build_lib(sources(PROBE), PROBE_LIB, verbose, jobs)
    return LIB


def build_stage_marks(verbose: bool = False, jobs: int = 8) -> str:
    """The sampler with stage marks compiled in, beside the product library."""
    _build_lib(sources(CSRC), MARKS_LIB, verbose, jobs, defines=["-DTSS_STAGE_MARKS"])
    return MARKS_LIB


def _build_lib(srcs, lib_path: str, verbose: bool, jobs: int, defines=()) -> None:
    cc = hipcc()
    objdir = tempfile.mkdtemp(prefix="tssample_build_")
    try:
        procs = []
        objs = []
        for src in srcs:
            obj = os.path.join(objdir, os.path.basename(src) + ".o")
            objs.append(obj)
            cmd = [cc, *HIP_FLAGS, *defines, f"-I{INCLUDE}", f"-I{CSRC}", "-c", src, "-o", obj]
            if src.endswith(".cpp"):
                cmd[1:1] = ["-x", "hip"]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
            if len(procs) >= jobs:
                _wait(procs.pop(0))
        for p in procs:
            _wait(p)
        tmp = lib_path + ".tmp"
        link = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
        if verbose:
            print(" ".join(link), flush=True)
        subprocess.run(link, check=True)
        os.replace(tmp, lib_path)
    finally:
        shutil.rmtree(objdir, ignore_errors=True)


def _wait(item):
    src, proc = item
    out, _ = proc.communicate()
    if proc.returncode != 0:
        sys.stderr.write(out.decode(errors="replace"))
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)}")
    if out.strip():
        sys.stderr.write(out.decode(errors="replace"))


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    if "--stage-marks" in sys.argv:
        print(build_stage_marks(verbose="-v" in sys.argv))
