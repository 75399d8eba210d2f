"""Build the HIP attention library (libeiat_attn.so) in-tree for gfx950.

Every build compiles each HIP source with hipcc for gfx950 and links them into
one shared library next to this file.  The library exports only the C ABI of
include/eiat_attn.h.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libeiat_attn.so")
SOURCES = ["attn_api.hip", "attn_fwd.hip", "attn_bwd.hip", "attn_bwd_dq.hip", "attn_decode.hip",
           "attn_fp8.hip"]
# Machine-scheduler strategy per source, chosen by timing each kernel file's
# kernels under the strategies LLVM offers for AMDGPU: max-ilp for the forward
# (its exp/MFMA interleave) and for delta and dK/dV (1-4 % faster than under
# max-memory-clause).  The dQ kernel, compiled in its own unit, keeps LLVM's
# default strategy: 1-5 % faster than under max-ilp at n = 4096 causal (d = 64
# and 128), 1 % slower at d = 128 without mask, n = 16384.
PER_SOURCE_FLAGS = {
    "attn_fwd.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"],
    "attn_bwd.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"],
}
ARCH = os.environ.get("EIAT_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

CFLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-fPIC",
    "-std=c++17",
    "-fvisibility=hidden",
    # packed fp32 VALU forms are kept out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: the kernels rescale and read them with VALU
    # every tile, which AGPR accumulators would turn into copy traffic
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    f"-I{os.path.join(ROOT, 'include')}",
]


# Check builds, used only by tests (tests/test_check_builds_gpu.py): the same
# ABI compiled with a macro of csrc/attn_device.h into a library of its own.
# Each recompiles the sources that the macro changes and links the rest of the
# product build's objects.
#   libeiat_attn_poison.so  EIAT_LDS_POISON: every direct HBM -> LDS load
#                           first fills its destination with NaN
#   libeiat_attn_alt.so     EIAT_ALT_TILES: other tile shapes
CHECK_BUILDS = {
    "poison": (["-DEIAT_LDS_POISON"],
               ["attn_fwd.hip", "attn_bwd.hip", "attn_bwd_dq.hip", "attn_decode.hip"]),
    "alt": (["-DEIAT_ALT_TILES"], ["attn_fwd.hip", "attn_bwd.hip", "attn_bwd_dq.hip"]),
}


def check_lib_path(name: str) -> str:
    return os.path.join(HERE, f"libeiat_attn_{name}.so")


def _compile(src: str, extra: list[str], objdir: str = OBJ) -> str:
    obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, *PER_SOURCE_FLAGS.get(src, []), *extra, "-c", os.path.join(CSRC, src),
           "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def _link(objs: list[str], lib: str):
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs,
           "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False, extra: list[str] | None = None, checks: bool = True) -> str:
    """Compile the product library (and, with `checks`, the check builds) for gfx950."""
    os.makedirs(OBJ, exist_ok=True)
    extra = list(extra or [])
    jobs = [(src, extra, OBJ) for src in SOURCES]
    if checks:
        for name, (flags, srcs) in CHECK_BUILDS.items():
            d = os.path.join(OBJ, name)
            os.makedirs(d, exist_ok=True)
            jobs += [(src, extra + flags, d) for src in srcs]
    # the forward units (the slowest) first
    jobs.sort(key=lambda j: j[0] != "attn_fwd.hip")
    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    base = {src: os.path.join(OBJ, os.path.splitext(src)[0] + ".o") for src in SOURCES}
    _link([base[s] for s in SOURCES], LIB)
    if verbose:
        print(f"built {LIB}", file=sys.stderr)
    if checks:
        for name, (_, srcs) in CHECK_BUILDS.items():
            d = os.path.join(OBJ, name)
            objs = [os.path.join(d, os.path.splitext(s)[0] + ".o") if s in srcs else base[s]
                    for s in SOURCES]
            _link(objs, check_lib_path(name))
            if verbose:
                print(f"built {check_lib_path(name)}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
