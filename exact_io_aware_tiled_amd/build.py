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
# kernels under the strategies LLVM offers for AMDGPU (A/B on MI355X, page and
# training shapes): max-ilp for delta and dK/dV (LLVM's default is 3 % slower
# at d = 128, max-memory-clause 2 % slower at d = 64) and for dQ (1.3-1.6 %
# faster than the default at d = 128, equal at d = 64); the forward measures
# the same under max-ilp and the default (its inner region carries its own
# scheduling hint) and keeps max-ilp.
PER_SOURCE_FLAGS = {
    "attn_fwd.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"],
    "attn_bwd.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"],
    "attn_bwd_dq.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"],
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
#   libeiat_attn_timing.so  EIAT_WG_TIMING: per-workgroup start / prologue / end
#                           stamps of the forward, dQ and dK/dV (eiat_wg_times,
#                           eiat_wg_times_dq, eiat_wg_times_dkdv; wg_timeline.py)
CHECK_BUILDS = {
    "poison": (["-DEIAT_LDS_POISON"],
               ["attn_fwd.hip", "attn_bwd.hip", "attn_bwd_dq.hip", "attn_decode.hip"]),
    "alt": (["-DEIAT_ALT_TILES"], ["attn_fwd.hip", "attn_bwd.hip", "attn_bwd_dq.hip"]),
    "timing": (["-DEIAT_WG_TIMING"], ["attn_fwd.hip", "attn_bwd.hip", "attn_bwd_dq.hip"]),
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


def resource_report(out_path: str) -> str:
    """Per-kernel register, scratch, LDS and occupancy figures of the product
    build, from the compiler's resource-usage remarks (a CPU-side compile with
    -Rpass-analysis=kernel-resource-usage; nothing is linked or run)."""
    import re
    import tempfile

    rows = []
    with tempfile.TemporaryDirectory() as tmp:
        def one(src):
            cmd = [HIPCC, *CFLAGS, *PER_SOURCE_FLAGS.get(src, []),
                   "-Rpass-analysis=kernel-resource-usage", "-c", os.path.join(CSRC, src),
                   "-o", os.path.join(tmp, src + ".o")]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
            return src, r.stderr
        with cf.ThreadPoolExecutor(max_workers=8) as ex:
            outs = list(ex.map(one, SOURCES))
    for src, text in outs:
        cur = None
        for line in text.splitlines():
            m = re.search(r"remark: Function Name: (\S+)", line)
            if m:
                cur = {"src": src, "name": m.group(1)}
                rows.append(cur)
                continue
            m = re.search(r"remark:\s+([A-Za-z][A-Za-z \[\]/]*): (\S+) \[", line)
            if m and cur is not None:
                cur[m.group(1).strip()] = m.group(2)
    def short(mangled):
        # eiat::<kernel><template args>: the kernels' mangled names are all of
        # the form _ZN4eiat<len><name>I<args>E...
        m = re.match(r"_ZN4eiat(\d+)", mangled)
        if not m:
            return mangled
        k = int(m.group(1))
        name = mangled[m.end():m.end() + k]
        rest = mangled[m.end() + k:]
        args = []
        if rest.startswith("I"):
            body = rest[1:]
            while body and body[0] != "E":
                for pat, val in ((r"DF16b", "bf16"), (r"DF16_", "f16"), (r"f", "f32"),
                                 (r"Lb([01])E", None), (r"Li(-?\d+)E", None)):
                    mm = re.match(pat, body)
                    if mm:
                        args.append(val if val else mm.group(1))
                        body = body[mm.end():]
                        break
                else:
                    break
        return f"{name}<{','.join(args)}>"

    lines = [
        "# Kernel resources of the product build (compiler remarks, gfx950)",
        "",
        "command (from the repository root, on any machine with ROCm; compiles, runs nothing):",
        f"    python exact_io_aware_tiled_amd/build.py --resources {os.path.relpath(out_path, ROOT)}",
        "",
        "Per kernel: VGPRs / AGPRs / SGPRs allocated, VGPR and SGPR spills, scratch bytes per",
        "lane, the occupancy the registers allow (waves per SIMD) and the static LDS per",
        "workgroup.  LDS also bounds occupancy: 160 KiB per CU, so a 4-wave workgroup of L bytes",
        "runs floor(163840 / L) workgroups (waves per SIMD) per CU.",
        "",
        "Template arguments: element type, d, mask (0 none, 1 causal, 2 window), then",
        "dropout (0/1) and, for the forward, the FP8 mode (0 none, 1 scores, 2 scores and values).",
        "",
        f"{'kernel':<44} {'vgpr':>4} {'agpr':>4} {'sgpr':>4} {'spV':>3} {'spS':>3} "
        f"{'scr':>4} {'occ':>3} {'lds':>6}",
    ]
    for r in rows:
        d = short(r["name"])
        lines.append(f"{d:<44} {r.get('VGPRs', '?'):>4} {r.get('AGPRs', '?'):>4} "
                     f"{r.get('TotalSGPRs', '?'):>4} {r.get('VGPRs Spill', '?'):>3} "
                     f"{r.get('SGPRs Spill', '?'):>3} {r.get('ScratchSize [bytes/lane]', '?'):>4} "
                     f"{r.get('Occupancy [waves/SIMD]', '?'):>3} "
                     f"{r.get('LDS Size [bytes/block]', '?'):>6}")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return out_path


if __name__ == "__main__":
    if len(sys.argv) > 2 and sys.argv[1] == "--resources":
        print(resource_report(os.path.abspath(sys.argv[2])))
    else:
        build(verbose=True, extra=sys.argv[1:])
