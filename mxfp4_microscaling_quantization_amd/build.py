"""Build the HIP library (libmx355.so) in-tree for gfx950 with hipcc.

    python -m mxfp4_microscaling_quantization_amd.build

Each .hip source compiles to an object under _build/ in parallel, then one
shared library is linked next to this file.  Compiles every time it is called.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
BUILD = ROOT / "_build"
LIB = PKG / "libmx355.so"
SOURCES = ["quant.hip", "gemm.hip", "linear.hip", "deosc.hip"]
# The synthetic optimizer step that drives the de-oscillation workload (a
# workload generator, not part of the method) lives in a library of its own.
SYNTH_LIB = PKG / "libmx355_synth.so"
SYNTH_SOURCES = ["synth_step.hip"]
ARCH = os.environ.get("MX_OFFLOAD_ARCH", "gfx950")

# -ffp-contract=off: the quantizer, Hadamard and de-oscillation arithmetic is
# defined operation by operation (bit-exact with a CPU replay), so no a*b+c may
# be fused.  Denormals are kept: scales reach 2^-127.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    f"-I{ROOT / 'include'}",
]


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer build of the same
# sources (device code untouched): the CPU ABI tests run the argument checks
# of every entry point against it.  It is loaded with the sanitizer runtime
# preloaded, never by the product path.
SAN_BUILD = BUILD / "san"
SAN_LIB = SAN_BUILD / "libmx355_san.so"
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def sanitizer_runtime() -> Path:
    """The clang AddressSanitizer runtime that a sanitized library needs preloaded."""
    res = subprocess.run([hipcc(), "-print-resource-dir"], capture_output=True, text=True)
    rt = Path(res.stdout.strip()) / "lib" / "linux" / "libclang_rt.asan-x86_64.so"
    if not rt.exists():
        raise RuntimeError(f"sanitizer runtime not found at {rt}")
    return rt


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the MXFP4 HIP library cannot be built")


def _compile(src: str, sanitize: bool = False) -> Path:
    out = SAN_BUILD if sanitize else BUILD
    obj = out / (Path(src).stem + ".o")
    cmd = [hipcc(), *HIP_FLAGS, *(SAN_FLAGS if sanitize else []), "-c", str(CSRC / src), "-o",
           str(obj)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    if res.stderr.strip():
        sys.stderr.write(res.stderr)
    return obj


def _link(objs, lib: Path, extra=()) -> None:
    tmp = lib.with_suffix(".so.tmp")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra, "-o", str(tmp),
           *map(str, objs)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, lib)


# Rate probes (stand-alone programs, not part of the library): the VALU issue
# rates weight the quantizers' instruction counts in the ALU roofline; the MFMA
# probe measures the FP4 matrix instruction's sustained rate on register data.
PROBE_NAMES = ("valu_rate_probe", "mfma_rate_probe")
PROBE = BUILD / "valu_rate_probe"


def build_probe(name: str = "valu_rate_probe") -> Path:
    BUILD.mkdir(exist_ok=True)
    src = ROOT / "tests" / f"{name}.hip"
    out = BUILD / name
    cmd = [hipcc(), *[f for f in HIP_FLAGS if not f.startswith("-I")], str(src), "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src.name}:\n{' '.join(cmd)}\n{res.stderr}")
    return out


def build(verbose: bool = True) -> Path:
    BUILD.mkdir(exist_ok=True)
    srcs = SOURCES + SYNTH_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs) + 2, os.cpu_count() or 4)) as ex:
        probes = [ex.submit(build_probe, n) for n in PROBE_NAMES]
        objs = list(ex.map(_compile, srcs))
        for f in probes:
            f.result()
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], SYNTH_LIB)
    if verbose:
        print(f"built {LIB}, {SYNTH_LIB.name} and the probes {', '.join(PROBE_NAMES)} in {BUILD}")
    return LIB


def build_sanitized(verbose: bool = True) -> Path:
    """The host-sanitized library (see SAN_FLAGS); the sanitizer runtime is not
    linked in and must be preloaded (sanitizer_runtime())."""
    SAN_BUILD.mkdir(parents=True, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda src: _compile(src, True), SOURCES))
    _link(objs, SAN_LIB, ["-shared-libsan"])
    if verbose:
        print(f"built {SAN_LIB}")
    return SAN_LIB


if __name__ == "__main__":
    build()
