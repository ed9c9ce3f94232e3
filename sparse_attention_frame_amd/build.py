"""Build libsfa.so (host planner + gfx950 kernels + C ABI) and libsfa_probe.so (the
matrix-core microbenchmarks the benchmark compares against) with hipcc, in-tree."""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libsfa.so")
PROBE_LIB = os.path.join(PKG, "libsfa_probe.so")
OBJ_DIR = os.path.join(PKG, "_build")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # keep the compiler away from packed-fp32 VALU forms
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]

# Per-source additions to HIPCC_FLAGS (none at present).
EXTRA_FLAGS: dict = {}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the sfa library needs ROCm's hipcc to build")


def sources():
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def probe_sources():
    return sorted(glob.glob(os.path.join(PKG, "csrc", "probe", "*.hip")))


# the host pass warns that it does not know the packed-fp32 feature: harmless
_NOISE = "is not a recognized feature for this target"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(ln for ln in res.stderr.splitlines() if _NOISE not in ln)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = False) -> str:
    """Compile every source into sparse_attention_frame_amd/libsfa.so and the probes into
    libsfa_probe.so (always rebuilds). Returns the path of libsfa.so."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc")]
    targets = {LIB: [], PROBE_LIB: []}
    jobs = []
    for lib, srcs in ((LIB, sources()), (PROBE_LIB, probe_sources())):
        for src in srcs:
            name = os.path.basename(src)
            obj = os.path.join(OBJ_DIR, name + ".o")
            targets[lib].append(obj)
            jobs.append([hipcc(), *HIPCC_FLAGS, *EXTRA_FLAGS.get(name, []), *inc, "-c", src,
                         "-o", obj])
    workers = max(1, min(len(jobs), os.cpu_count() or 1, 16))
    with ThreadPoolExecutor(workers) as ex:
        for f in [ex.submit(_run, cmd, verbose) for cmd in jobs]:
            f.result()
    for lib, objs in targets.items():
        tmp = lib + ".tmp"
        _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
        os.replace(tmp, lib)
    return LIB


SAN_DIR = os.path.join(OBJ_DIR, "san")
SAN_LIB = os.path.join(SAN_DIR, "libsfa_san.so")
# host code under AddressSanitizer and UndefinedBehaviorSanitizer (each -fsanitize= goes to
# the host pass only); the device code is built as usual, at -O1 to build quickly
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-g", "-fno-omit-frame-pointer"]


def asan_runtime() -> str:
    """The shared ASan runtime of hipcc's clang (preloaded into the Python process that
    loads the sanitizer build)."""
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm", "bin", "clang")
    res = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True, check=True)
    path = res.stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("the clang ASan runtime was not found")
    return path


def build_sanitized(verbose: bool = False) -> str:
    """Build the library with the host code (planner, validation, C ABI) instrumented by
    ASan and UBSan into _build/san/libsfa_san.so, for the CPU tests; not for GPU runs."""
    os.makedirs(SAN_DIR, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc")]
    flags = [f if f != "-O3" else "-O1" for f in HIPCC_FLAGS] + SAN_FLAGS
    objs, jobs = [], []
    for src in sources():
        obj = os.path.join(SAN_DIR, os.path.basename(src) + ".o")
        objs.append(obj)
        jobs.append([hipcc(), *flags, *inc, "-c", src, "-o", obj])
    workers = max(1, min(len(jobs), os.cpu_count() or 1, 16))
    with ThreadPoolExecutor(workers) as ex:
        for f in [ex.submit(_run, cmd, verbose) for cmd in jobs]:
            f.result()
    tmp = SAN_LIB + ".tmp"
    _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
          "-Xarch_host", "-fsanitize=undefined", *objs, "-o", tmp], verbose)
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


if __name__ == "__main__":
    print(build(verbose=True))
