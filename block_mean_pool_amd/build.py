"""Builds the HIP library libsparse_attn.so in-tree for gfx950.

    python block_mean_pool_amd/build.py   (run by path: importing the
                                          package loads the built library)

Every .hip file under csrc/ is compiled with hipcc for gfx950 and linked
into one shared library next to this file; the benchmark's measurement
helpers (probe/ beside bench.py) go into a library of their own
(probe/libsa_probe.so), so the attention library's ABI holds only the
method.  Packed-fp32 VALU
instructions are disabled for all device code.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsparse_attn.so")
# the benchmark's measurement helpers live beside bench.py, not in the package
PROBE_DIR = os.path.join(os.path.dirname(HERE), "probe")
PROBE_LIB = os.path.join(PROBE_DIR, "libsa_probe.so")
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics",
]


# The pipelined forward kernels interleave, in one region per tile, MFMAs
# with the exp2/pack work of the softmax; the two branches of that region
# (with and without the previous tile's P.V) share the softmax code, and
# LLVM's machine CSE and SimplifyCFG would hoist that shared code out of both
# branches into a VALU-only block ahead of the MFMAs.  Keeping it in place
# measured 3 % (video) to 8 % (causal LM) faster on gfx950.
PER_FILE_FLAGS = {
    name: ["-mllvm", "-disable-machine-cse",
           "-mllvm", "-simplifycfg-sink-common=false",
           "-mllvm", "-simplifycfg-hoist-common=false"]
    for name in ("attn_pipe.hip", "attn_q.hip")
}


# The host-sanitizer build: the same library with AddressSanitizer and
# UndefinedBehaviorSanitizer on the host code only (each -fsanitize flag is
# scoped to the host pass; device code is built as usual), for the CPU tests
# of the C ABI's host layer.  It needs the compiler's ASan runtime preloaded
# (asan_runtime()) when loaded into an uninstrumented process.
SAN_LIB = os.path.join(HERE, "libsparse_attn_san.so")
SAN_FLAGS = ["-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]
SAN_LINK = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-shared-libsan"]


def asan_runtime() -> str:
    """Path of the compiler's shared ASan runtime (to preload)."""
    import glob
    root = os.path.join(os.path.dirname(os.path.dirname(HIPCC)), "lib", "llvm", "lib", "clang")
    hits = sorted(glob.glob(os.path.join(root, "*", "lib", "linux", "libclang_rt.asan-x86_64.so")))
    if not hits:
        raise FileNotFoundError(f"no libclang_rt.asan-x86_64.so under {root}")
    return hits[-1]


def build_sanitized(verbose: bool = False, jobs: int = 8) -> str:
    """Builds SAN_LIB (host code under ASan + UBSan).  Returns its path."""
    _build_lib(sources(CSRC), SAN_LIB, verbose, jobs, extra=SAN_FLAGS, link_extra=SAN_LINK)
    return SAN_LIB


def sources(folder=CSRC):
    return sorted(os.path.join(folder, f) for f in os.listdir(folder) if f.endswith(".hip"))


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Builds LIB and PROBE_LIB.  Returns LIB's path."""
    _build_lib(sources(CSRC), LIB, verbose, jobs)
    _build_lib(sources(PROBE_DIR), PROBE_LIB, verbose, jobs)
    return LIB


def _build_lib(srcs, lib, verbose, jobs, extra=(), link_extra=()):
    """Compiles srcs (in parallel) and links them into lib."""
    objdir = tempfile.mkdtemp(prefix="sa_build_")
    try:
        procs, objs = [], []
        for src in srcs:
            obj = os.path.join(objdir, os.path.basename(src) + ".o")
            cmd = [HIPCC, *FLAGS, *PER_FILE_FLAGS.get(os.path.basename(src), []), *extra, "-c",
                   src, "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                stderr=subprocess.STDOUT, text=True)))
            objs.append(obj)
            if len(procs) >= jobs:
                _wait(procs.pop(0))
        for p in procs:
            _wait(p)
        tmp = lib + ".tmp"
        cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *link_extra, "-o", tmp, *objs]
        if verbose:
            print(" ".join(cmd), flush=True)
        out = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        if out.returncode:
            raise RuntimeError("link failed:\n" + out.stdout)
        os.replace(tmp, lib)
    finally:
        shutil.rmtree(objdir, ignore_errors=True)


def _wait(item):
    src, p = item
    out, _ = p.communicate()
    if p.returncode:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    # keep real warnings visible, drop the host pass's note about the
    # device-only target feature
    lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if lines:
        print("\n".join(lines), file=sys.stderr)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
