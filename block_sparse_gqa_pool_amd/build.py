"""Build the gfx950 shared library ``libbsg.so`` in-tree with hipcc.

    python -m block_sparse_gqa_pool_amd.build [-v] [--debug] [--asan] [--all]

Every ``csrc/*.hip`` file is compiled to an object under ``_build/`` (in parallel) and
linked into ``block_sparse_gqa_pool_amd/libbsg.so``.  Packed fp32 VALU instructions are
disabled for device code.  Two more variants, each in its own object folder:

* ``--debug``: ``libbsg_debug.so`` with ``-DBSG_DEBUG`` (kernels record the table ids they
  clamp; ``bsg_debug_errors`` reads them back);
* ``--asan``: ``libbsg_asan.so``, the host code built with AddressSanitizer (device code as
  usual), for the host-side argument checks of the C layer on a machine without a GPU.  Load
  it with the sanitizer runtime preloaded (``asan_runtime()``).
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shlex
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libbsg.so")
ARCH = os.environ.get("BSG_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC,
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{msg}")
    if verbose and msg.strip():
        print(msg)


# variant: (library file, object folder, extra compile flags, extra link flags)
VARIANTS = {
    "release": ("libbsg.so", "_build", [], []),
    "debug": ("libbsg_debug.so", "_build_debug", ["-DBSG_DEBUG"], []),
    "asan": ("libbsg_asan.so", "_build_asan",
             shlex.split("-Xarch_host -fsanitize=address -Xarch_host -fno-omit-frame-pointer"),
             shlex.split("-Xarch_host -fsanitize=address -shared-libasan")),
}


def lib_path(variant: str = "release") -> str:
    return os.path.join(PKG, VARIANTS[variant][0])


def source_hash() -> str:
    """Hash of the library's sources and headers (what a build was made from)."""
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(CSRC, "*")) + glob.glob(os.path.join(INCLUDE, "*.h"))):
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def is_stale(variant: str = "release") -> bool:
    """True when the variant's library is missing or was built from other sources (the hash
    written beside it at build time differs from the sources' hash now)."""
    lib = lib_path(variant)
    stamp = lib + ".srchash"
    if not (os.path.exists(lib) and os.path.exists(stamp)):
        return True
    with open(stamp) as fh:
        return fh.read().strip() != source_hash()


def asan_runtime() -> str:
    """The AddressSanitizer runtime of the ROCm clang that builds the asan variant."""
    import glob as _glob
    hits = sorted(_glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("no libclang_rt.asan-x86_64.so under /opt/rocm/llvm/lib/clang")
    return hits[-1]


def build(verbose: bool = False, jobs: int = 8, variant: str = "release") -> str:
    libname, objdir, cflags, lflags = VARIANTS[variant]
    out_dir = os.path.join(PKG, objdir)
    lib = os.path.join(PKG, libname)
    os.makedirs(out_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(out_dir, os.path.basename(s) + ".o") for s in srcs]
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        futs = [ex.submit(_run, [HIPCC, *FLAGS, *cflags, "-c", s, "-o", o], verbose) for s, o in zip(srcs, objs)]
        for f in futs:
            f.result()
    tmp = lib + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *lflags, *objs, "-o", tmp], verbose)
    os.replace(tmp, lib)
    with open(lib + ".srchash", "w") as fh:
        fh.write(source_hash() + "\n")
    return lib


if __name__ == "__main__":
    v = "-v" in sys.argv
    chosen = [k for k, flag in (("debug", "--debug"), ("asan", "--asan")) if flag in sys.argv or "--all" in sys.argv]
    if "--all" in sys.argv or not chosen:
        chosen = ["release"] + chosen
    for var in chosen:
        print(build(verbose=v, variant=var))
