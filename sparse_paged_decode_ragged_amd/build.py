"""Build libspd.so (HIP, gfx950) in-tree with hipcc, and beside it
libspd_probe.so (the benchmark's measurement kernels, include/spd_probe.h).

Every call compiles from source (the build check must really build); the
objects are compiled in parallel and linked into
``sparse_paged_decode_ragged_amd/_lib/``.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(PKG, "_lib")
LIB = os.path.join(OUT_DIR, "libspd.so")
PROBE_LIB = os.path.join(OUT_DIR, "libspd_probe.so")
PROBE_SOURCES = ["probe.hip"]
SOURCES = ["api.hip", "attn.hip", "attn_split.hip", "attn_fp8.hip", "indices.hip", "producer.hip",
           "noalloc.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "--offload-arch=" + ARCH,
    # packed fp32 VALU ops are disabled for all device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
]


# Host code only: AddressSanitizer + UndefinedBehaviorSanitizer for the CPU
# side of the library (argument checks, planning, launch set-up); device code
# is built as usual.
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
                  "-Xarch_host", "-g"]


def _compile(src: str, obj_dir: str, extra=()) -> str:
    obj = os.path.join(obj_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l and "(ignoring feature)" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, msgs))
    if msgs.strip():
        sys.stderr.write(msgs + "\n")
    return obj


def _link(objs, lib: str, extra=()) -> None:
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", *extra, "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, lib)


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Build both libraries into _lib/ (sanitize: host-sanitized copies into
    _lib/sanitize/, for the CPU tests run under AddressSanitizer)."""
    out_dir = os.path.join(OUT_DIR, "sanitize") if sanitize else OUT_DIR
    obj_dir = os.path.join(out_dir, "obj")
    os.makedirs(obj_dir, exist_ok=True)
    extra = SANITIZE_FLAGS if sanitize else []
    # the sanitizer runtime is not linked in: the process preloads it (the
    # instrumented objects' runtime references resolve against it at load)
    link_extra = []
    srcs = SOURCES + PROBE_SOURCES
    with ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, obj_dir, extra), srcs))
    lib = os.path.join(out_dir, "libspd.so")
    probe = os.path.join(out_dir, "libspd_probe.so")
    _link(objs[:len(SOURCES)], lib, link_extra)
    _link(objs[len(SOURCES):], probe, link_extra)
    if verbose:
        print("built", lib, "and", probe)
    return lib


if __name__ == "__main__":
    build(verbose=True, sanitize="--sanitize" in sys.argv[1:])
