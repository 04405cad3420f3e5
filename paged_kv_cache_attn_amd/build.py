"""Build libpagedattn.so for gfx950 with hipcc (in-tree, no JIT cache).

    python -m paged_kv_cache_attn_amd.build [--debug | --timeline | --all]

Each .hip source is compiled to an object under _build/ (in parallel), then
linked into paged_kv_cache_attn_amd/libpagedattn.so.  The debug build
(PAGED_ATTN_DEBUG=1: the kernels also report what their bounds checks mask,
read with pa_debug_flags) goes to libpagedattn_debug.so, its objects under
_build/debug/.  The timestamp build (PAGED_ATTN_TIMELINE=1: the balanced
decode's planned kernels record per-workgroup timestamps, read with
pa_timeline) goes to libpagedattn_timeline.so, its objects under
_build/timeline/.  Always rebuilds.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpagedattn.so")
DEBUG_LIB = os.path.join(PKG, "libpagedattn_debug.so")
TIMELINE_LIB = os.path.join(PKG, "libpagedattn_timeline.so")
VARIANTS = {"release": ("", [], LIB), "debug": ("debug", ["-DPAGED_ATTN_DEBUG=1"], DEBUG_LIB),
            "timeline": ("timeline", ["-DPAGED_ATTN_TIMELINE=1"], TIMELINE_LIB)}
ARCH = "gfx950"

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

CFLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    # packed-fp32 VALU forms are left to no one: plain fp32 math only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # no NaN operands are ever formed on purpose (masked scores are -inf and
    # every -inf - -inf is guarded), so max/min need no NaN-quieting copies
    "-fno-honor-nans",
    "-Wall", "-I" + INCLUDE, "-I" + CSRC,
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str, variant: str = "release") -> str:
    sub, defs, _ = VARIANTS[variant]
    obj = os.path.join(BUILD, sub, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC] + CFLAGS + defs + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s" % (src, err))
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(verbose: bool = True, debug: bool = False, timeline: bool = False) -> str:
    """Compile and link the release library (or, with debug=True, the debug one; with timeline=True, the
    timestamp one); returns its path."""
    variant = "debug" if debug else "timeline" if timeline else "release"
    sub, _, lib = VARIANTS[variant]
    os.makedirs(os.path.join(BUILD, sub), exist_ok=True)
    srcs = sources()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda src: _compile(src, variant), srcs))
    tmp = lib + ".tmp%d" % os.getpid()
    # -z defs: a symbol the objects leave undefined (a kernel stub the host
    # pass did not emit, say) fails the link instead of the first dlopen
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-Wl,-z,defs", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, lib)
    if verbose:
        print("built", lib)
    return lib


if __name__ == "__main__":
    args = sys.argv[1:]
    if "--all" in args:
        build()
        build(debug=True)
        build(timeline=True)
    else:
        build(debug="--debug" in args, timeline="--timeline" in args)
