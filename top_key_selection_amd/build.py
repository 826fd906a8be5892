"""Build libtks.so (the gfx950 kernels + C ABI) in-tree with hipcc.

    python -m top_key_selection_amd.build

Each source is compiled to its own object (in parallel; every kernel is
launched from the file that defines it, so no relocatable device code is
needed), then the objects are linked into one shared library.

    python -m top_key_selection_amd.build --sanitize

builds the same library with AddressSanitizer and UndefinedBehaviorSanitizer
in the host code only (device code is compiled as usual) into
_build/san/libtks.so, for checking the host glue on the CPU; objects are
reused while their sources are unchanged.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libtks.so")
OBJ = os.path.join(ROOT, "_build", "tks")
SOURCES = ["api.hip", "score.hip", "fused.hip", "select.hip", "pool.hip", "append.hip",
           "gather.hip", "attend.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-command-line-argument",
    # no packed fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; drop that note
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    return r.returncode, out


SAN_DIR = os.path.join(ROOT, "_build", "san")
SAN_LIB = os.path.join(SAN_DIR, "libtks.so")
# host-side sanitizers only: every -fsanitize= follows -Xarch_host
SAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined"]


def _newer(obj, src):
    if not os.path.exists(obj):
        return False
    deps = [src] + [os.path.join(CSRC, h) for h in os.listdir(CSRC) if h.endswith(".hpp")] + \
        [os.path.join(ROOT, "include", "tks.h")]
    return all(os.path.getmtime(obj) >= os.path.getmtime(d) for d in deps)


def build(verbose: bool = False, sanitize: bool = False) -> str:
    obj_dir = SAN_DIR if sanitize else OBJ
    lib = SAN_LIB if sanitize else LIB
    flags = [f for f in FLAGS if f != "-O3"] + SAN_FLAGS if sanitize else FLAGS
    os.makedirs(obj_dir, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    objs = [os.path.join(obj_dir, s.replace(".hip", ".o")) for s in srcs]
    cmds = [[HIPCC] + flags + ["-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(srcs, objs)
            if not (sanitize and _newer(o, os.path.join(CSRC, s)))]
    if verbose:
        for c in cmds:
            print(" ".join(c), flush=True)
    jobs = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with ThreadPoolExecutor(jobs) as ex:
        res = list(ex.map(_run, cmds))
    for (rc, out), c in zip(res, cmds):
        if rc != 0:
            raise RuntimeError("hipcc failed on %s:\n%s" % (c[-3], out))
        if verbose and out.strip():
            print(out)
    tmp = lib + ".tmp%d" % os.getpid()
    link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"]
    if sanitize:
        link += ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-shared-libsan"]
    rc, out = _run(link + objs + ["-o", tmp])
    if rc != 0:
        raise RuntimeError("link failed:\n" + out)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
