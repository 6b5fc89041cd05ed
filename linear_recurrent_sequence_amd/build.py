"""Build libretention.so (HIP, gfx950) in-tree with hipcc: one object per kernel-group source, compiled in
parallel, then linked into a shared library next to this file."""
from __future__ import annotations

import glob
import hashlib
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_PATH = os.path.join(PKG, "libretention.so")
OBJ_DIR = os.path.join(PKG, "_build")
ARCH = os.environ.get("RET_OFFLOAD_ARCH", "gfx950")

COMMON = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    # packed fp32 ops stay off: hipcc -O3 would otherwise form them from plain float code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the kernels' atomics are issued by one lane on purpose; the atomic optimizer would turn each into a
    # wave-level scan whose result is needed at once, which puts a wait for every earlier load right behind it
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-Wall", "-Wno-unused-function", "-Wno-unused-result",
]
# per-source additions: the wide-head kernel keeps its MFMA accumulators in architectural registers
EXTRA = {"chunk_wide.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
NOISE = "'-packed-fp32-ops' is not a recognized feature"


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if NOISE not in l)
    return r.returncode, err


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def source_digest() -> str:
    """Digest of every source the library is built from (kernels, host code, the public header). The library
    carries the digest of the sources it was built from (ret_source_digest), so a stale build is detected."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.h")) +
                   glob.glob(os.path.join(ROOT, "include", "*.h")))
    for f in files:
        with open(f, "rb") as fh:
            h.update(os.path.relpath(f, ROOT).encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def build(verbose: bool = False, jobs: int | None = None) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC, '-DRET_SOURCE_DIGEST="%s"' % source_digest()]
    objs, cmds = [], []
    for src in sources():
        obj = os.path.join(OBJ_DIR, os.path.basename(src)[:-4] + ".o")
        objs.append(obj)
        cmds.append(["hipcc"] + COMMON + EXTRA.get(os.path.basename(src), []) + inc + ["-c", src, "-o", obj])
    jobs = jobs or min(len(cmds), max(1, min(16, os.cpu_count() or 1)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(_run, cmds))
    failed = [(c, e) for c, (rc, e) in zip(cmds, results) if rc != 0]
    if failed:
        raise RuntimeError("hipcc failed:\n" + "\n\n".join(" ".join(c) + "\n" + e for c, e in failed))
    if verbose:
        for (rc, e) in results:
            if e.strip():
                print(e, file=sys.stderr)
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    rc, err = _run(["hipcc", "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs)
    if rc != 0:
        raise RuntimeError("link failed:\n" + err)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
