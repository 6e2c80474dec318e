"""Build libtgemm.so in-tree with hipcc for gfx950 (ahead of time; no JIT).

Each translation unit (the host code, the attention kernel, and the kernel variants split
over several units) is compiled to an object in parallel, then hipcc links the shared
library."""
from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SRCS = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
LIB = os.path.join(PKG, "libtgemm.so")
OBJ_DIR = os.path.join(PKG, "_build")
INCLUDE = os.path.join(ROOT, "include")
ARCH = "gfx950"

# No packed-fp32 VALU instructions anywhere (-packed-fp32-ops): the host pass does not
# know the feature and warns, which is harmless.
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]
_NOISE = "is not a recognized feature for this target"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else (shutil.which("hipcc") or "hipcc")


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if _NOISE not in ln]
    return res.returncode, msgs


def build(extra_flags=(), out: str = LIB, quiet: bool = True, jobs: int = 0) -> str:
    """Compile every kernel and the C ABI into ``out`` (always recompiles)."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    jobs = jobs or min(len(SRCS), os.cpu_count() or 1)
    objs, cmds = [], []
    for src in SRCS:
        obj = os.path.join(OBJ_DIR, os.path.splitext(os.path.basename(src))[0] + ".o")
        objs.append(obj)
        cmds.append([hipcc(), *FLAGS, *extra_flags, f"-I{INCLUDE}", "-c", src, "-o", obj])
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(_run, cmds))
    msgs = []
    for cmd, (rc, m) in zip(cmds, results):
        if rc != 0:
            raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + "\n".join(m))
        msgs += m
    tmp = out + ".tmp"
    link = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    rc, m = _run(link)
    if rc != 0:
        raise RuntimeError("hipcc link failed:\n" + " ".join(link) + "\n" + "\n".join(m))
    msgs += m
    if msgs and not quiet:
        print("\n".join(msgs), file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(quiet=False))
