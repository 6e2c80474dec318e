"""Build libtgemm.so in-tree with hipcc for gfx950 (ahead of time; no JIT)."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRCS = [os.path.join(PKG, "csrc", f) for f in ("tgemm.hip", "attention.hip")]
LIB = os.path.join(PKG, "libtgemm.so")
INCLUDE = os.path.join(ROOT, "include")
ARCH = "gfx950"

# No packed-fp32 VALU instructions anywhere (-packed-fp32-ops): the host pass does not
# know the feature and warns, which is harmless.
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else (shutil.which("hipcc") or "hipcc")


def build(extra_flags=(), out: str = LIB, quiet: bool = True) -> str:
    """Compile every kernel and the C ABI into ``out`` (always recompiles)."""
    tmp = out + ".tmp"
    cmd = [hipcc(), *FLAGS, *extra_flags, f"-I{INCLUDE}", *SRCS, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + "\n".join(msgs))
    if msgs and not quiet:
        print("\n".join(msgs), file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(quiet=False))
