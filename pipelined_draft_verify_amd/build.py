"""Build libspd.so (HIP, gfx950) in-tree with hipcc.

The library links against the HIP runtime with soname libamdhip64.so.7 and
carries an rpath to torch's bundled runtime, so a process that imported
torch first uses the one runtime torch already loaded.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libspd.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # packed fp32 instructions stay off: plain fp32 VALU ops only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden",
    "-Wall",
    "-Wno-unused-function",
    "-Wno-unused-variable",
    "-Wno-unused-but-set-variable",
]


def _torch_lib_dir():
    try:
        import importlib.util
        spec = importlib.util.find_spec("torch")
        if spec and spec.origin:
            return os.path.join(os.path.dirname(spec.origin), "lib")
    except Exception:
        pass
    return None


def build(verbose: bool = False) -> str:
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    cmd = [HIPCC] + FLAGS + ["-I", INCLUDE, "-I", CSRC] + srcs + ["-o", LIB + ".tmp"]
    tl = _torch_lib_dir()
    if tl:
        cmd += [f"-Wl,-rpath,{tl}"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libspd.so")
    if verbose and r.stderr.strip():
        # the host pass does not know the packed-fp32 target feature: harmless
        lines = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l]
        if lines:
            sys.stderr.write("\n".join(lines) + "\n")
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
