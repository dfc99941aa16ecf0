"""Compile tests/c_abi/bevpool_example.c, a plain C99 consumer of the C ABI,
with gcc against include/bevpool.h and libbevpool.so.

    python tests/c_abi/build_example.py [output]
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "bevpool_example.c")
BIN = os.path.join(HERE, "bevpool_example")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(out: str = BIN, werror: bool = False) -> str:
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no C compiler found")
    pkg = os.path.join(ROOT, "depth_weighted_scatter_amd")
    rel = os.path.relpath(pkg, os.path.dirname(os.path.abspath(out)))
    cmd = [cc, "-std=c99", "-O2", "-Wall", "-Wextra", *(["-Werror"] if werror else []),
           "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", f"-I{os.path.join(ROOT, 'include')}",
           SRC, "-o", out, f"-L{pkg}", "-lbevpool", f"-L{ROCM}/lib", "-lamdhip64",
           f"-Wl,-rpath,$ORIGIN/{rel}", f"-Wl,-rpath,{ROCM}/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling the C example failed:\n{' '.join(cmd)}\n{r.stdout}{r.stderr}")
    return out


if __name__ == "__main__":
    print(build(sys.argv[1] if len(sys.argv) > 1 else BIN))
