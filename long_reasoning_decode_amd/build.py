"""Build step for the HIP library: compiles csrc/*.hip for gfx950 with hipcc
into long_reasoning_decode_amd/libtriattn.so (in-tree, so it travels with the
source tree).  Run `python -m long_reasoning_decode_amd.build`."""
from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libtriattn.so")
SOURCES = ["api.hip", "score.hip", "select.hip", "decode.hip", "calib.hip"]
ARCH = os.environ.get("TRIATTN_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed-FP32 VALU forms stay off: every fp32 op is issued unpacked
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)

    def compile_one(src):
        out = os.path.join(OBJ, src.replace(".hip", ".o"))
        cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0 or verbose:
            msg = r.stderr.strip()
            if r.returncode != 0:
                raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
            if msg:
                print(msg)
        return out

    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
