"""Build the HIP libraries in-tree for gfx950.

    python sparse_key_value_amd/build.py

compiles every ``*.hip`` under ``sparse_key_value_amd/csrc`` into
``sparse_key_value_amd/libpkm.so`` and the input-generator kernels under
``synth/csrc`` into ``synth/libpkm_synth.so`` (hipcc, one object per source,
compiled in parallel, objects under ``_build/``).  It always recompiles.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ARCH = "gfx950"
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

# -packed-fp32-ops: keep the compiler from forming packed fp32 VALU ops.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]

ROCM_LIB = "/opt/rocm/lib"
# hipBLASLt for the plain bf16 GEMMs of the forward
LINK_LIBS = {"pkm": [f"-L{ROCM_LIB}", "-lhipblaslt", f"-Wl,-rpath,{ROCM_LIB}"]}

TARGETS = {
    "pkm": (os.path.join(ROOT, "sparse_key_value_amd", "csrc"), os.path.join(ROOT, "sparse_key_value_amd", "libpkm.so")),
    "synth": (os.path.join(ROOT, "synth", "csrc"), os.path.join(ROOT, "synth", "libpkm_synth.so")),
}


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build_target(name: str, jobs: int = 8, verbose: bool = False) -> str:
    src_dir, out = TARGETS[name]
    srcs = sorted(os.path.join(src_dir, f) for f in os.listdir(src_dir) if f.endswith(".hip"))
    obj_dir = os.path.join(ROOT, "_build", name)
    os.makedirs(obj_dir, exist_ok=True)
    objs = [os.path.join(obj_dir, os.path.basename(s)[:-4] + ".o") for s in srcs]

    def compile_one(pair):
        s, o = pair
        msg = _run([HIPCC, *HIP_FLAGS, "-I", os.path.join(ROOT, "include"), "-c", s, "-o", o])
        if verbose and msg.strip():
            print(msg)
        return o

    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        list(ex.map(compile_one, zip(srcs, objs)))
    tmp = out + ".tmp"
    libs = LINK_LIBS.get(name, [])
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs, *libs])
    os.replace(tmp, out)
    return out


def build_all(jobs: int | None = None, verbose: bool = False) -> list[str]:
    jobs = jobs or min(8, os.cpu_count() or 4)
    return [build_target(n, jobs, verbose) for n in TARGETS]


if __name__ == "__main__":
    for p in build_all(verbose="-v" in sys.argv):
        print("built", p)
