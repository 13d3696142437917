"""Build libgdnspec.so (HIP, gfx950) in-tree with hipcc.

``python -m linear_attention_gdn_amd.build`` compiles every ``csrc/*.hip``
into ``linear_attention_gdn_amd/libgdnspec.so``.  All device code is built
with packed-FP32 instructions disabled and kernel-argument preloading on.
"""

from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgdnspec.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the first 16 dwords of kernel arguments arrive in SGPRs at wave launch
    # instead of through a scalar load the first global loads would wait for
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    # keep the intermediate files (among them the gfx950 assembly,
    # _build/<source>-hip-amdgcn-amd-amdhsa-gfx950.s) beside the objects, for
    # the static checks of the generated code
    "-save-temps=obj",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def device_asm_path(src: str) -> str:
    """Where the build leaves the gfx950 assembly of one source."""
    stem = os.path.splitext(os.path.basename(src))[0]
    return os.path.join(HERE, "_build", f"{stem}-hip-amdgcn-amd-amdhsa-{ARCH}.s")


def build(verbose: bool = False) -> str:
    """Compile all HIP sources into the shared library; returns its path."""
    from concurrent.futures import ThreadPoolExecutor

    build_dir = os.path.join(HERE, "_build")
    os.makedirs(build_dir, exist_ok=True)
    cmds = []
    for src in sources():
        obj = os.path.join(build_dir, os.path.basename(src) + ".o")
        cmds.append((obj, [hipcc(), *HIPCC_FLAGS, "-c", src, "-o", obj]))
    for _, cmd in cmds:
        if verbose:
            print(" ".join(cmd), flush=True)
    # one hipcc per source, in parallel (each is single-threaded)
    jobs = max(1, min(len(cmds), os.cpu_count() or 1, 8))
    with ThreadPoolExecutor(jobs) as ex:
        for f in [ex.submit(subprocess.run, cmd, check=True) for _, cmd in cmds]:
            f.result()
    objs = [obj for obj, _ in cmds]
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
