"""Build libdlrm_mi355x.so (the HIP kernels and the C ABI) for gfx950.

hipcc compiles ahead of time for gfx950 only, one object per source in
parallel, then links them.  Packed-FP32 instructions are disabled: ordinary
float code is compiled to scalar VALU operations.
"""
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdlrm_mi355x.so")
OBJ_DIR = os.path.join(HERE, "_build")
SOURCES = ["abi.hip", "bottom_mlp.hip", "emb_interact.hip", "forward_small.hip", "linear.hip",
           "mlp_chain.hip", "probe.hip", "slice_mlp.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "-O3", "-std=c++17", "-fPIC",
    "--offload-arch=gfx950",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]


def build(out: str = LIB, extra_flags=(), verbose: bool = False) -> str:
    """Compile every HIP source into `out` and return its path."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    tag = os.path.basename(out).replace(".", "_")

    def compile_one(src):
        obj = os.path.join(OBJ_DIR, f"{tag}_{src}.o")
        cmd = [HIPCC, *FLAGS, *extra_flags, "-c", "-o", obj, os.path.join(CSRC, src)]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True, cwd=CSRC)
        return obj

    with ThreadPoolExecutor(max_workers=len(SOURCES)) as pool:
        objs = list(pool.map(compile_one, SOURCES))
    tmp = out + ".tmp"
    cmd = [HIPCC, "-shared", "--offload-arch=gfx950", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, cwd=CSRC)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
