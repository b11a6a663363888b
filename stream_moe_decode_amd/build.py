"""Compile the HIP library libflint.so for gfx950 (in-tree)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SO = os.path.join(HERE, "libflint.so")
SOURCES = [os.path.join(HERE, "csrc", f) for f in ("flint_kernel.hip", "flint_batch.hip", "flint_micro.hip", "flint_runtime.cpp")]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 instructions stay off (plain float code only)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = SO + ".tmp%d" % os.getpid()
    cmd = [hipcc] + HIPCC_FLAGS + ["-x", "hip"] + SOURCES + ["-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + r.stderr[-8000:])
    if verbose and r.stderr:
        print(r.stderr)
    os.replace(tmp, SO)
    return SO


if __name__ == "__main__":
    print(build(verbose=True))
