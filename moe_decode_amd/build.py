"""Build libmoedecode.so (all HIP kernels + the C-ABI) for gfx950, in-tree."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SO = os.path.join(HERE, "libmoedecode.so")
SRC = os.path.join(HERE, "csrc", "moe_capi.hip")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-std=c++17",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-result"]


def build(extra=()):
    cmd = [HIPCC] + FLAGS + list(extra) + [SRC, "-o", SO + ".tmp"]
    r = subprocess.run(cmd, cwd=HERE, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("libmoedecode build failed:\n%s\n%s" % (r.stdout, r.stderr))
    os.replace(SO + ".tmp", SO)
    return r.stderr


if __name__ == "__main__":
    build()
