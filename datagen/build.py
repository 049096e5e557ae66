"""Build the seeded input generator's two shared libraries (host C and device HIP)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
HOST_SO = os.path.join(HERE, "libdg_host.so")
DEV_SO = os.path.join(HERE, "libdg_device.so")

HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-std=c++17",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _run(cmd):
    r = subprocess.run(cmd, cwd=HERE, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("build failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))


def build_host():
    _run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
          "dg_host.c", "-o", HOST_SO + ".tmp"])
    os.replace(HOST_SO + ".tmp", HOST_SO)


def build_device():
    _run(["/opt/rocm/bin/hipcc"] + HIP_FLAGS + ["dg_device.hip", "-o", DEV_SO + ".tmp"])
    os.replace(DEV_SO + ".tmp", DEV_SO)


def build():
    build_host()
    build_device()


if __name__ == "__main__":
    build()
