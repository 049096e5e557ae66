"""Build the CPU oracle (test infrastructure) with gcc: no fast-math, no FP contraction."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SO = os.path.join(HERE, "liboracle.so")


def build():
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "oracle.c", "-o", SO + ".tmp", "-lm"]
    r = subprocess.run(cmd, cwd=HERE, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("oracle build failed:\n%s\n%s" % (r.stdout, r.stderr))
    os.replace(SO + ".tmp", SO)


if __name__ == "__main__":
    build()
