"""Build the CPU oracle: gcc -O2 (no fast-math) with OpenMP -> libssd_oracle.so."""
import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))


def build_oracle(verbose=False):
    src = os.path.join(_HERE, "ssd_oracle.c")
    out = os.path.join(_HERE, "libssd_oracle.so")
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared", "-std=c99",
           "-Wall", "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_oracle(verbose=True))
