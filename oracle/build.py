"""Compile the CPU oracle (plain C, OpenMP) in place.  Test infrastructure."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def build(verbose: bool = False) -> str:
    out = os.path.join(HERE, "liboracle.so")
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c11",
           "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra", "-Werror",
           os.path.join(HERE, "oracle.c"), "-o", out + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
