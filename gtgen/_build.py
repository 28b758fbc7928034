"""Compile gtgen.c into libgtgen.so beside it (plain gcc, OpenMP)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gtgen.c")
# GT_SANITIZE=1: an AddressSanitizer + UndefinedBehaviorSanitizer build (a
# library of its own; the process must preload gcc's libasan).
SANITIZE = os.environ.get("GT_SANITIZE", "") == "1"
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]
LIB = os.path.join(HERE, "libgtgen_san.so" if SANITIZE else "libgtgen.so")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    san = SAN_FLAGS if SANITIZE else []
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", *san, "-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
