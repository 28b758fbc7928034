"""Compile the oracle (oracle.c) into liboracle.so beside it.  Test infrastructure."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
# GT_SANITIZE=1: an AddressSanitizer + UndefinedBehaviorSanitizer build of the
# oracle (a library of its own, loaded instead of the plain one).  The process
# must preload gcc's libasan, e.g.
#   GT_SANITIZE=1 LD_PRELOAD=$(gcc -print-file-name=libasan.so) ASAN_OPTIONS=detect_leaks=0 \
#   python -m pytest tests -m "not gpu"
SANITIZE = os.environ.get("GT_SANITIZE", "") == "1"
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]
LIB = os.path.join(HERE, "liboracle_san.so" if SANITIZE else "liboracle.so")


def build(src: str = SRC, out: str = LIB, extra_flags=(), verbose: bool = False) -> str:
    tmp = out + ".tmp%d" % os.getpid()
    san = SAN_FLAGS if SANITIZE and out == LIB else []  # planted mutants are built plain
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", *san, *extra_flags, "-o", tmp, src,
           "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
