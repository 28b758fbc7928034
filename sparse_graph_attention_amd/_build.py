"""Compile the gfx950 HIP sources under csrc/ into libgtattn.so beside this file."""
import concurrent.futures
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
# GT_SANITIZE=lib: the host code built with AddressSanitizer and
# UndefinedBehaviorSanitizer (device code unchanged), as a library of its own
# for CPU tests of the argument checks.  The process must preload clang's ASan
# runtime, e.g.
#   GT_SANITIZE=lib LD_PRELOAD=/opt/rocm/llvm/lib/clang/22/lib/linux/libclang_rt.asan-x86_64.so \
#   ASAN_OPTIONS=detect_leaks=0 python -m pytest tests/test_abi_cpu.py tests/test_abi_c.py
# Never used on a GPU.  (GT_SANITIZE=1 instruments the oracle and the
# generators instead, with gcc's runtime, which cannot load this library.)
SANITIZE = os.environ.get("GT_SANITIZE", "") == "lib"
LIB = os.path.join(HERE, "libgtattn_san.so" if SANITIZE else "libgtattn.so")
OBJDIR = os.path.join(ROOT, "_build_san" if SANITIZE else "_build")
HOST_SAN_FLAGS = ("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
                  "-Xarch_host -fno-omit-frame-pointer -Xarch_host -shared-libsan").split()
# bwd.hip is built as its two passes (bwd_dq.hip, bwd_dkv.hip include it)
SOURCES = ["api.hip", "plan.hip", "fused.hip", "sddmm.hip", "softmax.hip", "spmm.hip", "bwd_dq.hip", "bwd_dkv.hip",
           "graph.hip", "calib.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # no packed-fp32 instructions (v_pk_*_f32) anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
    "-I", CSRC,
]


def _compile(src, verbose, objdir, extra):
    obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
    san = HOST_SAN_FLAGS if SANITIZE else []
    cmd = [HIPCC, *FLAGS, *san, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s%s" % (src, r.stdout, r.stderr))
    return obj, r.stderr


def build(verbose: bool = False, out: str = LIB, extra_flags=(), objdir: str = OBJDIR) -> str:
    """Compile every source; extra_flags (e.g. -DGT_F32_D64_U=8) build a tuning variant at `out`."""
    os.makedirs(objdir, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        results = list(ex.map(lambda s: _compile(s, verbose, objdir, list(extra_flags)), SOURCES))
    if verbose:
        for _, err in results:
            lines = [l for l in err.splitlines() if "packed-fp32-ops" not in l and l.strip()]
            if lines:
                print("\n".join(lines))
    tmp = out + ".tmp%d" % os.getpid()
    san = HOST_SAN_FLAGS if SANITIZE else []
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *san, "-o", tmp, *[o for o, _ in results]]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
