"""Host-sanitizer build of libnq: AddressSanitizer and UndefinedBehaviorSanitizer
on the host pass of every translation unit (argument validation, routing,
plans, launch setup); device code is compiled as in the normal build.  The
result, _build/libnq_hostsan.so, is for running the CPU test suite against:

    python -m group_wise_affine_quantize_amd.build_sanitized
    LD_PRELOAD=<clang asan runtime> ASAN_OPTIONS=detect_leaks=0 \\
        NQ_LIBRARY=_build/libnq_hostsan.so python -m pytest tests -m "not gpu"

The sanitizer runtime is not linked in; it is preloaded (the path is printed
by this script), since the Python interpreter that loads the library is not
instrumented.
"""
import glob
import os
import subprocess
import sys

from group_wise_affine_quantize_amd import build as nq_build

OUT_DIR = os.path.join(nq_build.ROOT, "_build", "hostsan")
LIB = os.path.join(nq_build.ROOT, "_build", "libnq_hostsan.so")
# every sanitizer flag is scoped to the host pass
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-g"]


def runtime():
    """The clang AddressSanitizer runtime to preload."""
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else ""


def build(verbose=False):
    os.makedirs(OUT_DIR, exist_ok=True)
    objs, procs = [], []
    for src in nq_build.SOURCES:
        obj = os.path.join(OUT_DIR, os.path.splitext(src)[0] + ".o")
        cmd = [nq_build.HIPCC, *nq_build.FLAGS, *HOST_SAN, "-c", os.path.join(nq_build.CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(obj)
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        if p.returncode:
            print(out.decode(errors="replace"), file=sys.stderr)
            failed.append(src)
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    # the runtime's symbols stay undefined here and come from the preload
    cmd = [nq_build.HIPCC, f"--offload-arch={nq_build.ARCH}", "-shared", "-fPIC", "-o", LIB, *objs]
    subprocess.run(cmd, check=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    print("preload:", runtime())
