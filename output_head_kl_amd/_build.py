"""Build the HIP library ``libkdkl.so`` in-tree for gfx950 (hipcc cross-compiles; no GPU needed)."""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = [os.path.join(PKG, "csrc", f) for f in ("kd_kernels.hip", "kd_api.hip", "kd_topk.hip")]
OUT = os.path.join(PKG, "libkdkl.so")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 vector ops stay off in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


# A C caller of the library (no Python in its process), used by the tests.
DRIVER_SRC = os.path.join(ROOT, "tests", "c_abi", "kd_driver.c")
DRIVER = os.path.join(ROOT, "tests", "c_abi", "kd_driver")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in res.stderr.splitlines()
                     if "packed-fp32-ops" not in l and l.strip())
    if res.returncode != 0:
        raise RuntimeError(f"{cmd[0]} failed ({res.returncode}):\n{errs}")
    if verbose and errs:
        print(errs, file=sys.stderr)


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = OUT + ".tmp"
    _run([hipcc, *FLAGS, *SRC, "-o", tmp], verbose)
    os.replace(tmp, OUT)
    # host code only (plain C against the HIP runtime's C API); at run time it loads the
    # library next to the package
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc)))
    tmp = DRIVER + ".tmp"
    _run([os.environ.get("CC", "gcc"), "-O2", "-std=c11", "-Wall",
          "-I", os.path.join(ROOT, "include"), "-I", os.path.join(rocm, "include"),
          "-D__HIP_PLATFORM_AMD__", DRIVER_SRC, "-o", tmp,
          "-L", PKG, "-lkdkl", "-L", os.path.join(rocm, "lib"), "-lamdhip64",
          "-Wl,-rpath,$ORIGIN/../../output_head_kl_amd:" + os.path.join(rocm, "lib")], verbose)
    os.replace(tmp, DRIVER)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
