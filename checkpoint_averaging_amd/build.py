"""Builds libdlmerge.so (HIP kernels + C ABI) for gfx950, in the package
directory, with hipcc.

    python -m checkpoint_averaging_amd.build

Flags that fix the arithmetic: -ffp-contract=off (no fused multiply-add),
-fhip-fp32-correctly-rounded-divide-sqrt (IEEE division),
-fno-gpu-flush-denormals-to-zero (subnormals kept).  Packed fp32 instructions
are switched off for the device code.
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libdlmerge.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = [os.path.join(CSRC, "kernels.hip"), os.path.join(CSRC, "polar.hip"),
           os.path.join(CSRC, "noalloc.hip"), os.path.join(CSRC, "api.cpp")]
DRIVER = os.path.join(PKG, "dlmerge_driver")
DRIVER_SOURCES = [os.path.join(CSRC, "merge_driver.hip")]
POLAR_DRIVER = os.path.join(PKG, "dlpolar_driver")
POLAR_DRIVER_SOURCES = [os.path.join(CSRC, "polar_driver.hip")]

HIPFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wextra",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so;
    # that note is harmless and is filtered out.
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if noise not in l]
    if msgs and (verbose or res.returncode != 0):
        print("\n".join(msgs), file=sys.stderr)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}")


def build(verbose: bool = False) -> str:
    """Builds libdlmerge.so and the dlmerge_driver and dlpolar_driver
    executables that link it."""
    _run([HIPCC, *HIPFLAGS, "-shared", "-o", LIB + ".tmp", *SOURCES], verbose)
    os.replace(LIB + ".tmp", LIB)
    for exe, srcs in ((DRIVER, DRIVER_SOURCES), (POLAR_DRIVER, POLAR_DRIVER_SOURCES)):
        _run([HIPCC, *HIPFLAGS, "-o", exe + ".tmp", *srcs, f"-L{PKG}", "-ldlmerge",
              "-Wl,-rpath,$ORIGIN"], verbose)
        os.replace(exe + ".tmp", exe)
    return LIB


def device_asm(out_path: str, source: str = "kernels.hip") -> str:
    """gfx950 assembly of one source's kernels (for inspecting the instruction mix)."""
    cmd = [HIPCC, *HIPFLAGS, "--cuda-device-only", "-S", "-o", out_path,
           os.path.join(CSRC, source)]
    subprocess.run(cmd, check=True, capture_output=True)
    return out_path


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
