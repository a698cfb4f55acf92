"""Build libleapquant.so in-tree with hipcc for gfx950."""
import os
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
LIB_PATH = os.path.join(PKG_DIR, "libleapquant.so")
KERNEL_SOURCES = ("lq_device.h", "lq_decode_one.h", "lq_decode_body.inc", "lq_close16_body.inc", "lq_decode.hip",
                  "lq_close.hip", "lq_baselines.hip")
SOURCES = [os.path.join(PKG_DIR, "csrc", f) for f in ("lq_decode.hip", "lq_close.hip", "lq_baselines.hip",
                                                     "lq_abi.cpp")]
ARCH = "gfx950"


def hipcc_command(out=LIB_PATH, extra=()):
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    return [hipcc, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            # packed fp32 VALU ops stay off: only scalar fp32 ops are emitted
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # MFMA accumulators in VGPRs: the close kernel post-processes them
            # on the VALU, and AGPR copies would double its register footprint
            "-mllvm", "-amdgpu-mfma-vgpr-form=1",
            # products fused into adds only within one expression (a*b + c
            # becomes one fma, as written): the fusion the default mode leaves
            # to the back end picks an operand by the shape of the code around
            # it, so one body included in two kernels could round differently
            "-ffp-contract=on",
            "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG_DIR, "csrc"),
            *extra, "-o", out, *SOURCES]


C_DRIVER_SRC = os.path.join(ROOT, "tests", "c_abi", "lq_c_driver.c")
C_DRIVER = os.path.join(ROOT, "tests", "c_abi", "lq_c_driver")


def c_driver_command(out=C_DRIVER):
    """gcc line of the plain-C client of the ABI (tests/c_abi): C11, the
    public header only, linked against the in-tree library."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
            "-I", os.path.join(ROOT, "include"), "-I", os.path.join(rocm, "include"),
            "-o", out, C_DRIVER_SRC, "-L", PKG_DIR, "-lleapquant", "-L", os.path.join(rocm, "lib"),
            "-lamdhip64", "-Wl,-rpath,$ORIGIN/../../recurrent_state_quant_amd",
            "-Wl,-rpath," + os.path.join(rocm, "lib")]


def build_c_driver(verbose=False):
    """Compile tests/c_abi/lq_c_driver against the built library."""
    cmd = c_driver_command()
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise subprocess.CalledProcessError(res.returncode, cmd, res.stdout, res.stderr)
    return C_DRIVER


def build(verbose=False):
    """Compile the HIP library; raises CalledProcessError on failure."""
    tmp = LIB_PATH + ".tmp"
    cmd = hipcc_command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise subprocess.CalledProcessError(res.returncode, cmd, res.stdout, res.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_c_driver(verbose=True))
