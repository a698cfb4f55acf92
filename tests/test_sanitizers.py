"""Host-side argument validation under AddressSanitizer and UBSan (CPU).

The C ABI's validation (recurrent_state_quant_amd/csrc/lq_abi.cpp) is
compiled by the host compiler with -fsanitize=address,undefined into a
library of its own, linked with stand-in kernel launchers that abort if
they are ever reached, and driven by the plain-C client's --check mode
(tests/c_abi/lq_c_driver.c, also sanitized): every rejected call must
return its status code without a sanitizer report and without reaching a
launch.  Only host code is built here; the GPU kernels are not involved.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]

STUB = r"""
#include <stdio.h>
#include <stdlib.h>
#include "lq_kernels.h"
namespace lq {
static hipError_t reached(const char *what) {
  fprintf(stderr, "launch reached: %s\n", what);
  abort();
}
hipError_t launch_decode_step(const DecodeArgs &, bool, hipStream_t) { return reached("decode_step"); }
hipError_t launch_bf16w_decode(const Bf16WinArgs &, bool, hipStream_t) { return reached("bf16w_decode"); }
hipError_t launch_bf16w_close(const Bf16WinArgs &, bool, hipStream_t) { return reached("bf16w_close"); }
hipError_t launch_dense_step(const DenseArgs &, bool, bool, hipStream_t) { return reached("dense_step"); }
hipError_t launch_window_close(const CloseArgs &, bool, hipStream_t) { return reached("window_close"); }
hipError_t launch_decode_close(const CloseArgs &, bool, hipStream_t) { return reached("decode_close"); }
hipError_t launch_quantize_state(const CloseArgs &, hipStream_t) { return reached("quantize_state"); }
hipError_t launch_dequantize(const DequantArgs &, hipStream_t) { return reached("dequantize"); }
hipError_t launch_mixed(const MixedArgs &, bool, hipStream_t) { return reached("mixed"); }
bool mixed_supported(const CloseArgs &) { return true; }
hipError_t launch_stream_ref(const void *, uint32_t, void *, uint32_t, int, int, uint32_t *, hipStream_t) {
  return reached("stream_ref");
}
}  // namespace lq
"""


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, " ".join(cmd) + "\n" + res.stdout + res.stderr
    return res


@pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None, reason="host compilers")
def test_argument_checks_under_asan_and_ubsan(tmp_path):
    inc = ["-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "recurrent_state_quant_amd", "csrc"), "-I", os.path.join(ROCM, "include")]
    stub = tmp_path / "launch_stub.cpp"
    stub.write_text(STUB)
    lib = tmp_path / "libleapquant.so"
    _run(["g++", "-std=c++17", "-O1", "-fPIC", "-shared", *SAN, *inc, "-o", str(lib),
          os.path.join(ROOT, "recurrent_state_quant_amd", "csrc", "lq_abi.cpp"), str(stub)])
    drv = tmp_path / "lq_c_driver"
    _run(["gcc", "-std=c11", "-O1", "-Wall", "-Wextra", "-Werror", *SAN, *inc, "-o", str(drv),
          os.path.join(ROOT, "tests", "c_abi", "lq_c_driver.c"), "-L", str(tmp_path), "-lleapquant",
          "-L", os.path.join(ROCM, "lib"), "-lamdhip64", f"-Wl,-rpath,{tmp_path}",
          "-Wl,-rpath," + os.path.join(ROCM, "lib")])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = _run([str(drv), "--check"], env=env, timeout=120)
    assert "argument checks passed" in res.stdout
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr, res.stderr
