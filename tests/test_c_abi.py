"""The C ABI from plain C (tests/c_abi/lq_c_driver.c, built by
__graft_entry__.build()).

CPU: include/leapquant.h compiles as C99 and C11 with warnings as errors,
and the driver's argument checks (status codes of rejected calls, status
strings, ABI version) pass without a GPU.  GPU: the driver quantizes,
decodes and closes windows through the ABI on seeded inputs written by this
test, and its outputs are compared with the oracle under the rules of the
entry-point tests.
"""
import os
import subprocess
import sys

import numpy as np
import pytest

from oracle import leapquant_oracle as O
from tests import parity as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "c_abi", "lq_c_driver")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
MAGIC = 0x3143514C


def _driver():
    if not os.path.exists(DRIVER):
        sys.path.insert(0, ROOT)
        from recurrent_state_quant_amd import build as B
        if not os.path.exists(B.LIB_PATH):
            pytest.fail("libleapquant.so is not built (run __graft_entry__.build())")
        B.build_c_driver()
    return DRIVER


@pytest.mark.parametrize("std", ["c99", "c11"])
def test_header_compiles_as_c(tmp_path, std):
    src = tmp_path / "h.c"
    src.write_text('#include "leapquant.h"\n'
                   "int main(void) { lq_params p; lq_state s; (void)p; (void)s;\n"
                   "  return leapquant_abi_version() == LEAPQUANT_ABI_VERSION ? 0 : 1; }\n")
    res = subprocess.run(["gcc", f"-std={std}", "-Wall", "-Wextra", "-Werror", "-fsyntax-only",
                          "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                          "-I", os.path.join(ROCM, "include"), str(src)], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr


def test_c_driver_argument_checks():
    res = subprocess.run([_driver(), "--check"], capture_output=True, text=True, timeout=60)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "argument checks passed" in res.stdout


def _inputs(rng, n, T, gate):
    from tests.test_gpu_parity import _states_with_outliers, _token
    S0 = _states_with_outliers(rng, n)
    toks = [_token(rng, n, gate) for _ in range(T)]
    return S0, {k: np.stack([t[k] for t in toks]) for k in toks[0]}


def _run_driver(tmp_path, S0, tok, n, p, r, gate, flags):
    T = tok["q"].shape[0]
    fin, fout = tmp_path / "in.bin", tmp_path / "out.bin"
    g = 0 if gate == "gdn" else 1
    with open(fin, "wb") as f:
        np.array([MAGIC, n, p, r, g, flags, T], "<i4").tofile(f)
        for x in (S0, tok["q"], tok["k"], tok["v"], tok["beta"], tok["alpha"]):
            np.ascontiguousarray(x, "<f4").tofile(f)
    print(f"c driver: n={n} p={p} r={r} gate={gate} flags={flags} T={T}", flush=True)
    res = subprocess.run([_driver(), str(fin), str(fout)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    raw = np.fromfile(fout, np.uint8)
    out, off = {}, 0

    def take(name, dtype, shape):
        nonlocal off
        size = int(np.prod(shape)) * np.dtype(dtype).itemsize
        out[name] = raw[off:off + size].view(dtype).reshape(shape)
        off += size
    take("o", "<f4", (T, n, 128))
    take("codes_raw", "i1", (n, 128 * 128))
    take("row_scale", "<f4", (n, 128))
    take("col_scale", "<f4", (n, 128))
    if r:
        take("comp_idx", "<i4", (n, r))
        take("comp_val", "<f4", (n, r, 128))
    take("S_out", "<f4", (n, 128, 128))
    assert off == raw.size
    # stored layout -> row-major codes (the layout of include/leapquant.h)
    i = np.arange(128)[:, None]
    j = np.arange(128)[None, :]
    x = i & 63
    offs = (i >> 6) * 8192 + j * 64 + (((x & 0x0C) << 2) | ((x & 0x30) >> 2) | (x & 3))
    out["codes"] = out["codes_raw"][:, offs]
    return out


@pytest.mark.gpu
@pytest.mark.parametrize("gate,p,r,flags,extra", [("gdn", 8, 4, 0, 3), ("kda", 8, 8, 0, 2),
                                                  ("gdn", 16, 0, O.NO_SMOOTH, 5), ("gdn", 4, 16, O.NO_DELTA, 1)])
def test_c_driver_matches_oracle(tmp_path, gate, p, r, flags, extra):
    rng = np.random.default_rng(7100 + 13 * p + r + flags + (gate == "kda"))
    n = 5
    T = p + extra
    S0, tok = _inputs(rng, n, T, gate)
    got = _run_driver(tmp_path, S0, tok, n, p, r, gate, flags)
    G = O.GATE_KDA if gate == "kda" else O.GATE_GDN
    t64 = {k: v.astype(np.float64) for k, v in tok.items()}
    # window 0 from the oracle's split of S0 (the driver's quantize of the
    # same fp32 states is bit-exact), the last token fused with the close
    b0 = O.quantize(S0, r, flags & O.NO_SMOOTH)
    o_ref, _, S_p, b1 = O.window(b0, t64, 0, p, G, r, flags)
    P.assert_close(got["o"][:p], o_ref, f"c driver {gate}: window 0 outputs")
    b_gpu = {k: got[k] for k in ("codes", "row_scale", "col_scale") + (("comp_idx", "comp_val") if r else ())}
    if not r:
        b_gpu["comp_idx"] = np.zeros((n, 0), np.int32)
        b_gpu["comp_val"] = np.zeros((n, 0, 128), np.float32)
    P.compare_boundary(b_gpu, b1, S_p.astype(np.float32), r, f"c driver {gate}: boundary")
    # the partial second window starts from the driver's own boundary
    o2, _, _, _ = O.window(b_gpu, t64, p, extra, G, r, flags)
    P.assert_close(got["o"][p:], o2, f"c driver {gate}: window 1 outputs")
    # dequantize_state of that boundary
    P.assert_close(got["S_out"], O.dequantize(b_gpu), f"c driver {gate}: dequantized", rtol=1e-6, atol=0)
