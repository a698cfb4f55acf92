"""A slab past 2^31 bytes of codes: every per-state offset in the kernels and
the ABI's range checks must be 64-bit.

140,000 states hold 2.29e9 bytes of codes (the fp32 source of the initial
split is 9.2 GB).  The slab is quantized, decodes one token and closes its
window with the fused last token (p = 2, r = 2); states at the start, the
middle and the end are compared with the oracle under the entry-point rules.
"""
import numpy as np
import pytest
import torch

import recurrent_state_quant_amd as lq
from oracle import leapquant_oracle as O
from tests import parity as P
from tests.gpu_run import to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    lq.load()
    yield
    torch.cuda.synchronize()


def test_offsets_beyond_2_31_bytes():
    n, p, r = 140_000, 2, 2
    assert n * 128 * 128 > 2 ** 31
    sample = np.array([0, 1, 70_001, n - 2, n - 1])
    print(f"large slab: n={n} (codes {n * 128 * 128 / 1e9:.2f} GB)", flush=True)
    g = torch.Generator(device=DEV).manual_seed(31)
    st = lq.LeapQuantState(n, p, r, "gdn", DEV)
    S = torch.randn((n, 128, 128), generator=g, device=DEV).mul_(0.02)
    lq.leapquant_quantize_state(st, S)
    S_host = to_np(S[torch.as_tensor(sample, device=DEV)])
    del S
    tok = {}
    for name, shape in (("q", (p, n, 128)), ("k", (p, n, 128)), ("v", (p, n, 128)), ("beta", (p, n)),
                        ("alpha", (p, n))):
        tok[name] = torch.rand(shape, generator=g, device=DEV) if name in ("beta", "alpha") else \
            torch.randn(shape, generator=g, device=DEV)
    tok["q"] /= tok["q"].norm(dim=-1, keepdim=True)
    tok["k"] /= tok["k"].norm(dim=-1, keepdim=True)
    tok["alpha"].mul_(0.9).add_(0.05)
    torch.cuda.synchronize()
    b0 = {k: to_np(v) for k, v in st.boundary(sample).items()}
    # the initial split of the same fp32 states is bit-exact
    P.compare_boundary(b0, O.quantize(S_host, r), S_host, r, "large slab: quantize", exact=True)

    o = torch.empty((p, n, 128), device=DEV)
    lq.leapquant_decode_step(st, 0, *[tok[x][0] for x in ("q", "k", "v", "beta", "alpha")], o[0])
    lq.leapquant_decode_close(st, 1, *[tok[x][1] for x in ("q", "k", "v", "beta", "alpha")], o[1])
    torch.cuda.synchronize()
    ix = torch.as_tensor(sample, device=DEV)
    t64 = {k: to_np(v.index_select(1, ix)).astype(np.float64) for k, v in tok.items()}
    o_ref, _, S_p, b1 = O.window(b0, t64, 0, p, O.GATE_GDN, r)
    P.assert_close(to_np(o.index_select(1, ix)), o_ref, "large slab: outputs")
    got = {k: to_np(v) for k, v in st.boundary(sample).items()}
    P.compare_boundary(got, b1, S_p.astype(np.float32), r, "large slab: boundary after the close")
