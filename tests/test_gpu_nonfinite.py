"""Non-finite values stay in their own state.

The ABI leaves results for NaN or Inf inputs unspecified but in bounds.
Every data-dependent index in the kernels is bounded (compensator row
indices are checked where read, the top-r selection falls back to the
lowest unpicked row when norms are NaN), so a state fed NaN or Inf must
not disturb any other state.  A slab mixes such states (and tokens) with
clean ones; the clean states must match the oracle exactly as in the
entry-point tests, and every compensator index must stay in [0, 128).
"""
import numpy as np
import pytest
import torch

import recurrent_state_quant_amd as lq
from oracle import leapquant_oracle as O
from tests import parity as P
from tests.gpu_run import boundary_np, to_np, upload_boundary
from tests.test_gpu_parity import _dev, _gate, _oracle_records, _random_window_inputs, _states_with_outliers, \
    _token, _upload_records

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    lq.load()
    yield
    torch.cuda.synchronize()


def test_quantize_isolates_nonfinite_states():
    rng = np.random.default_rng(9300)
    n, r = 11, 4
    S = _states_with_outliers(rng, n)
    bad = np.array([2, 5, 9])
    S[2, 3, 7] = np.nan
    S[5, :, 4] = np.inf
    S[9] = np.nan
    st = lq.LeapQuantState(n, 16, r, "gdn", DEV)
    lq.leapquant_quantize_state(st, _dev(S))
    torch.cuda.synchronize()
    got = boundary_np(st)
    assert ((got["comp_idx"] >= 0) & (got["comp_idx"] < 128)).all()
    good = np.setdiff1d(np.arange(n), bad)
    P.compare_boundary({k: v[good] for k, v in got.items()}, O.quantize(S[good], r), S[good], r,
                       "clean states beside non-finite ones", exact=True)


@pytest.mark.parametrize("gate", ["gdn", "kda"])
@pytest.mark.parametrize("fused", [True, False])
def test_window_isolates_nonfinite_tokens(gate, fused):
    rng = np.random.default_rng(9400 + 2 * (gate == "kda") + fused)
    n, p, r = 13, 16, 4
    t = p - 1
    b, recs = _random_window_inputs(rng, n, p, t, gate, r)
    tok = _token(rng, n, gate)
    bad = np.array([1, 6, 12])
    tok["q"][1, 5] = np.nan
    tok["v"][6, :] = np.inf
    tok["alpha"][12] = np.nan
    recs[3][2][6, 9] = np.nan          # a buffered u row of a bad state
    st = lq.LeapQuantState(n, p, r, gate, DEV)
    upload_boundary(st, b)
    _upload_records(st, recs, gate)
    o = torch.empty((n, 128), device=DEV)
    args = [_dev(tok[x]) for x in ("q", "k", "v", "beta", "alpha")]
    if fused:
        lq.leapquant_decode_close(st, t, *args, o)
    else:
        lq.leapquant_decode_step(st, t, *args, o)
        lq.leapquant_window_close(st, t + 1)
    torch.cuda.synchronize()
    got = boundary_np(st)
    assert ((got["comp_idx"] >= 0) & (got["comp_idx"] < 128)).all()
    good = np.setdiff1d(np.arange(n), bad)
    sel = lambda d: {k: np.asarray(v)[good] for k, v in d.items()}  # noqa: E731
    S_prev = O.replay(O.dequantize(sel(b)), _oracle_records([(a[good], kt[good], u[good]) for a, kt, u in recs], gate))
    t64 = {k: v[good].astype(np.float64) for k, v in tok.items()}
    o_ref, S_t, _ = O.step(S_prev, *[t64[x] for x in ("q", "k", "v", "beta", "alpha")], _gate(gate))
    P.assert_close(to_np(o)[good], o_ref, "clean outputs beside non-finite ones")
    P.compare_boundary(sel(got), O.quantize(S_t, r), S_t.astype(np.float32), r,
                       "clean boundaries beside non-finite ones")
