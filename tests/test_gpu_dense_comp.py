"""Parity of the dense Compensator Tokens (LQ_DENSE_COMP) on the HIP path.

The boundary state carries r tokens (k_c, w_c) with dense unit keys from
subspace iteration (the oracle's `dense_keys`).  Entry-point tests feed both
sides the same boundary state and buffered records.  Boundaries written by
the GPU are compared with P.compare_dense_boundary: keys within KEY_ATOL of
the oracle's, then values, scales and codes against the oracle's split of
the same state with the GPU's keys.  With zero iterations the split is the
row extraction, bit for bit.
"""
import numpy as np
import pytest
import torch

import recurrent_state_quant_amd as lq
from oracle import leapquant_oracle as O
from tests import parity as P
from tests.gpu_run import boundary_np, run_window, to_np, upload_boundary
from tests.test_gpu_parity import (_dev, _gate, _oracle_records, _random_window_inputs, _states_with_outliers,
                                   _token, _upload_records, _workload)

pytestmark = pytest.mark.gpu
DEV = "cuda"
DENSE = lq.LQ_DENSE_COMP


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    lq.load()
    yield
    torch.cuda.synchronize()


def _slab(n, p, r, gate, iters, flags=0):
    return lq.LeapQuantState(n, p, r, gate, DEV, flags=flags | DENSE, comp_iters=iters)


def _special_states(rng, n):
    S = _states_with_outliers(rng, n)
    S[3] = 0.0                                                   # zero state: zero keys
    a, c = rng.standard_normal((128, 2)), rng.standard_normal((2, 128))
    S[5] = (0.1 * a @ c).astype(np.float32)                      # rank 2: keys past it dropped
    return S


@pytest.mark.parametrize("r,iters,flags", [(1, 0, 0), (4, 0, 0), (16, 0, 0), (4, 0, lq.LQ_NO_SMOOTH),
                                           (1, 1, 0), (4, 1, 0), (4, 2, 0), (8, 3, 0), (16, 2, 0),
                                           (4, 2, lq.LQ_NO_SMOOTH), (4, 8, 0)])
def test_quantize_state(r, iters, flags):
    rng = np.random.default_rng(3000 + 17 * r + iters + 5 * flags)
    n = 23
    S = _special_states(rng, n)
    st = _slab(n, 16, r, "gdn", iters, flags)
    lq.leapquant_quantize_state(st, _dev(S))
    torch.cuda.synchronize()
    gb = boundary_np(st)
    if iters == 0:
        # the row extraction, bit for bit, with one-hot keys
        ref = O.quantize(S, r, flags | O.DENSE_COMP, 0)
        P.compare_boundary(gb, ref, S, r, "dense quantize, 0 iterations", exact=True)
        rows = O.quantize(S, r, flags)
        for k in ("codes", "row_scale", "col_scale", "comp_idx", "comp_val"):
            np.testing.assert_array_equal(gb[k], rows[k], err_msg=k)
    else:
        stats = P.compare_dense_boundary(gb, S, r, iters, flags, f"dense quantize r={r} iters={iters}")
        print(stats)
    if iters > 0:
        # iterated keys of the zero state are zero, and so are those past rank 2
        K = gb["comp_key"].astype(np.float64)
        np.testing.assert_array_equal(K[3], 0)
        np.testing.assert_array_equal(K[5, 2:], 0)


def test_dequantize():
    rng = np.random.default_rng(3100)
    n, r = 11, 4
    S = _states_with_outliers(rng, n)
    b = O.quantize(S, r, O.DENSE_COMP, 2)
    st = _slab(n, 16, r, "gdn", 2)
    upload_boundary(st, b)
    out = torch.empty((n, 128, 128), device=DEV)
    lq.leapquant_dequantize_state(st, out)
    torch.cuda.synchronize()
    ref = O.dequantize(b)
    P.assert_close(to_np(out), ref, "dense dequantize", rtol=1e-6, atol=1e-6 * np.abs(ref).max())


@pytest.mark.parametrize("gate", ["gdn", "kda"])
@pytest.mark.parametrize("p,t", [(1, 0), (16, 0), (16, 9), (16, 15), (32, 31)])
@pytest.mark.parametrize("r", [1, 4, 16])
def test_decode_step_entry(gate, p, t, r):
    rng = np.random.default_rng(3200 + 1000 * p + 10 * t + r + (gate == "kda"))
    n = 19
    b, recs = _random_window_inputs(rng, n, p, t, gate, r, dense_iters=2)
    st = _slab(n, p, r, gate, 2)
    upload_boundary(st, b)
    _upload_records(st, recs, gate)
    tok = _token(rng, n, gate)
    o = torch.empty((n, 128), device=DEV)
    lq.leapquant_decode_step(st, t, *[_dev(tok[x]) for x in ("q", "k", "v", "beta", "alpha")], o)
    torch.cuda.synchronize()
    S_prev = O.replay(O.dequantize(b), _oracle_records(recs, gate))
    t64 = {k: v.astype(np.float64) for k, v in tok.items()}
    o_ref, _, (_, _, u) = O.step(S_prev, *[t64[x] for x in ("q", "k", "v", "beta", "alpha")], _gate(gate))
    P.assert_close(to_np(o), o_ref, "o_t")
    P.assert_close(to_np(st.buf_u[:, t]), u, "u_t")


@pytest.mark.parametrize("gate", ["gdn", "kda"])
@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("p,length", [(1, 1), (16, 16), (16, 5), (32, 32), (64, 37)])
@pytest.mark.parametrize("r,iters", [(1, 2), (4, 0), (4, 2), (16, 2)])
def test_window_close_entry(gate, fused, p, length, r, iters):
    rng = np.random.default_rng(3300 + 7 * p + length + 100 * r + iters + 2 * fused + (gate == "kda"))
    n = 21
    nrec = length - 1 if fused else length
    b, recs = _random_window_inputs(rng, n, p, nrec, gate, r, dense_iters=iters)
    st = _slab(n, p, r, gate, iters)
    upload_boundary(st, b)
    _upload_records(st, recs, gate)
    S = O.replay(O.dequantize(b), _oracle_records(recs, gate))
    if fused:
        tok = _token(rng, n, gate)
        o = torch.empty((n, 128), device=DEV)
        lq.leapquant_decode_close(st, nrec, *[_dev(tok[x]) for x in ("q", "k", "v", "beta", "alpha")], o)
        t64 = {k: v.astype(np.float64) for k, v in tok.items()}
        o_ref, S, _ = O.step(S, *[t64[x] for x in ("q", "k", "v", "beta", "alpha")], _gate(gate))
    else:
        lq.leapquant_window_close(st, length)
    torch.cuda.synchronize()
    if fused:
        P.assert_close(to_np(o), o_ref, "o_t")
    stats = P.compare_dense_boundary(boundary_np(st), S.astype(np.float32), r, iters, 0,
                                     f"dense {'decode_close' if fused else 'window_close'}")
    print(stats)


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("name,n,steps", [("gdn_layer_h32_b64", 16, 96), ("kda_h32_b128", 16, 96)])
def test_oracle_forced_windows(name, n, steps, fused):
    """Whole windows of the synthetic workloads with dense tokens (2
    iterations); every GPU window starts from the oracle's boundary."""
    iters = 2
    cfg, S0, tok = _workload(name, n, steps)
    S0n = S0.numpy()
    tokn = {k: v.numpy().astype(np.float64) for k, v in tok.items()}
    o_ref, bounds = O.run_windowed(S0n, tokn, cfg.p, cfg.r, _gate(cfg.gate), O.DENSE_COMP, iters=iters)
    tokd = {k: v.to(DEV) for k, v in tok.items()}
    st = _slab(n, cfg.p, cfg.r, cfg.gate, iters)
    out = torch.empty((steps, n, 128), device=DEV)
    flips = 0
    for w in range(steps // cfg.p):
        upload_boundary(st, bounds[w])
        run_window(st, tokd, w * cfg.p, cfg.p, out, fused=fused)
        torch.cuda.synchronize()
        sl = slice(w * cfg.p, (w + 1) * cfg.p)
        P.assert_close(to_np(out[sl]), o_ref[sl], f"{name} window {w} outputs")
        _, _, S_end, _ = O.window(bounds[w], tokn, w * cfg.p, cfg.p, _gate(cfg.gate), cfg.r, O.DENSE_COMP,
                                  iters=iters)
        s = P.compare_dense_boundary(boundary_np(st), S_end.astype(np.float32), cfg.r, iters, 0,
                                     f"{name} boundary {w + 1}")
        flips += s["flips"]
    print(f"{name} dense: {flips} flipped codes")


def test_zero_iterations_decode_matches_row_extraction():
    """A boundary with one-hot keys decodes exactly as the same boundary in
    row form: the decode kernels give bit-identical o_t and u_t."""
    rng = np.random.default_rng(3400)
    n, p, t, r = 19, 16, 9, 4
    b, recs = _random_window_inputs(rng, n, p, t, "gdn", r, dense_iters=0)
    tok = {k: _dev(v) for k, v in _token(rng, n, "gdn").items()}
    outs = []
    for dense in (False, True):
        st = _slab(n, p, r, "gdn", 0) if dense else lq.LeapQuantState(n, p, r, "gdn", DEV)
        upload_boundary(st, b)
        _upload_records(st, recs, "gdn")
        o = torch.empty((n, 128), device=DEV)
        lq.leapquant_decode_step(st, t, tok["q"], tok["k"], tok["v"], tok["beta"], tok["alpha"], o)
        torch.cuda.synchronize()
        outs.append((to_np(o), to_np(st.buf_u[:, t])))
    np.testing.assert_array_equal(outs[0][0], outs[1][0])
    np.testing.assert_array_equal(outs[0][1], outs[1][1])
