"""Parity of the "BF16 + per-window" row ([EL] Table 2) on the HIP path.

A dense bf16 boundary state B stays fixed for a window; the tokens are
buffered in fp32 records; the close stores Gamma * B + K_w U rounded to
bf16.  The oracle is `window_bf16` / `step` from the same boundary and
records.  The close's rounding to bf16 is decided from an fp32 rebuild on
the GPU and an fp64 one in the oracle: they may differ by one bf16 step
where the value sits at a rounding tie, plus the fp32 error of the rebuild's
terms (Gamma B and the p products k~_i u_i), which dominates where they
cancel.
"""
import numpy as np
import pytest
import torch

import recurrent_state_quant_amd as lq
from oracle import leapquant_oracle as O
from tests import parity as P
from tests.gpu_run import to_np
from tests.test_gpu_parity import (_bf16_ulp, _dev, _gate, _oracle_records, _random_window_inputs,
                                   _states_with_outliers, _token, _upload_records, _workload)

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    lq.load()
    yield
    torch.cuda.synchronize()


def _bf16_dev(B64):
    B = torch.as_tensor(B64).to(torch.float32).to(torch.bfloat16).to(DEV)
    assert torch.equal(B.double().cpu(), torch.as_tensor(B64))   # exact upload
    return B


def _check_close(Bg, S_ref, terms, what):
    ref = O.round_bf16(S_ref)
    d = np.abs(Bg - ref)
    bound = _bf16_ulp(ref) * 1.0001 + 64 * 2.0 ** -24 * terms
    worst = np.unravel_index(np.argmax(d - bound), d.shape)
    assert np.all(d <= bound), (what, worst, float(Bg[worst]), float(ref[worst]), float(bound[worst]))
    assert (d > 0).mean() <= 1e-3, (what, float((d > 0).mean()))


def _terms(B64, recs, gate):
    """|Gamma * B| + sum_i |K_w[i] u_i^T|: the magnitudes the fp32 rebuild adds."""
    n = B64.shape[0]
    P_ = np.ones((n, 128))
    acc = np.zeros_like(B64)
    for a, kt, u in reversed(recs):
        acc += np.abs((P_ * kt.astype(np.float64))[:, :, None] * u.astype(np.float64)[:, None, :])
        P_ = P_ * np.broadcast_to(a.astype(np.float64).reshape(n, -1), (n, 128))
    return acc + np.abs(P_[:, :, None] * B64)


@pytest.mark.parametrize("gate", ["gdn", "kda"])
@pytest.mark.parametrize("p,t", [(1, 0), (16, 0), (16, 9), (16, 15), (32, 20), (64, 63)])
def test_decode_step_entry(gate, p, t):
    rng = np.random.default_rng(6000 + 100 * p + t + (gate == "kda"))
    n = 19
    _, recs = _random_window_inputs(rng, n, p, t, gate, 0)
    B64 = O.round_bf16(_states_with_outliers(rng, n))
    st = lq.LeapQuantState(n, p, 0, gate, DEV)
    _upload_records(st, recs, gate)
    B = _bf16_dev(B64)
    tok = _token(rng, n, gate)
    o = torch.empty((n, 128), device=DEV)
    lq.leapquant_bf16w_decode_step(st, B, t, *[_dev(tok[x]) for x in ("q", "k", "v", "beta", "alpha")], o)
    torch.cuda.synchronize()
    S_prev = O.replay(B64, _oracle_records(recs, gate))
    t64 = {k: v.astype(np.float64) for k, v in tok.items()}
    o_ref, _, (_, kt, u) = O.step(S_prev, *[t64[x] for x in ("q", "k", "v", "beta", "alpha")], _gate(gate))
    P.assert_close(to_np(o), o_ref, "bf16w o_t")
    P.assert_close(to_np(st.buf_u[:, t]), u, "bf16w u_t")
    P.assert_close(to_np(st.buf_k[:, t]), kt, "bf16w k~_t", rtol=1e-6, atol=0)
    assert torch.equal(B.double().cpu(), torch.as_tensor(B64)), "the decode step wrote B"


@pytest.mark.parametrize("gate", ["gdn", "kda"])
@pytest.mark.parametrize("p,length", [(1, 1), (16, 16), (16, 5), (32, 32), (64, 37)])
def test_window_close_entry(gate, p, length):
    rng = np.random.default_rng(6100 + 7 * p + length + (gate == "kda"))
    n = 21
    _, recs = _random_window_inputs(rng, n, p, length, gate, 0)
    B64 = O.round_bf16(_states_with_outliers(rng, n))
    st = lq.LeapQuantState(n, p, 0, gate, DEV)
    _upload_records(st, recs, gate)
    B = _bf16_dev(B64)
    lq.leapquant_bf16w_window_close(st, B, length)
    torch.cuda.synchronize()
    S = O.replay(B64, _oracle_records(recs, gate))
    _check_close(B.double().cpu().numpy(), S, _terms(B64, recs, gate), f"bf16w close p={p} len={length}")


@pytest.mark.parametrize("name,n,steps", [("gdn_layer_h32_b64", 16, 64), ("kda_h32_b128", 16, 64)])
def test_oracle_forced_windows(name, n, steps):
    """Whole windows of the synthetic workloads; every GPU window starts from
    the oracle's bf16 boundary."""
    cfg, S0, tok = _workload(name, n, steps)
    tokn = {k: v.numpy().astype(np.float64) for k, v in tok.items()}
    tokd = {k: v.to(DEV) for k, v in tok.items()}
    gate = _gate(cfg.gate)
    o_ref, bounds = O.run_windowed_bf16(S0.numpy(), tokn, cfg.p, gate)
    st = lq.LeapQuantState(n, cfg.p, 0, cfg.gate, DEV)
    out = torch.empty((n, 128), device=DEV)
    for w in range(steps // cfg.p):
        B = _bf16_dev(bounds[w])
        for j in range(cfg.p):
            t = w * cfg.p + j
            lq.leapquant_bf16w_decode_step(st, B, j, *[tokd[x][t] for x in ("q", "k", "v", "beta", "alpha")], out)
            torch.cuda.synchronize()
            P.assert_close(to_np(out), o_ref[t], f"{name} token {t}")
        lq.leapquant_bf16w_window_close(st, B, cfg.p)
        torch.cuda.synchronize()
        _, recs, S_end, _ = O.window_bf16(bounds[w], tokn, w * cfg.p, cfg.p, gate)
        recs32 = [(np.asarray(d[:, 0] if cfg.gate == "gdn" else d, np.float32), kt.astype(np.float32),
                   u.astype(np.float32)) for d, kt, u in recs]
        _check_close(B.double().cpu().numpy(), S_end, _terms(bounds[w], recs32, cfg.gate), f"{name} window {w}")
