"""Seeded random sweep of the dense-state baselines ([EL] Table 2).

Each of 160 cases draws a gate, with or without the delta correction, a
slab of 1 to 4,500 states tiled from m distinct ones (the oracle computes m,
every slot is compared), a window length p and position, then runs one of:
  - the FP32 per-step decode over 1 to 6 tokens;
  - one BF16 per-step token;
  - a "BF16 + per-window" decode step at position t;
  - a "BF16 + per-window" close over len records.
The comparisons are those of the fixed-grid tests: outputs, u and the fp32
state within the fp32 tolerance; a bf16 state within one bf16 step plus the
fp32 error of the terms it sums, with at most 0.1% of elements off the
oracle's rounding.
"""
import os

import numpy as np
import pytest
import torch

import recurrent_state_quant_amd as lq
from oracle import leapquant_oracle as O
from tests import parity as P
from tests.gpu_run import to_np
from tests.test_gpu_parity import (_bf16_ulp, _dev, _gate, _oracle_records, _random_window_inputs,
                                   _states_with_outliers, _token, _upload_records)

pytestmark = pytest.mark.gpu
DEV = "cuda"
# Wider runs of the same generators: LQ_SWEEP_SCALE multiplies the case
# counts, LQ_SWEEP_SEED moves every seed to another family (0, the default:
# the committed cases).
SCALE = int(os.environ.get("LQ_SWEEP_SCALE", "1"))
SEED_SHIFT = 10_000_000 * int(os.environ.get("LQ_SWEEP_SEED", "0"))
N_CASES = 160 * SCALE
KEYS = ("q", "k", "v", "beta", "alpha")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    lq.load()
    yield
    torch.cuda.synchronize()


def _check_bf16(Sg, S_ref, terms, what):
    d = np.abs(Sg - S_ref)
    bound = _bf16_ulp(S_ref) * 1.0001 + 64 * 2.0 ** -24 * terms
    worst = np.unravel_index(np.argmax(d - bound), d.shape)
    assert np.all(d <= bound), (what, worst, float(Sg[worst]), float(S_ref[worst]), float(bound[worst]))
    assert (d > 0).mean() <= 1e-3, (what, float((d > 0).mean()))


def _bf16_dev(B64, tile):
    B = torch.as_tensor(B64[tile]).to(torch.float32).to(torch.bfloat16).to(DEV)
    assert torch.equal(B.double().cpu(), torch.as_tensor(B64[tile]))   # exact upload
    return B


@pytest.mark.parametrize("i", range(N_CASES))
def test_baselines(i):
    rng = np.random.default_rng(7270000 + 13 * i + SEED_SHIFT)
    gate = ["gdn", "kda"][rng.integers(2)]
    flags = O.NO_DELTA if rng.random() < 0.3 else 0
    entry = ["fp32_steps", "bf16_step", "bf16w_decode", "bf16w_close"][rng.integers(4)]
    m = int(rng.choice([1, 5, 13]))
    n = int(rng.choice([m, 33, 300, 4500]))
    p = int(rng.choice([1, 2, 5, 16, 17, 32, 64]))
    tile = np.arange(n) % m
    what = f"baselines case {i}: {entry} gate={gate} flags={flags} m={m} n={n} p={p}"
    print(what, flush=True)
    lqflags = lq.LQ_NO_DELTA if flags else 0
    g = _gate(gate)

    if entry == "fp32_steps":
        T = int(rng.integers(1, 7))
        S0 = _states_with_outliers(rng, m)
        S = _dev(S0[tile])
        S_ref = S0.astype(np.float64)
        o = torch.empty((n, 128), device=DEV)
        for t in range(T):
            tok = _token(rng, m, gate)
            lq.leapquant_dense_step(S, gate, *(_dev(tok[x][tile]) for x in KEYS), o, flags=lqflags)
            t64 = {x: y.astype(np.float64) for x, y in tok.items()}
            o_ref, S_ref, _ = O.step(S_ref, *[t64[x] for x in KEYS], g, flags)
            torch.cuda.synchronize()
            P.assert_close(to_np(o), o_ref[tile], f"{what} o_{t}")
        P.assert_close(to_np(S), S_ref[tile], what + " state")
        return

    if entry == "bf16_step":
        S0 = O.round_bf16(_states_with_outliers(rng, m))
        tok = _token(rng, m, gate)
        S = _bf16_dev(S0, tile)
        o = torch.empty((n, 128), device=DEV)
        lq.leapquant_dense_step(S, gate, *(_dev(tok[x][tile]) for x in KEYS), o, flags=lqflags)
        torch.cuda.synchronize()
        t64 = {x: y.astype(np.float64) for x, y in tok.items()}
        o_ref, S_ref = O.step_dense_bf16(S0, *[t64[x] for x in KEYS], g, flags)
        P.assert_close(to_np(o), o_ref[tile], what + " o")
        d_, kt_, _ = O.transition(g, t64["k"], t64["beta"], t64["alpha"], 128)
        _, _, (_, _, u_) = O.step(S0, *[t64[x] for x in KEYS], g, flags)
        terms = np.abs(d_[:, :, None] * S0) + np.abs(kt_[:, :, None] * u_[:, None, :])
        _check_bf16(S.double().cpu().numpy(), S_ref[tile], terms[tile], what + " state")
        return

    B64 = O.round_bf16(_states_with_outliers(rng, m))
    st = lq.LeapQuantState(n, p, 0, gate, DEV, flags=lqflags)
    B = _bf16_dev(B64, tile)
    if entry == "bf16w_decode":
        t = int(rng.integers(0, p))
        _, recs = _random_window_inputs(rng, m, p, t, gate, 0)
        _upload_records(st, [(a[tile], kt[tile], u[tile]) for a, kt, u in recs], gate)
        tok = _token(rng, m, gate)
        o = torch.empty((n, 128), device=DEV)
        lq.leapquant_bf16w_decode_step(st, B, t, *[_dev(tok[x][tile]) for x in KEYS], o)
        torch.cuda.synchronize()
        S_prev = O.replay(B64, _oracle_records(recs, gate))
        t64 = {k: v.astype(np.float64) for k, v in tok.items()}
        o_ref, _, (_, kt, u) = O.step(S_prev, *[t64[x] for x in KEYS], g, flags)
        P.assert_close(to_np(o), o_ref[tile], f"{what} t={t} o_t")
        P.assert_close(to_np(st.buf_u[:, t]), u[tile], f"{what} t={t} u_t")
        P.assert_close(to_np(st.buf_k[:, t]), kt[tile], f"{what} t={t} k~_t", rtol=1e-6, atol=0)
        assert torch.equal(B.double().cpu(), torch.as_tensor(B64[tile])), what + ": the decode step wrote B"
        return

    length = int(rng.integers(1, p + 1))
    _, recs = _random_window_inputs(rng, m, p, length, gate, 0)
    _upload_records(st, [(a[tile], kt[tile], u[tile]) for a, kt, u in recs], gate)
    lq.leapquant_bf16w_window_close(st, B, length)
    torch.cuda.synchronize()
    S = O.replay(B64, _oracle_records(recs, gate))
    # |Gamma * B| + sum_i |K_w[i] u_i^T|: the magnitudes the fp32 rebuild adds
    Pd = np.ones((m, 128))
    terms = np.zeros_like(B64)
    for a, kt, u in reversed(recs):
        terms += np.abs((Pd * kt.astype(np.float64))[:, :, None] * u.astype(np.float64)[:, None, :])
        Pd = Pd * np.broadcast_to(a.astype(np.float64).reshape(m, -1), (m, 128))
    terms += np.abs(Pd[:, :, None] * B64)
    _check_bf16(B.double().cpu().numpy(), O.round_bf16(S)[tile], terms[tile], f"{what} len={length}")
