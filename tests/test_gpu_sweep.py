"""Seeded random sweep over the entry points' configuration space.

Each of 200 cases draws a gate, window length p, compensator count r, flags
(no smoothing, no delta correction, dense compensator tokens with 0-3
subspace iterations), slab size n and window position, then runs one entry
point (decode step, fused decode_close, window close, quantize) on random
boundary states and records and compares it with the oracle under the same
rules as the entry-point tests.  Slabs of 1 to 300 states take the two-wave
decode kernel; 60 further cases tile slabs of 4,097 to 6,000 states from 13
distinct states, so that the decode step and the fused close run the
one-wave decode kernel and large launches.  The cases are fixed by the
seed, so a failure names a reproducible configuration.
"""
import os

import numpy as np
import pytest
import torch

import recurrent_state_quant_amd as lq
from oracle import leapquant_oracle as O
from tests import parity as P
from tests.gpu_run import boundary_np, to_np, upload_boundary
from tests.test_gpu_parity import (_dev, _gate, _oracle_records, _random_window_inputs, _states_with_outliers,
                                   _token, _upload_records)

pytestmark = pytest.mark.gpu
DEV = "cuda"
# Wider runs of the same generators: LQ_SWEEP_SCALE multiplies the case
# counts, LQ_SWEEP_SEED moves every seed to another family (0, the default:
# the committed cases).
SCALE = int(os.environ.get("LQ_SWEEP_SCALE", "1"))
SEED_SHIFT = 10_000_000 * int(os.environ.get("LQ_SWEEP_SEED", "0"))
N_CASES = 200 * SCALE


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    lq.load()
    yield
    torch.cuda.synchronize()


def _case(i):
    rng = np.random.default_rng(90000 + i + SEED_SHIFT)
    gate = ["gdn", "kda"][rng.integers(2)]
    p = int(rng.choice([1, 2, 3, 5, 8, 16, 17, 31, 32, 48, 64]))
    r = int(rng.choice([0, 1, 2, 4, 7, 8, 16]))
    flags = 0
    if rng.random() < 0.25:
        flags |= O.NO_SMOOTH
    if rng.random() < 0.25:
        flags |= O.NO_DELTA
    iters = None
    if r > 0 and rng.random() < 0.35:
        iters = int(rng.integers(0, 4))
    n = int(rng.choice([1, 2, 7, 19, 33, 129, 300]))
    entry = ["decode", "decode_close", "close", "quantize"][rng.integers(4)]
    t = int(rng.integers(0, p))
    return rng, gate, p, r, flags, iters, n, entry, t


@pytest.mark.parametrize("i", range(N_CASES))
def test_sweep(i):
    rng, gate, p, r, flags, iters, n, entry, t = _case(i)
    what = f"case {i}: {entry} gate={gate} p={p} r={r} flags={flags} iters={iters} n={n} t={t}"
    print(what, flush=True)
    dense = iters is not None
    qflags = flags & O.NO_SMOOTH
    lqflags = (lq.LQ_NO_SMOOTH if flags & O.NO_SMOOTH else 0) | (lq.LQ_NO_DELTA if flags & O.NO_DELTA else 0) | \
        (lq.LQ_DENSE_COMP if dense else 0)
    st = lq.LeapQuantState(n, p, r, gate, DEV, flags=lqflags, comp_iters=iters or 0)

    def check_boundary(S):
        S32 = S.astype(np.float32)
        gb = boundary_np(st)
        if dense:
            P.compare_dense_boundary(gb, S32, r, iters, qflags, what)
        else:
            P.compare_boundary(gb, O.quantize(S32, r, qflags), S32, r, what)

    if entry == "quantize":
        S = _states_with_outliers(rng, n)
        lq.leapquant_quantize_state(st, _dev(S))
        torch.cuda.synchronize()
        if dense:
            P.compare_dense_boundary(boundary_np(st), S, r, iters, qflags, what)
        else:
            P.compare_boundary(boundary_np(st), O.quantize(S, r, qflags), S, r, what, exact=True)
        return
    nrec = {"decode": t, "decode_close": t, "close": t + 1}[entry]
    b, recs = _random_window_inputs(rng, n, p, nrec, gate, r, dense_iters=iters)
    upload_boundary(st, b)
    _upload_records(st, recs, gate)
    S_prev = O.replay(O.dequantize(b), _oracle_records(recs, gate))
    if entry == "close":
        lq.leapquant_window_close(st, nrec)
        torch.cuda.synchronize()
        check_boundary(S_prev)
        return
    tok = _token(rng, n, gate)
    o = torch.empty((n, 128), device=DEV)
    call = lq.leapquant_decode_step if entry == "decode" else lq.leapquant_decode_close
    call(st, t, *[_dev(tok[x]) for x in ("q", "k", "v", "beta", "alpha")], o)
    torch.cuda.synchronize()
    t64 = {k: v.astype(np.float64) for k, v in tok.items()}
    o_ref, S_t, (_, _, u) = O.step(S_prev, *[t64[x] for x in ("q", "k", "v", "beta", "alpha")], _gate(gate),
                                   flags & O.NO_DELTA)
    P.assert_close(to_np(o), o_ref, what + " o_t")
    if entry == "decode":
        P.assert_close(to_np(st.buf_u[:, t]), u, what + " u_t")
    else:
        check_boundary(S_t)


# Slabs above 4,096 states take the one-wave decode kernel (the throughput
# workload's): a slab is tiled from m distinct states, so that the oracle
# computes m states while every slot is still compared.
N_LARGE = 60 * SCALE


def _large_case(i):
    rng = np.random.default_rng(5150000 + 11 * i + SEED_SHIFT)
    gate = ["gdn", "kda"][rng.integers(2)]
    p = int(rng.choice([1, 2, 3, 5, 8, 16, 17, 31, 32, 48, 64]))
    r = int(rng.choice([0, 1, 2, 4, 7, 8, 16]))
    flags = 0
    if rng.random() < 0.25:
        flags |= O.NO_SMOOTH
    if rng.random() < 0.25:
        flags |= O.NO_DELTA
    iters = None
    if r > 0 and rng.random() < 0.35:
        iters = int(rng.integers(0, 4))
    n = int(rng.choice([4097, 4609, 6000]))
    entry = ["decode", "decode_close"][rng.integers(2)]
    t = int(rng.integers(0, p))
    return rng, gate, p, r, flags, iters, n, entry, t


@pytest.mark.parametrize("i", range(N_LARGE))
def test_sweep_large_slab(i):
    rng, gate, p, r, flags, iters, n, entry, t = _large_case(i)
    what = f"large case {i}: {entry} gate={gate} p={p} r={r} flags={flags} iters={iters} n={n} t={t}"
    print(what, flush=True)
    m = 13
    dense = iters is not None
    lqflags = (lq.LQ_NO_SMOOTH if flags & O.NO_SMOOTH else 0) | (lq.LQ_NO_DELTA if flags & O.NO_DELTA else 0) | \
        (lq.LQ_DENSE_COMP if dense else 0)
    b, recs = _random_window_inputs(rng, m, p, t, gate, r, dense_iters=iters)
    tok = _token(rng, m, gate)
    tile = np.arange(n) % m
    st = lq.LeapQuantState(n, p, r, gate, DEV, flags=lqflags, comp_iters=iters or 0)
    upload_boundary(st, {k: v[tile] for k, v in b.items()})
    _upload_records(st, [(a[tile], kt[tile], u[tile]) for a, kt, u in recs], gate)
    o = torch.empty((n, 128), device=DEV)
    call = lq.leapquant_decode_step if entry == "decode" else lq.leapquant_decode_close
    call(st, t, *[_dev(tok[x][tile]) for x in ("q", "k", "v", "beta", "alpha")], o)
    torch.cuda.synchronize()
    S_prev = O.replay(O.dequantize(b), _oracle_records(recs, gate))
    t64 = {k: v.astype(np.float64) for k, v in tok.items()}
    o_ref, S_t, (_, _, u) = O.step(S_prev, *[t64[x] for x in ("q", "k", "v", "beta", "alpha")], _gate(gate),
                                   flags & O.NO_DELTA)
    P.assert_close(to_np(o), o_ref[tile], what + " o_t")
    if entry == "decode":
        P.assert_close(to_np(st.buf_u[:, t]), u[tile], what + " u_t")
        return
    g = boundary_np(st)
    S32 = S_t.astype(np.float32)
    for first in (0, (n // 2) // m * m, (n - m) // m * m):   # blocks of slots holding the m states in order
        gs = {k: v[first:first + m] for k, v in g.items()}
        if dense:
            P.compare_dense_boundary(gs, S32, r, iters, flags & O.NO_SMOOTH, what)
        else:
            P.compare_boundary(gs, O.quantize(S32, r, flags & O.NO_SMOOTH), S32, r, what)
