"""Seeded random sweep of the continuous-batching entry points.

Each of 300 cases draws a gate, window length p, compensator count r, flags
(no delta correction, no smoothing, dense compensator tokens), a slab tiled
from m distinct states (up to 4,500 slots, so both decode kernels run) and
a position per slot that may fall outside the valid range, then runs one of
decode_step_slots, decode_close_slots, window_close_slots,
decode_close_list or window_close_list (the lists are random subsets of
distinct slots in random order, possibly empty).  Every active slot is
compared with the oracle at its own position; idle slots, and slots left out
of a list, must keep their o row (pre-filled with NaN) and their boundary
state bit for bit.
"""
import os

import numpy as np
import pytest
import torch

import recurrent_state_quant_amd as lq
from oracle import leapquant_oracle as O
from tests import parity as P
from tests.gpu_run import boundary_np, to_np, upload_boundary
from tests.test_gpu_parity import _dev, _gate, _oracle_records, _random_window_inputs, _token, _upload_records

pytestmark = pytest.mark.gpu
DEV = "cuda"
# Wider runs of the same generators: LQ_SWEEP_SCALE multiplies the case
# counts, LQ_SWEEP_SEED moves every seed to another family (0, the default:
# the committed cases).
SCALE = int(os.environ.get("LQ_SWEEP_SCALE", "1"))
SEED_SHIFT = 10_000_000 * int(os.environ.get("LQ_SWEEP_SEED", "0"))
N_CASES = 300 * SCALE


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    lq.load()
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("i", range(N_CASES))
def test_slots(i):
    rng = np.random.default_rng(6160000 + 7 * i + SEED_SHIFT)
    gate = ["gdn", "kda"][rng.integers(2)]
    p = int(rng.choice([1, 2, 3, 5, 8, 16, 17, 32, 64]))
    r = int(rng.choice([0, 2, 4, 8, 16]))
    flags = (O.NO_DELTA if rng.random() < 0.2 else 0) | (O.NO_SMOOTH if rng.random() < 0.2 else 0)
    qflags = flags & O.NO_SMOOTH
    iters = int(rng.integers(0, 3)) if (r > 0 and rng.random() < 0.3) else None
    entry = ["step", "close", "window", "close_list", "window_list"][rng.integers(5)]
    m = int(rng.choice([3, 7, 13]))
    n = int(rng.choice([m, 50, 300, 4500]))
    what = f"slots case {i}: {entry} gate={gate} p={p} r={r} flags={flags} iters={iters} m={m} n={n}"
    print(what, flush=True)
    dense = iters is not None
    lqflags = (lq.LQ_NO_DELTA if flags & O.NO_DELTA else 0) | (lq.LQ_NO_SMOOTH if qflags else 0) | \
        (lq.LQ_DENSE_COMP if dense else 0)
    win = entry.startswith("window")
    nrec = p if win else p - 1
    b, recs = _random_window_inputs(rng, m, p, nrec, gate, r, dense_iters=iters)
    tok = _token(rng, m, gate)
    tile = np.arange(n) % m
    lo, hi = (1, p + 1) if win else (0, p)
    pos = rng.integers(lo - 1, hi + 1, n).astype(np.int32)   # includes out-of-range (idle) values
    listed = np.ones(n, bool)
    if entry.endswith("_list"):
        sel = rng.choice(n, int(rng.integers(0, n + 1)), replace=False).astype(np.int32)
        listed[:] = False
        listed[sel] = True
        sl_d = torch.as_tensor(rng.permutation(sel), device=DEV)
    st = lq.LeapQuantState(n, p, r, gate, DEV, flags=lqflags, comp_iters=iters or 0)
    upload_boundary(st, {k: v[tile] for k, v in b.items()})
    _upload_records(st, [(a[tile], kt[tile], u[tile]) for a, kt, u in recs], gate)
    pos_d = torch.as_tensor(pos, device=DEV)
    o = torch.full((n, 128), float("nan"), device=DEV)
    args = [_dev(tok[x][tile]) for x in ("q", "k", "v", "beta", "alpha")]
    if entry == "step":
        lq.leapquant_decode_step_slots(st, pos_d, *args, o)
    elif entry == "close":
        lq.leapquant_decode_close_slots(st, pos_d, *args, o)
    elif entry == "window":
        lq.leapquant_window_close_slots(st, pos_d)
    elif entry == "close_list":
        lq.leapquant_decode_close_list(st, pos_d, sl_d, *args, o)
    else:
        lq.leapquant_window_close_list(st, pos_d, sl_d)
    torch.cuda.synchronize()
    active = (pos >= lo) & (pos < hi) & listed
    og = to_np(o)
    if not win:
        assert np.isnan(og[~active]).all(), what + ": idle slots wrote o"
    g = boundary_np(st)
    t64 = {k: v.astype(np.float64) for k, v in tok.items()}
    for t in np.unique(pos[active]):
        sl = np.nonzero(active & (pos == t))[0]
        j = np.unique(tile[sl])
        B = O.dequantize({k: v[j] for k, v in b.items()})
        S_prev = O.replay(B, _oracle_records([(a[j], kt[j], u[j]) for a, kt, u in recs[:t]], gate))
        if win:
            S_end = S_prev
        else:
            o_ref, S_end, (_, _, u) = O.step(S_prev, *[t64[x][j] for x in ("q", "k", "v", "beta", "alpha")],
                                             _gate(gate), flags & O.NO_DELTA)
            ref_of = {int(x): y for x, y in zip(j, o_ref)}
            P.assert_close(og[sl], np.stack([ref_of[int(x)] for x in tile[sl]]), f"{what} t={t} o")
            if entry == "step":
                uref = {int(x): y for x, y in zip(j, u)}
                P.assert_close(to_np(st.buf_u[torch.as_tensor(sl, device=DEV), int(t)]),
                               np.stack([uref[int(x)] for x in tile[sl]]), f"{what} t={t} u")
        if entry != "step":
            # one representative slot per distinct state
            first = {}
            for s_ in sl:
                first.setdefault(int(tile[s_]), s_)
            rep = np.array([first[int(x)] for x in j])
            gs = {k: v[rep] for k, v in g.items()}
            S32 = S_end.astype(np.float32)
            if dense:
                P.compare_dense_boundary(gs, S32, r, iters, qflags, f"{what} t={t}")
            else:
                P.compare_boundary(gs, O.quantize(S32, r, qflags), S32, r, f"{what} t={t}")
    # untouched slots keep the boundary they had
    idle = np.nonzero(~active)[0]
    if entry == "step":
        idle = np.arange(n)   # a decode step leaves every boundary as it is
    if len(idle):
        for k, v in g.items():
            np.testing.assert_array_equal(v[idle], np.asarray(b[k])[tile[idle]], err_msg=f"{what}: idle {k}")
