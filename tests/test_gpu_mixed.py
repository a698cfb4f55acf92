"""leapquant_decode_step_close_list (one continuous-batching token in one
launch) against the two calls it stands for, bit for bit: decode_step_slots
over the positions with p - 1 made idle, then decode_close_list over the
listed slots that sit at p - 1.  Both calls are checked against the oracle
elsewhere (tests/test_gpu_slot_list.py, tests/test_gpu_sweep_slots.py).

Cases cross the single-launch shapes (more than 4,096 slots, 4 <= p <= 16,
r <= 8) with the two-launch path (smaller slabs, p = 2 and 32, r = 16), both gates, slab sizes that are not multiples of
the four slots a decode workgroup takes, idle and out-of-range positions,
listed slots not at p - 1 (skipped), unlisted slots at p - 1 (untouched),
ids outside [0, n) and an empty list.
"""
import numpy as np
import pytest
import torch

import recurrent_state_quant_amd as lq
from oracle import leapquant_oracle as O
from tests.gpu_run import upload_boundary
from tests.test_gpu_parity import _random_window_inputs, _upload_records, _token, _dev

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    lq.load()
    yield
    torch.cuda.synchronize()


def _slab(n, m, p, r, gate, b, recs, tile):
    st = lq.LeapQuantState(n, p, r, gate, DEV)
    upload_boundary(st, {k: v[tile] for k, v in b.items()})
    _upload_records(st, [(a[tile], kt[tile], u[tile]) for a, kt, u in recs], gate)
    return st


@pytest.mark.parametrize("gate", ["gdn", "kda"])
@pytest.mark.parametrize("n,p,r", [(4097, 16, 4), (4099, 16, 8), (8190, 16, 4), (5001, 16, 0), (13, 16, 4),
                                   (301, 16, 4), (4201, 32, 4), (4400, 16, 16), (4500, 4, 4), (4300, 2, 4)])
@pytest.mark.parametrize("listing", ["all", "partial", "empty"])
def test_mixed_equals_the_two_calls(gate, n, p, r, listing):
    rng = np.random.default_rng(9000 + n + 7 * p + r + 3 * (gate == "kda") + len(listing))
    m = 11
    b, recs = _random_window_inputs(rng, m, p, p - 1, gate, r)
    tok = _token(rng, m, gate)
    tile = np.arange(n) % m
    pos = rng.integers(0, p, n).astype(np.int32)
    pos[rng.random(n) < 0.25] = p - 1                 # plenty of closing slots
    pos[rng.random(n) < 0.05] = -1                    # idle
    pos[rng.random(n) < 0.03] = p                     # out of range: idle
    last = np.nonzero(pos == p - 1)[0]
    if listing == "all":
        lst = last.copy()
    elif listing == "partial":
        lst = last[rng.random(len(last)) < 0.7]       # some closing slots unlisted
        extra = np.nonzero((pos >= 0) & (pos < p - 1))[0]
        lst = np.concatenate([lst, rng.choice(extra, min(5, len(extra)), replace=False), [n, n + 7, -3]])
    else:
        lst = np.zeros(0, np.int64)
    lst = rng.permutation(lst).astype(np.int32)
    args = [_dev(tok[x][tile]) for x in ("q", "k", "v", "beta", "alpha")]

    a = _slab(n, m, p, r, gate, b, recs, tile)
    bb = _slab(n, m, p, r, gate, b, recs, tile)
    oa = torch.full((n, 128), float("nan"), device=DEV)
    ob = oa.clone()
    pos_d = torch.as_tensor(pos, device=DEV)
    lq.leapquant_decode_step_close_list(a, pos_d, torch.as_tensor(lst, device=DEV), *args, oa)

    step_pos = torch.as_tensor(np.where(pos == p - 1, -1, pos).astype(np.int32), device=DEV)
    lq.leapquant_decode_step_slots(bb, step_pos, *args, ob)
    ref_list = lst[(lst >= 0) & (lst < n)]
    ref_list = ref_list[pos[ref_list] == p - 1].astype(np.int32)
    lq.leapquant_decode_close_list(bb, pos_d, torch.as_tensor(ref_list, device=DEV), *args, ob)
    torch.cuda.synchronize()

    assert torch.equal(torch.isnan(oa), torch.isnan(ob))
    torch.testing.assert_close(oa, ob, rtol=0, atol=0, equal_nan=True)
    for k in ("codes", "row_scale", "col_scale", "comp_idx", "comp_val", "buf_gate", "buf_k", "buf_u"):
        torch.testing.assert_close(getattr(a, k), getattr(bb, k), rtol=0, atol=0, equal_nan=True,
                                   msg=lambda s, k=k: f"{k}: {s}")
    # something happened: decoded and closed slots exist in every case but "empty"
    decoded = (pos >= 0) & (pos < p - 1)
    assert not torch.isnan(oa[torch.as_tensor(decoded, device=DEV)]).any()
    if listing != "empty" and len(ref_list):
        assert not torch.isnan(oa[torch.as_tensor(ref_list.astype(np.int64), device=DEV)]).any()


@pytest.mark.parametrize("gate", ["gdn", "kda"])
def test_two_stream_schedule_equals_single_launch(gate):
    """The continuous-batching schedule with the closing slots' closes on a
    second stream beside the other slots' decode step (decode_close_list and
    decode_step_slots on disjoint slots, joined by events before the next
    token) gives the single-launch results bit for bit, token after token."""
    rng = np.random.default_rng(9100 + (gate == "kda"))
    n, p, r, m, L = 4500, 8, 4, 11, 2
    T = 2 * p + 3
    b, recs = _random_window_inputs(rng, m, p, p - 1, gate, r)
    tile = np.arange(n) % m
    phase = rng.integers(0, p, n).astype(np.int32)
    toks = [_token(rng, m, gate) for _ in range(T)]
    args = [[_dev(tk[x][tile]) for x in ("q", "k", "v", "beta", "alpha")] for tk in toks]
    a = [_slab(n, m, p, r, gate, b, recs, tile) for _ in range(L)]
    bb = [_slab(n, m, p, r, gate, b, recs, tile) for _ in range(L)]
    oa = [[torch.full((n, 128), float("nan"), device=DEV) for _ in range(L)] for _ in range(T)]
    ob = [[x.clone() for x in row] for row in oa]
    pos = [(phase + t) % p for t in range(T)]
    pos_d = [torch.as_tensor(x, device=DEV) for x in pos]
    lst = [torch.as_tensor(np.nonzero(x == p - 1)[0].astype(np.int32), device=DEV) for x in pos]
    step = [torch.as_tensor(np.where(x == p - 1, -1, x).astype(np.int32), device=DEV) for x in pos]
    for t in range(T):
        for l in range(L):
            lq.leapquant_decode_step_close_list(a[l], pos_d[t], lst[t], *args[t], oa[t][l])
    torch.cuda.synchronize()

    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    joins = [None] * L
    for t in range(T):
        for l in range(L):
            if joins[l] is not None:
                main.wait_event(joins[l])
            fork = torch.cuda.Event()
            fork.record(main)
            side.wait_event(fork)
            with torch.cuda.stream(side):
                lq.leapquant_decode_close_list(bb[l], pos_d[t], lst[t], *args[t], ob[t][l])
            joins[l] = torch.cuda.Event()
            joins[l].record(side)
            lq.leapquant_decode_step_slots(bb[l], step[t], *args[t], ob[t][l])
    for e in joins:
        main.wait_event(e)
    torch.cuda.synchronize()

    for t in range(T):
        for l in range(L):
            assert not torch.isnan(oa[t][l]).any()
            torch.testing.assert_close(oa[t][l], ob[t][l], rtol=0, atol=0, msg=lambda s, t=t: f"o at token {t}: {s}")
    for l in range(L):
        for k in ("codes", "row_scale", "col_scale", "comp_idx", "comp_val", "buf_gate", "buf_k", "buf_u"):
            torch.testing.assert_close(getattr(a[l], k), getattr(bb[l], k), rtol=0, atol=0,
                                       msg=lambda s, k=k: f"{k}: {s}")
