"""Compacted closes (leapquant_decode_close_list, leapquant_window_close_list).

The list forms start one workgroup per listed slot instead of one per slot.
For every listed slot the result must equal the per-slot form's bit for bit
(the same kernel runs on the same inputs), whose parity with the oracle the
continuous-batching tests establish; unlisted slots, ids outside [0, n) and
slots whose position is out of range must be left untouched, and an empty
list must change nothing.
"""
import numpy as np
import pytest
import torch

import recurrent_state_quant_amd as lq
from tests.gpu_run import boundary_np, to_np, upload_boundary
from tests.test_gpu_parity import _dev, _random_window_inputs, _token, _upload_records

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    lq.load()
    yield
    torch.cuda.synchronize()


def _slab(b, recs, n, p, r, gate, flags=0, iters=0):
    st = lq.LeapQuantState(n, p, r, gate, DEV, flags=flags, comp_iters=iters)
    upload_boundary(st, b)
    _upload_records(st, recs, gate)
    return st


def _assert_same(got, ref, idx, what):
    for k in got:
        np.testing.assert_array_equal(got[k][idx], np.asarray(ref[k])[idx], err_msg=f"{what}: {k}")


@pytest.mark.parametrize("gate,dense", [("gdn", False), ("kda", False), ("gdn", True)])
def test_decode_close_list_matches_slots(gate, dense):
    rng = np.random.default_rng(8800 + (gate == "kda") + 2 * dense)
    n, p, r = 37, 16, 4
    iters = 2 if dense else None
    flags = lq.LQ_DENSE_COMP if dense else 0
    b, recs = _random_window_inputs(rng, n, p, p - 1, gate, r, dense_iters=iters)
    tok = _token(rng, n, gate)
    pos = rng.integers(0, p, n).astype(np.int32)
    pos[rng.choice(n, 10, replace=False)] = p - 1
    pos[[3, 4]] = [-1, p]                       # idle slots
    closing = np.nonzero(pos == p - 1)[0]
    listed = np.unique(np.concatenate([closing, [3, 4, 5, 6]]))  # plus idle slots and lower positions; each once
    ids = np.concatenate([listed, [-1, n, n + 7]]).astype(np.int32)  # ids outside [0, n): skipped
    rng.shuffle(ids)
    print(f"close list: gate={gate} dense={dense} listed={len(listed)} of {n}", flush=True)
    targs = [_dev(tok[x]) for x in ("q", "k", "v", "beta", "alpha")]
    pos_d = torch.as_tensor(pos, device=DEV)

    ref = _slab(b, recs, n, p, r, gate, flags, iters or 0)
    o_ref = torch.full((n, 128), float("nan"), device=DEV)
    lq.leapquant_decode_close_slots(ref, pos_d, *targs, o_ref)

    st = _slab(b, recs, n, p, r, gate, flags, iters or 0)
    o = torch.full((n, 128), float("nan"), device=DEV)
    lq.leapquant_decode_close_list(st, pos_d, torch.as_tensor(ids, device=DEV), *targs, o)
    torch.cuda.synchronize()
    g, gr, og, orf = boundary_np(st), boundary_np(ref), to_np(o), to_np(o_ref)
    active = np.array([s for s in listed if 0 <= pos[s] < p])
    _assert_same(g, gr, active, "listed slots")
    np.testing.assert_array_equal(og[active], orf[active])
    rest = np.setdiff1d(np.arange(n), active)
    _assert_same(g, b, rest, "untouched slots")
    assert np.isnan(og[rest]).all(), "unlisted or idle slots wrote o"

    # an empty list changes nothing
    before = boundary_np(st)
    lq.leapquant_decode_close_list(st, pos_d, torch.empty(0, dtype=torch.int32, device=DEV), *targs, o)
    torch.cuda.synchronize()
    _assert_same(boundary_np(st), before, np.arange(n), "empty list")


@pytest.mark.parametrize("gate", ["gdn", "kda"])
def test_window_close_list_matches_slots(gate):
    rng = np.random.default_rng(8900 + (gate == "kda"))
    n, p, r = 29, 16, 4
    b, recs = _random_window_inputs(rng, n, p, p, gate, r)
    lens = rng.integers(1, p + 1, n).astype(np.int32)
    lens[[0, 1]] = [0, p + 1]                  # slots left as they are
    listed = np.array([0, 1, 2, 7, 8, 9, 20, 28])
    ids = np.concatenate([listed, [-3, n]]).astype(np.int32)
    print(f"window close list: gate={gate} listed={len(listed)} of {n}", flush=True)
    lens_d = torch.as_tensor(lens, device=DEV)

    ref = _slab(b, recs, n, p, r, gate)
    lq.leapquant_window_close_slots(ref, lens_d)
    st = _slab(b, recs, n, p, r, gate)
    lq.leapquant_window_close_list(st, lens_d, torch.as_tensor(ids, device=DEV))
    torch.cuda.synchronize()
    g, gr = boundary_np(st), boundary_np(ref)
    active = np.array([s for s in listed if 1 <= lens[s] <= p])
    _assert_same(g, gr, active, "listed slots")
    rest = np.setdiff1d(np.arange(n), active)
    _assert_same(g, b, rest, "untouched slots")
