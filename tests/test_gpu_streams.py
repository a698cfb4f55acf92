"""Reentrancy: the library keeps no global state, so independent slabs can
be driven from several host threads on their own streams at once.

Two host threads each run windows of their own slab on their own stream
(default priority); the outputs and boundary states must equal, bit for
bit, those of the same work run one slab after the other on one stream.
"""
import threading

import numpy as np
import pytest
import torch

import recurrent_state_quant_amd as lq
from tests.gpu_run import boundary_np, upload_boundary
from tests.test_gpu_parity import _dev, _random_window_inputs, _token

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    lq.load()
    yield
    torch.cuda.synchronize()


def _problem(seed, gate, n, p, r, windows):
    rng = np.random.default_rng(seed)
    b, _ = _random_window_inputs(rng, n, p, 0, gate, r)
    toks = [[_token(rng, n, gate) for _ in range(p)] for _ in range(windows)]
    return b, toks


def _run(prob, gate, n, p, r, stream):
    """Decode the problem's windows (fused last token) on `stream`; returns
    the outputs and the final boundary state."""
    b, toks = prob
    with torch.cuda.stream(stream):
        st = lq.LeapQuantState(n, p, r, gate, DEV)
        upload_boundary(st, b)
        outs = torch.empty((len(toks), p, n, 128), device=DEV)
        dev_toks = [[{k: _dev(v) for k, v in tk.items()} for tk in w] for w in toks]
        for w, window in enumerate(dev_toks):
            for t, tk in enumerate(window):
                args = [tk[x] for x in ("q", "k", "v", "beta", "alpha")]
                call = lq.leapquant_decode_close if t == p - 1 else lq.leapquant_decode_step
                call(st, t, *args, outs[w, t], stream=stream)
    stream.synchronize()
    return outs.cpu().numpy(), boundary_np(st)


def test_two_threads_two_streams():
    n, p, r, windows = 300, 8, 4, 3
    cases = [(1100, "gdn"), (1101, "kda")]
    probs = [_problem(seed, gate, n, p, r, windows) for seed, gate in cases]
    ref_stream = torch.cuda.Stream(device=DEV)
    ref = [_run(pr, gate, n, p, r, ref_stream) for pr, (_, gate) in zip(probs, cases)]

    got = [None, None]
    errors = []

    def worker(i):
        try:
            got[i] = _run(probs[i], cases[i][1], n, p, r, torch.cuda.Stream(device=DEV))
        except Exception as e:  # surfaced below
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in threads), "a worker thread did not finish"
    assert not errors, errors
    for i in range(2):
        np.testing.assert_array_equal(got[i][0], ref[i][0], err_msg=f"slab {i}: outputs")
        for k in ref[i][1]:
            np.testing.assert_array_equal(got[i][1][k], ref[i][1][k], err_msg=f"slab {i}: {k}")
