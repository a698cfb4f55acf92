"""Graph replay of a continuous-batching decode step.

Per-slot window positions live in device memory so that a serving loop can
capture its step once and replay it for every token.  The captured step
decodes the slots inside their window (decode_step_slots), decodes and
closes the slots at their window's last position (decode_close_slots), and
advances every slot's position on the device.  Replayed for 2p + 3 tokens,
with new token inputs copied in and unrelated eager work between replays,
it must give the outputs, boundary states, window buffers and positions of
the same steps run eagerly, bit for bit.
"""
import numpy as np
import pytest
import torch

import recurrent_state_quant_amd as lq
from tests.gpu_run import to_np, upload_boundary
from tests.test_gpu_parity import _dev, _random_window_inputs, _token, _upload_records

pytestmark = pytest.mark.gpu
DEV = "cuda"
KEYS = ("q", "k", "v", "beta", "alpha")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    lq.load()
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("gate", ["gdn", "kda"])
def test_graph_replay_serving_step(gate):
    rng = np.random.default_rng(7700 + (gate == "kda"))
    n, p, r = 300, 8, 4
    T = 2 * p + 3
    b, recs = _random_window_inputs(rng, n, p, p - 1, gate, r)
    toks = [{k: _dev(v) for k, v in _token(rng, n, gate).items()} for _ in range(T)]
    pos0 = rng.integers(0, p, n).astype(np.int32)

    def fresh():
        st = lq.LeapQuantState(n, p, r, gate, DEV)
        upload_boundary(st, b)
        _upload_records(st, recs, gate)
        return st, torch.as_tensor(pos0, device=DEV).clone()

    def step(st, pos, tk, o):
        last = pos == p - 1
        idle = torch.full_like(pos, -1)
        lq.leapquant_decode_step_slots(st, torch.where(last, idle, pos), *[tk[x] for x in KEYS], o)
        lq.leapquant_decode_close_slots(st, torch.where(last, pos, idle), *[tk[x] for x in KEYS], o)
        pos.copy_(torch.remainder(pos + 1, p))

    def snapshot(st, pos):
        out = {k: to_np(getattr(st, k)) for k in st.boundary_keys + ("buf_gate", "buf_k", "buf_u")}
        out["pos"] = to_np(pos)
        return out

    # eager reference
    st_e, pos_e = fresh()
    o_e = torch.empty((T, n, 128), device=DEV)
    for t in range(T):
        step(st_e, pos_e, toks[t], o_e[t])
    torch.cuda.synchronize()
    ref, ref_o = snapshot(st_e, pos_e), to_np(o_e)

    # capture one step on static buffers
    static = {k: torch.empty_like(v) for k, v in toks[0].items()}
    o_g = torch.empty((n, 128), device=DEV)
    stream = torch.cuda.Stream(device=DEV)
    st_w, pos_w = fresh()          # warm-up on a scratch slab (lazy init outside the capture)
    with torch.cuda.stream(stream):
        step(st_w, pos_w, toks[0], o_g)
    stream.synchronize()
    st_g, pos_g = fresh()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        step(st_g, pos_g, static, o_g)
    torch.cuda.synchronize()

    outs = []
    for t in range(T):
        for k in KEYS:
            static[k].copy_(toks[t][k])
        graph.replay()
        outs.append(o_g.clone())
        torch.zeros(1 << 20, device=DEV).sum()   # unrelated eager work between replays
        torch.cuda.synchronize()
    got = snapshot(st_g, pos_g)
    for t in range(T):
        np.testing.assert_array_equal(to_np(outs[t]), ref_o[t], err_msg=f"{gate} token {t}: outputs")
    for k in ref:
        np.testing.assert_array_equal(got[k], ref[k], err_msg=f"{gate}: {k} after {T} replays")
    assert (got["pos"] == (pos0 + T) % p).all()
