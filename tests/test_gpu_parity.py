"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Entry-point tests feed both sides the same boundary state and buffered
records; window tests start every window of the GPU from the oracle's own
boundary state (the oracle never reads a GPU result); free-running tests let
the GPU run on its own and compare until the two trajectories legitimately
part at a rounding boundary.
"""
import numpy as np
import pytest
import torch

import recurrent_state_quant_amd as lq
from oracle import leapquant_oracle as O
from tests import parity as P
from tests.gpu_run import boundary_np, run_window, to_np, tokens_np, upload_boundary
from workloads import generators as G
from workloads.configs import WORKLOADS

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    lq.load()
    yield
    torch.cuda.synchronize()


def _states_with_outliers(rng, n, scale=0.02):
    S = (scale * rng.standard_normal((n, 128, 128))).astype(np.float32)
    for s in range(n):
        rows = rng.choice(128, 3, replace=False)
        cols = rng.choice(128, 2, replace=False)
        S[s, rows] *= rng.uniform(10, 30, (3, 1)).astype(np.float32)
        S[s, :, cols] *= rng.uniform(10, 30, (2, 1)).astype(np.float32)
    return S


def _dev(x, dtype=torch.float32):
    return torch.as_tensor(np.ascontiguousarray(x)).to(device=DEV, dtype=dtype)


def _gate(g):
    return O.GATE_GDN if g == "gdn" else O.GATE_KDA


# ---------------------------------------------------------------------------
# a9 / a6-a8: quantize_state on the same fp32 input is bit-exact
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("r,flags", [(0, 0), (4, 0), (8, 0), (16, 0), (4, lq.LQ_NO_SMOOTH)])
def test_quantize_state_bitexact(r, flags):
    rng = np.random.default_rng(100 + r + 7 * flags)
    n = 37
    S = _states_with_outliers(rng, n)
    S[3] = 0.0                       # all-zero state: ties, zero columns
    S[5] = 0.0
    S[5, 17, 99] = -0.25             # single nonzero entry
    S[7, 10] = S[7, 20]              # duplicated rows: exact norm tie
    st = lq.LeapQuantState(n, 16, r, "gdn", DEV, flags)
    lq.leapquant_quantize_state(st, _dev(S))
    torch.cuda.synchronize()
    ref = O.quantize(S, r, flags)
    stats = P.compare_boundary(boundary_np(st), ref, S, r, "quantize_state", exact=True)
    assert stats["ties"] == 0


def test_quantize_state_workload_initial_states():
    for name in ("gdn_single_head_b1", "gdn_layer_h32_b64", "kda_h32_b128"):
        cfg = WORKLOADS[name]
        n = 1 if cfg.n_states == 1 else 64
        S = G.initial_state(cfg, n, G.make_generator(cfg.seed, "cpu"), "cpu").numpy()
        st = lq.LeapQuantState(n, cfg.p, cfg.r, cfg.gate, DEV)
        lq.leapquant_quantize_state(st, _dev(S))
        torch.cuda.synchronize()
        P.compare_boundary(boundary_np(st), O.quantize(S, cfg.r), S, cfg.r, f"{name} init", exact=True)


def test_dequantize_state():
    rng = np.random.default_rng(5)
    n, r = 9, 4
    S = _states_with_outliers(rng, n)
    b = O.quantize(S, r)
    st = lq.LeapQuantState(n, 16, r, "gdn", DEV)
    upload_boundary(st, b)
    out = torch.empty((n, 128, 128), device=DEV)
    lq.leapquant_dequantize_state(st, out)
    P.assert_close(to_np(out), O.dequantize(b), "dequantize", rtol=1e-6, atol=0)


# ---------------------------------------------------------------------------
# a1-a4: one decode step against synthetic buffered records
# ---------------------------------------------------------------------------
def _random_window_inputs(rng, n, p, nrec, gate, r, dense_iters=None):
    S = _states_with_outliers(rng, n)
    b = O.quantize(S, r) if dense_iters is None else O.quantize(S, r, O.DENSE_COMP, dense_iters)
    kda = gate == "kda"
    recs = []
    for _ in range(nrec):
        a = rng.uniform(0.05, 1.0, (n, 128) if kda else (n,)).astype(np.float32)
        k = rng.standard_normal((n, 128))
        k /= np.linalg.norm(k, axis=1, keepdims=True)
        kt = (rng.uniform(0.05, 1.0, (n, 1)) * k).astype(np.float32)
        u = (0.5 * rng.standard_normal((n, 128))).astype(np.float32)
        recs.append((a, kt, u))
    return b, recs


def _upload_records(st, recs, gate):
    for i, (a, kt, u) in enumerate(recs):
        st.buf_gate[:, i] = _dev(a)
        st.buf_k[:, i] = _dev(kt)
        st.buf_u[:, i] = _dev(u)


def _oracle_records(recs, gate):
    out = []
    for a, kt, u in recs:
        n = kt.shape[0]
        d = np.broadcast_to(a.astype(np.float64).reshape(n, -1), (n, 128))
        out.append((d, kt.astype(np.float64), u.astype(np.float64)))
    return out


def _token(rng, n, gate):
    q = rng.standard_normal((n, 128)); q /= np.linalg.norm(q, axis=1, keepdims=True)
    k = rng.standard_normal((n, 128)); k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((n, 128))
    beta = rng.uniform(0.05, 1, n)
    alpha = rng.uniform(0.05, 1, (n, 128) if gate == "kda" else n)
    return {x: y.astype(np.float32) for x, y in dict(q=q, k=k, v=v, beta=beta, alpha=alpha).items()}


@pytest.mark.parametrize("gate", ["gdn", "kda"])
@pytest.mark.parametrize("p,t", [(1, 0), (16, 0), (16, 1), (16, 9), (16, 15), (32, 16), (32, 31), (64, 40), (64, 63)])
@pytest.mark.parametrize("r", [0, 4, 16])
def test_decode_step_entry(gate, p, t, r):
    rng = np.random.default_rng(1000 * p + 10 * t + r + (gate == "kda"))
    n = 19
    b, recs = _random_window_inputs(rng, n, p, t, gate, r)
    st = lq.LeapQuantState(n, p, r, gate, DEV)
    upload_boundary(st, b)
    _upload_records(st, recs, gate)
    tok = _token(rng, n, gate)
    o = torch.empty((n, 128), device=DEV)
    lq.leapquant_decode_step(st, t, _dev(tok["q"]), _dev(tok["k"]), _dev(tok["v"]), _dev(tok["beta"]),
                             _dev(tok["alpha"]), o)
    torch.cuda.synchronize()
    S_prev = O.replay(O.dequantize(b), _oracle_records(recs, gate))
    t64 = {k: v.astype(np.float64) for k, v in tok.items()}
    o_ref, _, (d, kt, u) = O.step(S_prev, t64["q"], t64["k"], t64["v"], t64["beta"], t64["alpha"], _gate(gate))
    P.assert_close(to_np(o), o_ref, "o_t")
    P.assert_close(to_np(st.buf_u[:, t]), u, "u_t")
    P.assert_close(to_np(st.buf_k[:, t]), kt, "k~_t", rtol=1e-6, atol=0)
    np.testing.assert_array_equal(to_np(st.buf_gate[:, t]), tok["alpha"])
    # records < t untouched
    for i, (a, ktr, ur) in enumerate(recs):
        np.testing.assert_array_equal(to_np(st.buf_u[:, i]), ur)


# The decode launcher picks its kernel by slab size (two waves per state up
# to 4,096 states, one wave above).  Both sides of the switch, with per-slot
# window positions and idle slots, on slabs tiled from m distinct states so
# that the oracle computes m states and every slot is still compared.
@pytest.mark.parametrize("gate", ["gdn", "kda"])
@pytest.mark.parametrize("n,dense", [(4096, False), (4097, False), (4096, True), (4097, True)])
def test_decode_step_slab_sizes(gate, n, dense):
    rng = np.random.default_rng(2000 + n + 7 * (gate == "kda") + 3 * dense)
    m, p, r = 13, 16, 4
    base_t = rng.integers(0, p, m)
    base_t[0], base_t[1] = 0, p - 1
    b, recs = _random_window_inputs(rng, m, p, p - 1, gate, r, 2 if dense else None)
    tok = _token(rng, m, gate)
    tile = np.arange(n) % m
    pos = base_t[tile].astype(np.int32)
    idle = np.zeros(n, bool)
    idle[[5, n // 2, n - 1]] = True
    pos[idle] = [-1, p, -1]
    st = lq.LeapQuantState(n, p, r, gate, DEV, flags=lq.LQ_DENSE_COMP if dense else 0, comp_iters=2)
    upload_boundary(st, {k: v[tile] for k, v in b.items()})
    _upload_records(st, [(a[tile], kt[tile], u[tile]) for a, kt, u in recs], gate)
    st.buf_u[:, p - 1] = float("nan")
    o = torch.full((n, 128), float("nan"), device=DEV)
    lq.leapquant_decode_step_slots(st, torch.as_tensor(pos, device=DEV),
                                   *[_dev(tok[x][tile]) for x in ("q", "k", "v", "beta", "alpha")], o)
    torch.cuda.synchronize()
    o_ref = np.empty((m, 128))
    u_ref = np.empty((m, 128))
    t64 = {k: v.astype(np.float64) for k, v in tok.items()}
    for t in np.unique(base_t):
        j = np.nonzero(base_t == t)[0]
        S_prev = O.replay(O.dequantize({k: v[j] for k, v in b.items()}),
                          _oracle_records([(a[j], kt[j], u[j]) for a, kt, u in recs[:t]], gate))
        o_j, _, (_, _, u_j) = O.step(S_prev, *[t64[x][j] for x in ("q", "k", "v", "beta", "alpha")],
                                     _gate(gate))
        o_ref[j], u_ref[j] = o_j, u_j
    og, ug = to_np(o), to_np(st.buf_u)
    act = ~idle
    P.assert_close(og[act], o_ref[tile[act]], f"o_t, {n} slots")
    P.assert_close(ug[act, pos[act]], u_ref[tile[act]], f"u_t, {n} slots")
    assert np.isnan(og[idle]).all(), "idle slots wrote o"
    assert np.isnan(ug[idle, p - 1]).all(), "idle slots wrote a record"


# ---------------------------------------------------------------------------
# a5-a8: window close against synthetic records
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("gate", ["gdn", "kda"])
@pytest.mark.parametrize("p,length", [(1, 1), (16, 16), (16, 1), (16, 7), (32, 32), (64, 64), (64, 37)])
@pytest.mark.parametrize("r,flags", [(0, 0), (4, 0), (8, 0), (16, 0), (4, lq.LQ_NO_SMOOTH)])
def test_window_close_entry(gate, p, length, r, flags):
    rng = np.random.default_rng(7 * p + length + 100 * r + flags + (gate == "kda"))
    n = 21
    b, recs = _random_window_inputs(rng, n, p, length, gate, r)
    st = lq.LeapQuantState(n, p, r, gate, DEV, flags)
    upload_boundary(st, b)
    _upload_records(st, recs, gate)
    lq.leapquant_window_close(st, length)
    torch.cuda.synchronize()
    S = O.replay(O.dequantize(b), _oracle_records(recs, gate))
    ref = O.quantize(S, r, flags)
    P.compare_boundary(boundary_np(st), ref, S.astype(np.float32), r, "window_close", flags=flags,
                       mag=P.rebuild_magnitude(b, _oracle_records(recs, gate)))


# ---------------------------------------------------------------------------
# a1-a8 fused: decode the window's last token and close the window
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("gate", ["gdn", "kda"])
@pytest.mark.parametrize("p,t", [(1, 0), (16, 0), (16, 7), (16, 15), (32, 31), (64, 40), (64, 63)])
@pytest.mark.parametrize("r,flags", [(0, 0), (4, 0), (16, 0), (4, lq.LQ_NO_SMOOTH)])
def test_decode_close_entry(gate, p, t, r, flags):
    rng = np.random.default_rng(5000 + 100 * p + t + 7 * r + flags + (gate == "kda"))
    n = 19
    b, recs = _random_window_inputs(rng, n, p, t, gate, r)
    st = lq.LeapQuantState(n, p, r, gate, DEV, flags)
    upload_boundary(st, b)
    _upload_records(st, recs, gate)
    tok = _token(rng, n, gate)
    o = torch.empty((n, 128), device=DEV)
    lq.leapquant_decode_close(st, t, _dev(tok["q"]), _dev(tok["k"]), _dev(tok["v"]), _dev(tok["beta"]),
                              _dev(tok["alpha"]), o)
    torch.cuda.synchronize()
    S_prev = O.replay(O.dequantize(b), _oracle_records(recs, gate))
    t64 = {k: v.astype(np.float64) for k, v in tok.items()}
    o_ref, S_t, rec_t = O.step(S_prev, t64["q"], t64["k"], t64["v"], t64["beta"], t64["alpha"], _gate(gate))
    P.assert_close(to_np(o), o_ref, "o_t")
    ref = O.quantize(S_t, r, flags)
    P.compare_boundary(boundary_np(st), ref, S_t.astype(np.float32), r, "decode_close", flags=flags,
                       mag=P.rebuild_magnitude(b, _oracle_records(recs, gate) + [rec_t]))
    # the buffer is read, never written
    for i, (a, ktr, ur) in enumerate(recs):
        np.testing.assert_array_equal(to_np(st.buf_u[:, i]), ur)
    assert not to_np(st.buf_u[:, t]).any() and not to_np(st.buf_k[:, t]).any()


# ---------------------------------------------------------------------------
# Whole windows: the GPU starts each window from the oracle's boundary
# ---------------------------------------------------------------------------
def _workload(name, n, steps, device="cpu", seed=None):
    cfg = WORKLOADS[name]
    g = G.make_generator(cfg.seed if seed is None else seed, device)
    S0 = G.initial_state(cfg, n, g, device)
    tok = G.token_inputs(cfg, n, steps, g, device)
    return cfg, S0, tok


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("name,n,steps", [("gdn_single_head_b1", 1, 256), ("gdn_layer_h32_b64", 24, 128),
                                          ("kda_h32_b128", 24, 128)])
def test_oracle_forced_windows(name, n, steps, fused):
    cfg, S0, tok = _workload(name, n, steps)
    S0n = S0.numpy()
    tokn = {k: v.numpy().astype(np.float64) for k, v in tok.items()}
    o_ref, bounds = O.run_windowed(S0n, tokn, cfg.p, cfg.r, _gate(cfg.gate))
    tokd = {k: v.to(DEV) for k, v in tok.items()}
    st = lq.LeapQuantState(n, cfg.p, cfg.r, cfg.gate, DEV)
    out = torch.empty((steps, n, 128), device=DEV)
    total = {"flips": 0, "codes": 0, "ties": 0}
    for w in range(steps // cfg.p):
        upload_boundary(st, bounds[w])
        run_window(st, tokd, w * cfg.p, cfg.p, out, fused=fused)
        torch.cuda.synchronize()
        sl = slice(w * cfg.p, (w + 1) * cfg.p)
        P.assert_close(to_np(out[sl]), o_ref[sl], f"{name} window {w} outputs")
        _, recs, S_end, _ = O.window(bounds[w], tokn, w * cfg.p, cfg.p, _gate(cfg.gate), cfg.r)
        s = P.compare_boundary(boundary_np(st), bounds[w + 1], S_end.astype(np.float32), cfg.r,
                               f"{name} boundary {w + 1}", mag=P.rebuild_magnitude(bounds[w], recs))
        for k in total:
            total[k] += s[k]
    print(f"{name}: {total}")


# ---------------------------------------------------------------------------
# Free-running: strict until the first legitimate rounding-boundary flip
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("name,n,steps", [("gdn_single_head_b1", 1, 256), ("gdn_layer_h32_b64", 16, 256),
                                          ("kda_h32_b128", 16, 256)])
def test_free_running(name, n, steps, fused):
    cfg, S0, tok = _workload(name, n, steps)
    S0n = S0.numpy()
    tokn = {k: v.numpy().astype(np.float64) for k, v in tok.items()}
    o_ref, bounds = O.run_windowed(S0n, tokn, cfg.p, cfg.r, _gate(cfg.gate))
    tokd = {k: v.to(DEV) for k, v in tok.items()}
    st = lq.LeapQuantState(n, cfg.p, cfg.r, cfg.gate, DEV)
    lq.leapquant_quantize_state(st, S0.to(DEV))
    out = torch.empty((steps, n, 128), device=DEV)
    diverged = np.zeros(n, bool)
    worst_rel = 0.0
    on_track = parted = 0
    for w in range(steps // cfg.p):
        run_window(st, tokd, w * cfg.p, cfg.p, out, fused=fused)
        torch.cuda.synchronize()
        sl = slice(w * cfg.p, (w + 1) * cfg.p)
        og, orf = to_np(out[sl]), o_ref[sl]
        strict = ~diverged
        if strict.any():
            P.assert_close(og[:, strict], orf[:, strict], f"{name} window {w} outputs")
        if diverged.any():
            rel = np.linalg.norm(og[:, diverged] - orf[:, diverged]) / np.linalg.norm(orf[:, diverged])
            worst_rel = max(worst_rel, rel)
            assert rel < 2e-2, f"{name} window {w}: diverged trajectories differ by {rel}"
        gb = boundary_np(st)
        if strict.any():
            # a state still on the oracle's trajectory closed this window from
            # the oracle's boundary: its new boundary is checked strictly, so
            # it can only part at a legitimate rounding flip or near tie
            sel = np.nonzero(strict)[0]
            _, recs, S_end, _ = O.window(O.copy_boundary(bounds[w], sel), {k: v[:, sel] for k, v in tokn.items()},
                                         w * cfg.p, cfg.p, _gate(cfg.gate), cfg.r)
            P.compare_boundary({k: v[sel] for k, v in gb.items()}, O.copy_boundary(bounds[w + 1], sel),
                               S_end.astype(np.float32), cfg.r, f"{name} free boundary {w + 1}",
                               mag=P.rebuild_magnitude(O.copy_boundary(bounds[w], sel), recs))
        same = np.all(gb["codes"] == bounds[w + 1]["codes"], axis=(1, 2))
        if cfg.r:
            same &= np.all(gb["comp_idx"] == bounds[w + 1]["comp_idx"], axis=1)
        newly = strict & ~same
        on_track += int(strict.sum())
        parted += int(newly.sum())
        diverged |= ~same
    # a state parts at a code within fp32 rounding of a half-integer (a few in
    # 10^5 codes, each checked above), so over the run most closes of a state
    # on the trajectory keep it there; a kernel error would flip codes far from
    # a rounding boundary in every state
    assert parted <= max(2, on_track // 2), f"{name}: {parted} of {on_track} closes parted a state"
    print(f"{name}: diverged states {diverged.sum()}/{n} ({parted} of {on_track} closes parted one), "
          f"worst diverged rel err {worst_rel:.2e}")


# ---------------------------------------------------------------------------
# Determinism and prefix-cache snapshot / resume
# ---------------------------------------------------------------------------
def _run_free(cfg, n, steps, S0d, tokd, snapshot_at=None, start=0, st=None):
    if st is None:
        st = lq.LeapQuantState(n, cfg.p, cfg.r, cfg.gate, DEV)
        lq.leapquant_quantize_state(st, S0d)
    out = torch.zeros((steps, n, 128), device=DEV)
    snap = None
    for w in range(start // cfg.p, steps // cfg.p):
        run_window(st, tokd, w * cfg.p, cfg.p, out)
        if snapshot_at is not None and (w + 1) * cfg.p == snapshot_at:
            snap = st.snapshot()
    torch.cuda.synchronize()
    return out, st, snap


def test_determinism_and_resume():
    cfg, S0, tok = _workload("gdn_layer_h32_b64", 96, 96, device=DEV)
    out1, st1, snap = _run_free(cfg, 96, 96, S0, tok, snapshot_at=48)
    out2, st2, _ = _run_free(cfg, 96, 96, S0, tok)
    assert torch.equal(out1, out2)
    for k in lq.LeapQuantState.BOUNDARY:
        assert torch.equal(getattr(st1, k), getattr(st2, k)), k
    st3 = lq.LeapQuantState(96, cfg.p, cfg.r, cfg.gate, DEV)
    st3.load_boundary(snap)
    out3, st3, _ = _run_free(cfg, 96, 96, None, tok, start=48, st=st3)
    assert torch.equal(out3[48:], out1[48:])
    for k in lq.LeapQuantState.BOUNDARY:
        assert torch.equal(getattr(st3, k), getattr(st1, k)), k


# ---------------------------------------------------------------------------
# Dense-state baselines ([EL] Table 2, FP32 and BF16 per-step)
# ---------------------------------------------------------------------------
def _bf16_ulp(x):
    """Spacing of bf16 values at |x| (normal range)."""
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return 2.0 ** (e - 7)


@pytest.mark.parametrize("gate", ["gdn", "kda"])
def test_dense_fp32_steps(gate):
    rng = np.random.default_rng(800 + (gate == "kda"))
    n, T = 23, 12
    S0 = _states_with_outliers(rng, n)
    toks = [_token(rng, n, gate) for _ in range(T)]
    S = _dev(S0)
    o = torch.empty((n, 128), device=DEV)
    S_ref = S0.astype(np.float64)
    for t in range(T):
        tok = toks[t]
        lq.leapquant_dense_step(S, gate, *(_dev(tok[x]) for x in ("q", "k", "v", "beta", "alpha")), o)
        t64 = {x: y.astype(np.float64) for x, y in tok.items()}
        o_ref, S_ref, _ = O.step(S_ref, t64["q"], t64["k"], t64["v"], t64["beta"], t64["alpha"], _gate(gate))
        torch.cuda.synchronize()
        P.assert_close(to_np(o), o_ref, f"dense fp32 o_{t}")
    P.assert_close(to_np(S), S_ref, "dense fp32 state")


@pytest.mark.parametrize("gate", ["gdn", "kda"])
def test_dense_bf16_step(gate):
    rng = np.random.default_rng(900 + (gate == "kda"))
    n = 23
    S0 = O.round_bf16(_states_with_outliers(rng, n))
    tok = _token(rng, n, gate)
    S = torch.as_tensor(S0).to(torch.float32).to(torch.bfloat16).to(DEV)
    assert torch.equal(S.double().cpu(), torch.as_tensor(S0))   # exact upload
    o = torch.empty((n, 128), device=DEV)
    lq.leapquant_dense_step(S, gate, *(_dev(tok[x]) for x in ("q", "k", "v", "beta", "alpha")), o)
    torch.cuda.synchronize()
    t64 = {x: y.astype(np.float64) for x, y in tok.items()}
    o_ref, S_ref = O.step_dense_bf16(S0, t64["q"], t64["k"], t64["v"], t64["beta"], t64["alpha"], _gate(gate))
    P.assert_close(to_np(o), o_ref, "dense bf16 o")
    Sg = S.double().cpu().numpy()
    # the rounding to bf16 is decided from the fp32 update on the GPU and from
    # the fp64 one in the oracle: they may differ by one bf16 step where the
    # update sits at a rounding tie, plus the fp32 error of the update's two
    # terms D S and k~ u, which dominates where they cancel
    d_, kt_, _ = O.transition(_gate(gate), t64["k"], t64["beta"], t64["alpha"], 128)
    _, _, (_, _, u_) = O.step(S0, t64["q"], t64["k"], t64["v"], t64["beta"], t64["alpha"], _gate(gate))
    terms = np.abs(d_[:, :, None] * S0) + np.abs(kt_[:, :, None] * u_[:, None, :])
    d = np.abs(Sg - S_ref)
    bound = _bf16_ulp(S_ref) * 1.0001 + 64 * 2.0 ** -24 * terms
    worst = np.unravel_index(np.argmax(d - bound), d.shape)
    assert np.all(d <= bound), (worst, float(Sg[worst]), float(S_ref[worst]), float(bound[worst]))
    assert (d > 0).mean() <= 1e-3, float((d > 0).mean())


# ---------------------------------------------------------------------------
# Continuous batching: slots join and finish at different steps, each with
# its own window phase; partial windows are closed at sequence end
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name,dense", [("gdn_layer_h32_b64", False), ("kda_h32_b128", False),
                                        ("gdn_layer_h32_b64", True)])
def test_continuous_batching_slots(name, dense):
    cfg = WORKLOADS[name]
    flags, iters = (O.DENSE_COMP, 2) if dense else (0, 0)
    n, T, p = 12, 64, cfg.p
    rng = np.random.default_rng(73 if cfg.gate == "kda" else 71)
    join = rng.integers(0, 24, n)
    end = np.minimum(T, join + rng.integers(8, 60, n))
    end[0], join[0] = T, 0                          # one slot runs the whole time
    cfgw, S0, tok = _workload(name, n, T)
    tokn = {k: v.numpy().astype(np.float64) for k, v in tok.items()}
    tokd = {k: v.to(DEV) for k, v in tok.items()}
    gate = _gate(cfg.gate)
    ref_o, ref_b, ref_tok = [], [], []
    for s in range(n):
        ts = {k: v[join[s]:end[s], s:s + 1] for k, v in tokn.items()}
        o_s, b_s = O.run_windowed(S0.numpy()[s:s + 1], ts, p, cfg.r, gate, flags, iters=iters)
        ref_o.append(o_s[:, 0])
        ref_b.append(b_s)
        ref_tok.append(ts)
    st = lq.LeapQuantState(n, p, cfg.r, cfg.gate, DEV, flags=lq.LQ_DENSE_COMP if dense else 0,
                           comp_iters=iters)
    for s in range(n):
        upload_boundary(st, ref_b[s][0], [s])
    window = np.zeros(n, int)
    out = torch.zeros((n, 128), device=DEV)
    flips = 0
    for t in range(T):
        active = (join <= t) & (t < end)
        pos = np.where(active, (t - join) % p, -1)
        closing = active & (pos == p - 1)
        ending = active & (t == end - 1) & ~closing
        step_pos = torch.as_tensor(np.where(closing, -1, pos), dtype=torch.int32, device=DEV)
        close_pos = torch.as_tensor(np.where(closing, pos, -1), dtype=torch.int32, device=DEV)
        args = [tokd[x][t] for x in ("q", "k", "v", "beta", "alpha")] + [out]
        lq.leapquant_decode_step_slots(st, step_pos, *args)
        lq.leapquant_decode_close_slots(st, close_pos, *args)
        if ending.any():
            lens = torch.as_tensor(np.where(ending, pos + 1, 0), dtype=torch.int32, device=DEV)
            lq.leapquant_window_close_slots(st, lens)
        torch.cuda.synchronize()
        og = to_np(out)
        for s in np.nonzero(active)[0]:
            P.assert_close(og[s:s + 1], ref_o[s][t - join[s]][None], f"slot {s} step {t}")
        for s in np.nonzero(closing | ending)[0]:
            window[s] += 1
            gb = boundary_np(st, [s])
            w0 = (window[s] - 1) * p          # the window's first token, in slot s's own count
            _, _, S_end, _ = O.window(ref_b[s][window[s] - 1], ref_tok[s], w0, t - join[s] + 1 - w0,
                                      gate, cfg.r, flags, iters=iters)
            what = f"slot {s} boundary {window[s]}"
            if dense:
                stats = P.compare_dense_boundary(gb, S_end.astype(np.float32), cfg.r, iters, 0, what)
            else:
                stats = P.compare_boundary(gb, ref_b[s][window[s]], S_end.astype(np.float32), cfg.r, what)
            flips += stats["flips"]
            upload_boundary(st, ref_b[s][window[s]], [s])   # next window starts from the oracle's state
    assert window.sum() == sum(int(np.ceil((end[s] - join[s]) / p)) for s in range(n))
    print(f"{name}{' dense' if dense else ''}: {window.sum()} slot windows, {flips} flipped codes")


# ---------------------------------------------------------------------------
# The other rows of [EL] Appendix Table 4 (LQ_NO_DELTA: b_t = 0)
# ---------------------------------------------------------------------------
_TABLE4 = {  # row: (gate, alpha rule, beta = 1?, no delta?)
    "linear_attention": ("gdn", "one", True, True),
    "retnet": ("gdn", "const", True, True),
    "mamba2": ("gdn", "token", True, True),
    "gla_rwkv6_hgrn2": ("kda", "token", True, True),
    "deltanet": ("gdn", "one", False, False),
}


def _table4_tokens(row, n, T, seed):
    gate, arule, beta1, _ = _TABLE4[row]
    cfg = WORKLOADS["kda_h32_b128" if gate == "kda" else "gdn_layer_h32_b64"]
    g = G.make_generator(seed, "cpu")
    S0 = G.initial_state(cfg, n, g, "cpu")
    tok = G.token_inputs(cfg, n, T, g, "cpu")
    if arule == "one":
        tok["alpha"] = torch.ones_like(tok["alpha"])
    elif arule == "const":
        tok["alpha"] = torch.full_like(tok["alpha"], 0.9)
    if beta1:
        tok["beta"] = torch.ones_like(tok["beta"])
    return cfg, S0, tok


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("row", list(_TABLE4))
def test_table4_rows_forced_windows(row, fused):
    gate, _, _, nodelta = _TABLE4[row]
    n, T, p, r = 12, 48, 16, 4
    flags = lq.LQ_NO_DELTA if nodelta else 0
    cfg, S0, tok = _table4_tokens(row, n, T, 31)
    tokn = {k: v.numpy().astype(np.float64) for k, v in tok.items()}
    oflags = O.NO_DELTA if nodelta else 0
    o_ref, bounds = O.run_windowed(S0.numpy(), tokn, p, r, _gate(gate), flags=oflags)
    tokd = {k: v.to(DEV) for k, v in tok.items()}
    st = lq.LeapQuantState(n, p, r, gate, DEV, flags)
    out = torch.empty((T, n, 128), device=DEV)
    for w in range(T // p):
        upload_boundary(st, bounds[w])
        run_window(st, tokd, w * p, p, out, fused=fused)
        torch.cuda.synchronize()
        sl = slice(w * p, (w + 1) * p)
        P.assert_close(to_np(out[sl]), o_ref[sl], f"{row} window {w} outputs")
        _, _, S_end, _ = O.window(bounds[w], tokn, w * p, p, _gate(gate), r, oflags)
        P.compare_boundary(boundary_np(st), bounds[w + 1], S_end.astype(np.float32), r,
                           f"{row} boundary {w + 1}")


@pytest.mark.parametrize("row", ["mamba2", "gla_rwkv6_hgrn2"])
def test_table4_rows_dense_baseline(row):
    gate, _, _, nodelta = _TABLE4[row]
    n, T = 10, 6
    cfg, S0, tok = _table4_tokens(row, n, T, 32)
    S = S0.to(DEV).contiguous()
    S_ref = S0.numpy().astype(np.float64)
    o = torch.empty((n, 128), device=DEV)
    for t in range(T):
        lq.leapquant_dense_step(S, gate, *(tok[x][t].to(DEV) for x in ("q", "k", "v", "beta", "alpha")), o,
                                flags=lq.LQ_NO_DELTA)
        t64 = {x: tok[x][t].numpy().astype(np.float64) for x in tok}
        o_ref, S_ref, _ = O.step(S_ref, t64["q"], t64["k"], t64["v"], t64["beta"], t64["alpha"], _gate(gate),
                                 O.NO_DELTA)
        torch.cuda.synchronize()
        P.assert_close(to_np(o), o_ref, f"{row} dense o_{t}")
    P.assert_close(to_np(S), S_ref, f"{row} dense state")


# ---------------------------------------------------------------------------
# DeltaProduct ([EL] Table 4 caption): n_h delta-rule sub-steps per token,
# each an instance of the recurrence with its own record; the token's output
# is read after the last sub-step.  The existing calls cover it: sub-steps
# are consecutive window positions (p a multiple of n_h), the window closes
# at a token boundary.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("fused", [False, True])
def test_deltaproduct_substeps(fused):
    nh, tokens_, n, p, r = 2, 24, 10, 16, 4
    steps = nh * tokens_
    cfg, S0, tok = _workload("gdn_layer_h32_b64", n, steps, seed=33)        # sub-step inputs, [steps, n, ...]
    tokn = {k: v.numpy().astype(np.float64) for k, v in tok.items()}
    o_ref, bounds = O.run_windowed(S0.numpy(), tokn, p, r, O.GATE_GDN)
    tokd = {k: v.to(DEV) for k, v in tok.items()}
    st = lq.LeapQuantState(n, p, r, "gdn", DEV)
    out = torch.empty((steps, n, 128), device=DEV)
    for w in range(steps // p):
        upload_boundary(st, bounds[w])
        run_window(st, tokd, w * p, p, out, fused=fused)
        torch.cuda.synchronize()
        # token outputs: after sub-steps nh-1, 2nh-1, ... of the window
        sl = slice(w * p + nh - 1, (w + 1) * p, nh)
        P.assert_close(to_np(out[sl]), o_ref[sl], f"DeltaProduct window {w} token outputs")
        _, _, S_end, _ = O.window(bounds[w], tokn, w * p, p, O.GATE_GDN, r)
        P.compare_boundary(boundary_np(st), bounds[w + 1], S_end.astype(np.float32), r,
                           f"DeltaProduct boundary {w + 1}")


# ---------------------------------------------------------------------------
# Graph replay (the benchmark's launch mode): a captured window replays to
# the eager result, bit for bit, on every replay
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dense", [False, True])
def test_graph_replay_matches_eager(dense):
    cfg, S0, tok = _workload("gdn_layer_h32_b64", 64, 16)
    flags = lq.LQ_DENSE_COMP if dense else 0
    st = lq.LeapQuantState(64, cfg.p, cfg.r, cfg.gate, DEV, flags=flags, comp_iters=2)
    tokd = {k: v.to(DEV) for k, v in tok.items()}
    out = torch.zeros((16, 64, 128), device=DEV)
    lq.leapquant_quantize_state(st, S0.to(DEV))
    torch.cuda.synchronize()
    start = {k: getattr(st, k).clone() for k in st.boundary_keys + ("buf_gate", "buf_k", "buf_u")}

    def restore():
        for k, v in start.items():
            getattr(st, k).copy_(v)
        out.zero_()

    def window():
        run_window(st, tokd, 0, cfg.p, out, fused=True)

    window()
    torch.cuda.synchronize()
    ref = {k: to_np(getattr(st, k)) for k in st.boundary_keys}
    ref_o = to_np(out)
    stream = torch.cuda.Stream(device=DEV)
    restore()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        window()
    torch.cuda.synchronize()
    for rep in range(3):
        restore()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_np(out), ref_o, err_msg=f"replay {rep}: outputs")
        for k in st.boundary_keys:
            np.testing.assert_array_equal(to_np(getattr(st, k)), ref[k], err_msg=f"replay {rep}: {k}")
        torch.zeros(1 << 20, device=DEV).sum()   # eager work between replays



# ---------------------------------------------------------------------------
# Degenerate tokens: full forgetting (alpha = 0), no decay (alpha = 1), no
# write (beta = 0), zero keys, queries and values, mixed across states
# ---------------------------------------------------------------------------
def _degenerate_token(rng, n, gate, t):
    tok = _token(rng, n, gate)
    kind = (np.arange(n) + t) % 6
    a = tok["alpha"]
    if gate == "kda":
        a[kind == 0] = 0.0                       # forget every channel
        a[kind == 1] = 1.0                       # no decay
        a[kind == 5, ::2] = 0.0                  # half the channels forget
    else:
        a[kind == 0] = 0.0
        a[kind == 1] = 1.0
    tok["beta"][kind == 2] = 0.0                 # no write
    tok["k"][kind == 3] = 0.0                    # zero key
    tok["q"][kind == 4] = 0.0                    # zero query
    tok["v"][kind == 4] = 0.0                    # and zero value
    return tok


@pytest.mark.parametrize("gate", ["gdn", "kda"])
@pytest.mark.parametrize("fused", [False, True])
def test_degenerate_tokens(gate, fused):
    """A whole window of degenerate tokens from the oracle's boundary: every
    output, and the next boundary, match the oracle."""
    rng = np.random.default_rng(7000 + 2 * (gate == "kda") + fused)
    n, p, r = 24, 16, 4
    S = _states_with_outliers(rng, n)
    b = O.quantize(S, r)
    toks = [_degenerate_token(rng, n, gate, t) for t in range(p)]
    tok = {k: np.stack([x[k] for x in toks]) for k in toks[0]}
    st = lq.LeapQuantState(n, p, r, gate, DEV)
    upload_boundary(st, b)
    tokd = {k: _dev(v) for k, v in tok.items()}
    out = torch.empty((p, n, 128), device=DEV)
    run_window(st, tokd, 0, p, out, fused=fused)
    torch.cuda.synchronize()
    t64 = {k: v.astype(np.float64) for k, v in tok.items()}
    o_ref, _, S_end, b_next = O.window(b, t64, 0, p, _gate(gate), r)
    P.assert_close(to_np(out), o_ref, "degenerate outputs")
    P.compare_boundary(boundary_np(st), b_next, S_end.astype(np.float32), r, "degenerate boundary")


# ---------------------------------------------------------------------------
# Near ties in the top-r selection: two rows holding the same values in a
# different order have the same norm; the fp32 sums on the GPU (in the
# kernel's order) rank them either way.  Each such state is compared with
# the oracle forced to the GPU's rows (tests/parity.py), and every case must
# produce some near ties, so that path is exercised.
# ---------------------------------------------------------------------------
def _tie_states(rng, n, r, n_old=0):
    """States whose r-th and (r+1)-th largest rows (after `n_old` larger
    rows) are permutations of one vector of wide dynamic range."""
    S = (0.02 * rng.standard_normal((n, 128, 128))).astype(np.float32)
    rows = np.zeros((n, n_old + r + 1), np.int64)
    for s in range(n):
        perm = rng.permutation(128)
        rows[s] = perm[:n_old + r + 1]
        for j in range(n_old):            # distinct, largest
            S[s, perm[j]] = (30.0 - 0.5 * j) * rng.standard_normal(128)
        for j in range(r - 1):            # distinct, above the tie
            S[s, perm[n_old + j]] = (15.0 - 0.25 * j) * rng.standard_normal(128)
        base = (rng.standard_normal(128) * 10.0 ** rng.uniform(-3, 0, 128)).astype(np.float32)
        base *= np.float32(40.0 / np.linalg.norm(base))
        S[s, perm[n_old + r - 1]] = base
        S[s, perm[n_old + r]] = base[rng.permutation(128)]
    return S, rows


@pytest.mark.parametrize("r", [1, 4, 8, 16])
def test_quantize_near_tie_rows(r):
    rng = np.random.default_rng(7100 + r)
    n = 64
    S, _ = _tie_states(rng, n, r)
    st = lq.LeapQuantState(n, 16, r, "gdn", DEV)
    lq.leapquant_quantize_state(st, _dev(S))
    torch.cuda.synchronize()
    stats = P.compare_boundary(boundary_np(st), O.quantize(S, r), S, r, "quantize near ties", exact=True)
    print(f"r={r}: {stats['ties']} of {n} states ranked the tied rows the other way")
    assert stats["ties"] > 0, "no near tie was exercised"


@pytest.mark.parametrize("gate", ["gdn", "kda"])
@pytest.mark.parametrize("r", [4, 8, 16])
@pytest.mark.parametrize("fused", [False, True])
def test_close_near_tie_rows(gate, r, fused):
    """The boundary's compensator rows are erased by the window's records
    (unit key on the row, u = -w_c, gate 1: the delta rule's exact erase),
    so the new top r come from the residual, where the tied pair sits."""
    rng = np.random.default_rng(7200 + 10 * r + 3 * fused + (gate == "kda"))
    n = 48
    p = 16 if r < 16 else 32
    S, rows = _tie_states(rng, n, r, n_old=r)
    b = O.quantize(S, r, O.NO_SMOOTH)
    np.testing.assert_array_equal(np.sort(b["comp_idx"], axis=1), np.sort(rows[:, :r], axis=1))
    kda = gate == "kda"
    recs = []
    for c in range(r):
        kt = np.zeros((n, 128), np.float32)
        kt[np.arange(n), b["comp_idx"][:, c]] = 1.0
        a = np.ones((n, 128) if kda else (n,), np.float32)
        recs.append((a, kt, -b["comp_val"][:, c].astype(np.float32)))
    st = lq.LeapQuantState(n, p, r, gate, DEV, lq.LQ_NO_SMOOTH)
    upload_boundary(st, b)
    _upload_records(st, recs, gate)
    S_prev = O.replay(O.dequantize(b), _oracle_records(recs, gate))
    mag_recs = _oracle_records(recs, gate)
    if fused:
        tok = _token(rng, n, gate)
        tok["beta"][:] = 0.0
        tok["alpha"][:] = 1.0
        o = torch.empty((n, 128), device=DEV)
        lq.leapquant_decode_close(st, r, *[_dev(tok[x]) for x in ("q", "k", "v", "beta", "alpha")], o)
        t64 = {k: v.astype(np.float64) for k, v in tok.items()}
        o_ref, S_end, rec_t = O.step(S_prev, t64["q"], t64["k"], t64["v"], t64["beta"], t64["alpha"],
                                     _gate(gate))
        mag_recs = mag_recs + [rec_t]
    else:
        lq.leapquant_window_close(st, r)
        S_end = S_prev
    torch.cuda.synchronize()
    if fused:
        P.assert_close(to_np(o), o_ref, "o_t")
    stats = P.compare_boundary(boundary_np(st), O.quantize(S_end, r, O.NO_SMOOTH), S_end.astype(np.float32), r,
                               "close near ties", flags=O.NO_SMOOTH, mag=P.rebuild_magnitude(b, mag_recs))
    print(f"{gate} r={r} fused={fused}: {stats['ties']} of {n} states ranked the tied rows the other way")
    assert stats["ties"] > 0, "no near tie was exercised"
