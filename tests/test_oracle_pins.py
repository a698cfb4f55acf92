"""Pins that tie the CPU oracle to what the pages and mathematics fix.

Each test names the passage it follows.  Page abbreviations:
  [EL] "LeapQuant: Efficient Linear Attention with Accurate Recurrent State
       Quantization" (paper listing page)
  [TM] "LeapQuant trims the memory burden of linear-attention models"
None of these tests needs a GPU.
"""
import glob
import json
import os

import numpy as np
import pytest
import torch

from oracle import leapquant_oracle as O
from tests import brute
from workloads import generators as G
from workloads.configs import WORKLOADS, WorkloadConfig

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _hx(x):
    return float.fromhex(x) if isinstance(x, str) else float(x)


def _rand_tokens(rng, T, n, dk, dv, kda, alpha_lo=0.05, alpha_hi=1.0):
    q = rng.standard_normal((T, n, dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((T, n, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, n, dv))
    beta = rng.uniform(0.05, 1.0, (T, n))
    alpha = rng.uniform(alpha_lo, alpha_hi, (T, n, dk) if kda else (T, n))
    return {"q": q, "k": k, "v": v, "beta": beta, "alpha": alpha}


# ---------------------------------------------------------------------------
# [EL] Appendix Table 4: closed forms of the recurrence instances
# ---------------------------------------------------------------------------
def test_gated_deltanet_closed_form():
    """Gated DeltaNet row: S_t = alpha (I - beta k k^T) S + beta k v^T, o = S_t^T q.

    dk != dv so a transposed state or operand cannot pass."""
    rng = np.random.default_rng(1)
    n, dk, dv = 3, 5, 3
    S = rng.standard_normal((n, dk, dv))
    tok = _rand_tokens(rng, 1, n, dk, dv, kda=False)
    o, S1, rec = O.step(S, tok["q"][0], tok["k"][0], tok["v"][0], tok["beta"][0], tok["alpha"][0], O.GATE_GDN)
    for s in range(n):
        a, b_ = tok["alpha"][0][s], tok["beta"][0][s]
        k = tok["k"][0][s]
        want = a * (np.eye(dk) - b_ * np.outer(k, k)) @ S[s] + b_ * np.outer(k, tok["v"][0][s])
        np.testing.assert_allclose(S1[s], want, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(o[s], want.T @ tok["q"][0][s], rtol=1e-13, atol=1e-14)
        # record = (d, k~, u) with u = v - S^T (alpha k): [EL] Table 4 last column
        np.testing.assert_allclose(rec[1][s], b_ * k, rtol=1e-15)
        np.testing.assert_allclose(rec[2][s], tok["v"][0][s] - S[s].T @ (a * k), rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(rec[0][s], np.full(dk, a), rtol=0)


def test_deltanet_row_is_gdn_with_unit_gate():
    """DeltaNet row (D = I, b = k): S - beta k (k^T S) + beta k v^T."""
    rng = np.random.default_rng(2)
    n, dk, dv = 2, 4, 6
    S = rng.standard_normal((n, dk, dv))
    tok = _rand_tokens(rng, 1, n, dk, dv, kda=False)
    alpha = np.ones(n)
    _, S1, _ = O.step(S, tok["q"][0], tok["k"][0], tok["v"][0], tok["beta"][0], alpha, O.GATE_GDN)
    for s in range(n):
        k, b_ = tok["k"][0][s], tok["beta"][0][s]
        want = S[s] - b_ * np.outer(k, k @ S[s]) + b_ * np.outer(k, tok["v"][0][s])
        np.testing.assert_allclose(S1[s], want, rtol=1e-13, atol=1e-14)


def test_kda_closed_form():
    """Kimi Delta Attention (named in [EL] Abstract; channel-wise decay):
    S_t = (I - beta k k^T) Diag(alpha) S + beta k v^T."""
    rng = np.random.default_rng(3)
    n, dk, dv = 2, 6, 4
    S = rng.standard_normal((n, dk, dv))
    tok = _rand_tokens(rng, 1, n, dk, dv, kda=True)
    o, S1, _ = O.step(S, tok["q"][0], tok["k"][0], tok["v"][0], tok["beta"][0], tok["alpha"][0], O.GATE_KDA)
    for s in range(n):
        k, b_, al = tok["k"][0][s], tok["beta"][0][s], tok["alpha"][0][s]
        want = (np.eye(dk) - b_ * np.outer(k, k)) @ np.diag(al) @ S[s] + b_ * np.outer(k, tok["v"][0][s])
        np.testing.assert_allclose(S1[s], want, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(o[s], want.T @ tok["q"][0][s], rtol=1e-13, atol=1e-14)


def test_kda_with_equal_channels_is_gdn():
    rng = np.random.default_rng(4)
    n, dk, dv = 3, 8, 5
    S = rng.standard_normal((n, dk, dv))
    tok = _rand_tokens(rng, 1, n, dk, dv, kda=False)
    a_diag = np.repeat(tok["alpha"][0][:, None], dk, axis=1)
    o1, S1, _ = O.step(S, tok["q"][0], tok["k"][0], tok["v"][0], tok["beta"][0], tok["alpha"][0], O.GATE_GDN)
    o2, S2, _ = O.step(S, tok["q"][0], tok["k"][0], tok["v"][0], tok["beta"][0], a_diag, O.GATE_KDA)
    np.testing.assert_allclose(S1, S2, rtol=1e-15, atol=0)
    np.testing.assert_allclose(o1, o2, rtol=1e-15, atol=0)


def test_zero_decay_forgets_state():
    """alpha = 0: D = 0 and b = 0, so S_t = beta k v^T whatever S_{t-1} was."""
    rng = np.random.default_rng(5)
    n, dk, dv = 2, 4, 3
    S = rng.standard_normal((n, dk, dv)) * 100
    tok = _rand_tokens(rng, 1, n, dk, dv, kda=False)
    o, S1, _ = O.step(S, tok["q"][0], tok["k"][0], tok["v"][0], tok["beta"][0], np.zeros(n), O.GATE_GDN)
    for s in range(n):
        kq = tok["beta"][0][s] * tok["k"][0][s] @ tok["q"][0][s]
        np.testing.assert_allclose(o[s], kq * tok["v"][0][s], rtol=1e-14, atol=1e-15)


# ---------------------------------------------------------------------------
# Quantizer: hand-derived fixtures, error bound, invariants
# ---------------------------------------------------------------------------
QUANT_FIXTURES = sorted(f for f in glob.glob(os.path.join(GOLDEN, "quant_*.json")))


@pytest.mark.parametrize("path", QUANT_FIXTURES, ids=[os.path.basename(p) for p in QUANT_FIXTURES])
def test_quantizer_golden(path):
    fx = json.load(open(path))
    S = np.asarray(fx["S"], np.float32)[None]
    b = O.quantize(S, fx["r"], fx["flags"])
    e = fx["expect"]
    dv = S.shape[2]
    np.testing.assert_array_equal(b["comp_idx"][0], np.asarray(e["comp_idx"], np.int32))
    np.testing.assert_array_equal(b["comp_val"][0], np.asarray(e["comp_val"], np.float32).reshape(-1, dv))
    np.testing.assert_array_equal(b["col_scale"][0], np.asarray([_hx(x) for x in e["col_scale"]], np.float32))
    np.testing.assert_array_equal(b["row_scale"][0], np.asarray([_hx(x) for x in e["row_scale"]], np.float32))
    np.testing.assert_array_equal(b["codes"][0], np.asarray(e["codes"], np.int8))


def _random_states(rng, n, dk, dv, outliers=True):
    S = (0.02 * rng.standard_normal((n, dk, dv))).astype(np.float32)
    if outliers:
        for s in range(n):
            rows = rng.choice(dk, 3, replace=False)
            cols = rng.choice(dv, 2, replace=False)
            S[s, rows] *= rng.uniform(10, 30, (3, 1)).astype(np.float32)
            S[s, :, cols] *= rng.uniform(10, 30, (2, 1)).astype(np.float32)
    return S


@pytest.mark.parametrize("r,flags", [(0, 0), (4, 0), (8, 0), (4, O.NO_SMOOTH)])
def test_half_step_bound(r, flags):
    """|R - c a s| <= (a s / 2)(1 + 1e-4) for every residual entry; compensator
    rows reproduce the fp32 state exactly.  The 1e-4 slack covers the five
    fp32 roundings between R and the rounded code (each <= 2^-24 relative,
    times |code| <= 127): 0.5 + 127 * 5 * 2^-24 < 0.5 (1 + 1e-4)."""
    rng = np.random.default_rng(10 + r)
    S = _random_states(rng, 6, 128, 128)
    b = O.quantize(S, r, flags)
    B = O.dequantize(b)
    for s in range(S.shape[0]):
        comp = set(b["comp_idx"][s].tolist())
        for i in range(128):
            if i in comp:
                np.testing.assert_array_equal(B[s, i], S[s, i].astype(np.float64))
                continue
            step_ = b["row_scale"][s, i].astype(np.float64) * b["col_scale"][s].astype(np.float64)
            err = np.abs(S[s, i].astype(np.float64) - B[s, i])
            assert np.all(err <= 0.5 * step_ * (1 + 1e-4) + 0.0), (s, i, (err / step_).max())


def test_extraction_and_smoothing_invariants():
    rng = np.random.default_rng(20)
    S = _random_states(rng, 8, 128, 128)
    r = 4
    b = O.quantize(S, r)
    for s in range(S.shape[0]):
        norms = np.linalg.norm(S[s].astype(np.float64), axis=1)
        idx = b["comp_idx"][s]
        rest = np.setdiff1d(np.arange(128), idx)
        # every extracted row is at least as large as every residual row
        assert norms[idx].min() >= norms[rest].max()
        # stored in descending-norm order
        assert np.all(np.diff(norms[idx]) <= 0)
        R = S[s].copy()
        R[idx] = 0
        # smoothing scale is the residual column absmax, so each smoothed
        # nonzero column peaks at magnitude 1 (up to one reciprocal rounding)
        np.testing.assert_array_equal(b["col_scale"][s], np.abs(R).max(axis=0))
        sm = np.abs(R.astype(np.float64) / b["col_scale"][s].astype(np.float64)).max(axis=0)
        np.testing.assert_allclose(sm, 1.0, rtol=2e-7)
        # every nonzero residual row uses the full code range
        c = b["codes"][s].astype(np.int32)
        assert np.all(np.abs(c[rest]).max(axis=1) == 127)
        assert np.all(c[idx] == 0)
        assert c.min() >= -127


def test_config0_planted_rows_are_extracted():
    """The four x20 rows planted in the single-head workload are exactly the
    compensator rows of the first boundary state ([EL] Abstract: compensators
    keep the largest outliers)."""
    cfg = WORKLOADS["gdn_single_head_b1"]
    g = G.make_generator(cfg.seed, "cpu")
    S = G.initial_state(cfg, 1, g, "cpu").numpy()
    norms = np.linalg.norm(S[0].astype(np.float64), axis=1)
    planted = np.nonzero(norms > 5 * np.median(norms))[0]
    assert len(planted) == 4
    b = O.quantize(S, cfg.r)
    assert sorted(b["comp_idx"][0].tolist()) == sorted(planted.tolist())


# ---------------------------------------------------------------------------
# Per-window quantization ([EL] Figure 2)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("kda", [False, True])
@pytest.mark.parametrize("p", [1, 2, 5, 16])
def test_windowing_without_quantization_is_exact(kda, p):
    """With the quantizer switched off, windowed decode equals the sequential
    recurrence: windowing changes nothing but where rounding enters."""
    rng = np.random.default_rng(30 + p)
    n, dk, dv, T = 3, 16, 12, 37
    S0 = rng.standard_normal((n, dk, dv))
    tok = _rand_tokens(rng, T, n, dk, dv, kda)
    gate = O.GATE_KDA if kda else O.GATE_GDN
    o_ref, S_ref, _ = O.sequential_exact(S0, tok, gate)
    o_w, bounds = O.run_windowed(S0, tok, p, 0, gate, quantizer=False)
    np.testing.assert_allclose(o_w, o_ref, rtol=1e-12, atol=1e-13)
    last = bounds[max(bounds)]
    np.testing.assert_allclose(last, S_ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("kda", [False, True])
def test_window_of_one_is_per_token_quantization(kda):
    """p = 1, r = 0 reduces per-window quantization to the per-token baseline
    that re-quantizes after every update ([EL] Figure 2)."""
    rng = np.random.default_rng(40)
    n, dk, dv, T = 2, 16, 16, 25
    S0 = _random_states(rng, n, dk, dv)
    tok = _rand_tokens(rng, T, n, dk, dv, kda)
    gate = O.GATE_KDA if kda else O.GATE_GDN
    o_w, bounds = O.run_windowed(S0, tok, 1, 0, gate)
    o_p, b_last = O.run_per_token(S0, tok, 0, gate)
    np.testing.assert_allclose(o_w, o_p, rtol=1e-13, atol=1e-14)
    np.testing.assert_array_equal(bounds[T]["codes"], b_last["codes"])


def test_worked_window_example():
    fx = json.load(open(os.path.join(GOLDEN, "window_gdn_p2.json")))
    S0 = np.asarray(fx["S_init"], np.float64)[None]
    tok = {k: np.asarray(v, np.float64) for k, v in fx["tokens"].items()}
    gate = O.GATE_GDN if fx["gate"] == "gdn" else O.GATE_KDA
    outs, bounds = O.run_windowed(S0, tok, fx["p"], fx["r"], gate, fx["flags"])
    want = np.asarray([[[_hx(x) for x in row] for row in t] for t in fx["expect"]["outputs"]])
    np.testing.assert_array_equal(outs, want)
    for w in (0, 1):
        e = fx["expect"][f"boundary_{w}"]
        np.testing.assert_array_equal(bounds[w]["codes"][0], np.asarray(e["codes"], np.int8))
        np.testing.assert_array_equal(bounds[w]["row_scale"][0],
                                      np.asarray([_hx(x) for x in e["row_scale"]], np.float32))


@pytest.mark.parametrize("kda", [False, True])
@pytest.mark.parametrize("dk,dv,p,r", [(2, 2, 1, 0), (3, 4, 2, 1), (4, 3, 3, 2), (8, 8, 5, 2), (8, 4, 2, 0)])
def test_brute_force_tiny_heads(kda, dk, dv, p, r):
    """Independent dense brute force (explicit A_t, scalar-loop quantizer,
    full sort) agrees with the oracle on tiny heads: outputs to 1e-12,
    codes, scales and compensators exactly."""
    rng = np.random.default_rng(dk * 100 + dv * 10 + p + r)
    n, T = 2, 11
    S0 = (rng.standard_normal((n, dk, dv)) * 0.3).astype(np.float32)
    tok = _rand_tokens(rng, T, n, dk, dv, kda)
    gate = O.GATE_KDA if kda else O.GATE_GDN
    outs, bounds = O.run_windowed(S0, tok, p, r, gate)
    for s in range(n):
        a_s = tok["alpha"][:, s]
        bo, bb = brute.brute_windowed(S0[s], tok["q"][:, s], tok["k"][:, s], tok["v"][:, s],
                                      tok["beta"][:, s], a_s, p, r, kda)
        np.testing.assert_allclose(outs[:, s], bo, rtol=1e-12, atol=1e-13)
        for w, (codes, a, sc, idx, wv) in enumerate(bb):
            ob = bounds[w]
            np.testing.assert_array_equal(ob["codes"][s], np.asarray(codes, np.int8))
            np.testing.assert_array_equal(ob["row_scale"][s], np.asarray(a, np.float32))
            np.testing.assert_array_equal(ob["col_scale"][s], np.asarray(sc, np.float32))
            np.testing.assert_array_equal(ob["comp_idx"][s], np.asarray(idx, np.int32))
            np.testing.assert_array_equal(ob["comp_val"][s], np.asarray(wv, np.float32).reshape(r, dv))


def test_per_window_beats_per_token_state_error():
    """Qualitative claim of [EL] Figure 3: quantizing once per window keeps the
    state closer to the exact recurrence than quantizing every token.  The
    pages print no values, so only the ordering is checked."""
    cfg = WorkloadConfig("mse_gdn_h4_b1", "gdn", 1, 4, 1, 256, 16, 4, "pct1")
    g = G.make_generator(7, "cpu")
    S0 = G.initial_state(cfg, 4, g, "cpu").numpy()
    tok = {k: v.numpy().astype(np.float64) for k, v in G.token_inputs(cfg, 4, 256, g, "cpu").items()}
    _, S_exact, _ = O.sequential_exact(S0, tok, O.GATE_GDN)
    _, bw = O.run_windowed(S0, tok, 16, 4, O.GATE_GDN)
    _, bp = O.run_per_token(S0, tok, 0, O.GATE_GDN)
    mse_w = O.state_mse(bw[max(bw)], S_exact).mean()
    mse_p = O.state_mse(bp, S_exact).mean()
    assert mse_w < mse_p, (mse_w, mse_p)


def test_generators_match_recipe():
    """Input recipe: unit-norm q and k, beta in (0,1), alpha in (0,1)."""
    cfg = WORKLOADS["kda_h32_b128"]
    g = G.make_generator(0, "cpu")
    tok = G.token_inputs(cfg, 5, 4, g, "cpu")
    assert tok["alpha"].shape == (4, 5, 128)
    torch.testing.assert_close(torch.linalg.vector_norm(tok["q"], dim=-1), torch.ones(4, 5))
    torch.testing.assert_close(torch.linalg.vector_norm(tok["k"], dim=-1), torch.ones(4, 5))
    assert float(tok["beta"].min()) > 0 and float(tok["beta"].max()) < 1
    assert float(tok["alpha"].min()) > 0 and float(tok["alpha"].max()) < 1
    # same seed, same draws
    g2 = G.make_generator(0, "cpu")
    tok2 = G.token_inputs(cfg, 5, 4, g2, "cpu")
    for k in tok:
        assert torch.equal(tok[k], tok2[k])


# ---------------------------------------------------------------------------
# Dense "BF16 per-step" baseline ([EL] Table 2): bf16 rounding of the state
# ---------------------------------------------------------------------------
def test_round_bf16_fixed_points_and_ties():
    # representable values are kept; halfway cases go to the even significand
    assert O.round_bf16(np.array([1.0, -2.5, 0.0, 3.0 * 2.0 ** -20])).tolist() == [1.0, -2.5, 0.0, 3.0 * 2.0 ** -20]
    assert O.round_bf16(1.0 + 2.0 ** -8) == 1.0                       # tie, 1.0 is even
    assert O.round_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6       # tie, 1 + 2^-6 is even
    assert O.round_bf16(1.0 + 2.0 ** -8 + 2.0 ** -20) == 1.0 + 2.0 ** -7
    assert O.round_bf16(-(1.0 + 2.0 ** -8 + 2.0 ** -20)) == -(1.0 + 2.0 ** -7)


def test_round_bf16_matches_torch_and_nearest():
    """Against torch's float32 -> bfloat16 conversion (round to nearest
    even), and by brute force: no bf16 neighbour of x is closer."""
    rng = np.random.default_rng(11)
    x = (rng.standard_normal(20000) * np.exp(rng.uniform(-30, 30, 20000))).astype(np.float32)
    r = O.round_bf16(x)
    t = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(r, t)
    # neighbours: truncation and the next value up in magnitude
    bits = x.view(np.uint32) & np.uint32(0xFFFF0000)
    lo = bits.view(np.float32).astype(np.float64)
    hi = (bits + np.uint32(0x10000)).view(np.float32).astype(np.float64)
    xd = x.astype(np.float64)
    assert np.all(np.abs(r - xd) <= np.minimum(np.abs(lo - xd), np.abs(hi - xd)))


def test_dense_bf16_step_is_rounded_exact_step():
    rng = np.random.default_rng(12)
    S = O.round_bf16(0.1 * rng.standard_normal((3, 8, 8)))
    q, k, v = (rng.standard_normal((3, 8)) for _ in range(3))
    beta, alpha = rng.uniform(0.1, 1, 3), rng.uniform(0.1, 1, 3)
    o, S_new = O.step_dense_bf16(S, q, k, v, beta, alpha, O.GATE_GDN)
    o2, S2, _ = O.step(S, q, k, v, beta, alpha, O.GATE_GDN)
    np.testing.assert_array_equal(o, o2)
    assert np.all(np.abs(S_new - S2) <= 2.0 ** -8 * np.abs(S2) + 1e-300)
    np.testing.assert_array_equal(O.round_bf16(S_new), S_new)


# ---------------------------------------------------------------------------
# Other rows of [EL] Appendix Table 4 (b_t = 0: NO_DELTA), closed forms
# ---------------------------------------------------------------------------
def _rows_tokens(rng, T, n, dk, dv, kda):
    q = rng.standard_normal((T, n, dk))
    k = rng.standard_normal((T, n, dk))
    v = rng.standard_normal((T, n, dv))
    beta = np.ones((T, n))
    alpha = rng.uniform(0.3, 1.0, (T, n, dk) if kda else (T, n))
    return dict(q=q, k=k, v=v, beta=beta, alpha=alpha)


@pytest.mark.parametrize("row", ["linear", "retnet", "mamba2", "gla"])
def test_table4_rows_without_delta_closed_form(row):
    """S_T = (prod_t D_t) S_0 + sum_t (prod_{s>t} D_s) k_t v_t^T, written with
    cumulative products instead of the step loop; outputs o_t = S_t^T q_t."""
    rng = np.random.default_rng(40)
    T, n, dk, dv = 7, 3, 5, 4
    kda = row == "gla"
    tok = _rows_tokens(rng, T, n, dk, dv, kda)
    if row == "linear":
        tok["alpha"] = np.ones((T, n))
    elif row == "retnet":
        tok["alpha"] = np.full((T, n), 0.8)
    gate = O.GATE_KDA if kda else O.GATE_GDN
    S0 = rng.standard_normal((n, dk, dv))
    outs, S_T, _ = O.sequential_exact(S0, tok, gate, flags=O.NO_DELTA)
    a = tok["alpha"] if kda else np.repeat(tok["alpha"][:, :, None], dk, axis=2)   # [T, n, dk]
    for t_end in range(1, T + 1):
        tail = lambda t: np.prod(a[t + 1:t_end], axis=0) if t + 1 < t_end else np.ones((n, dk))
        S = np.prod(a[:t_end], axis=0)[:, :, None] * S0
        for t in range(t_end):
            S = S + (tail(t) * tok["k"][t])[:, :, None] * tok["v"][t][:, None, :]
        np.testing.assert_allclose(np.einsum("nij,ni->nj", S, tok["q"][t_end - 1]), outs[t_end - 1],
                                   rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S, S_T, rtol=1e-12, atol=1e-12)


def test_delta_rule_writes_value_under_its_key():
    """DeltaNet row (alpha = 1, beta = 1, unit key): after the update the
    state maps the key exactly to the value, S_t^T k_t = v_t."""
    rng = np.random.default_rng(41)
    n, dk, dv = 4, 6, 5
    S = rng.standard_normal((n, dk, dv))
    k = rng.standard_normal((n, dk)); k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((n, dv))
    _, S1, _ = O.step(S, k, k, v, np.ones(n), np.ones(n), O.GATE_GDN)
    np.testing.assert_allclose(np.einsum("nij,ni->nj", S1, k), v, rtol=1e-12, atol=1e-12)
    # without the delta correction the same update only adds k v^T
    _, S2, _ = O.step(S, k, k, v, np.ones(n), np.ones(n), O.GATE_GDN, O.NO_DELTA)
    np.testing.assert_allclose(S2, S + k[:, :, None] * v[:, None, :], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("kda", [False, True])
def test_windowing_is_exact_without_delta(kda):
    """P1 for the NO_DELTA rows: with the quantizer off, windows reproduce the
    plain recurrence."""
    rng = np.random.default_rng(42)
    T, n, dk, dv = 11, 2, 6, 5
    tok = _rows_tokens(rng, T, n, dk, dv, kda)
    gate = O.GATE_KDA if kda else O.GATE_GDN
    S0 = rng.standard_normal((n, dk, dv))
    o_ref, S_ref, _ = O.sequential_exact(S0, tok, gate, flags=O.NO_DELTA)
    o_w, b = O.run_windowed(S0, tok, 4, 0, gate, flags=O.NO_DELTA, quantizer=False)
    np.testing.assert_allclose(o_w, o_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(b[max(b)], S_ref, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# "BF16 + per-window" ([EL] Table 2): a bf16 boundary state, fp32 records
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("kda", [False, True])
def test_bf16_window_of_one_is_bf16_per_step(kda):
    """With p = 1 the state is rounded to bf16 after every token: exactly the
    "BF16 per-step" row."""
    rng = np.random.default_rng(4100 + kda)
    T, n, dk, dv = 9, 3, 128, 128
    tok = _rand_tokens(rng, T, n, dk, dv, kda)
    gate = O.GATE_KDA if kda else O.GATE_GDN
    S0 = 0.1 * rng.standard_normal((n, dk, dv))
    o_w, bounds = O.run_windowed_bf16(S0, tok, 1, gate)
    S = O.round_bf16(S0)
    for t in range(T):
        o, S = O.step_dense_bf16(S, tok["q"][t], tok["k"][t], tok["v"][t], tok["beta"][t], tok["alpha"][t], gate)
        np.testing.assert_array_equal(o_w[t], o)
        np.testing.assert_array_equal(bounds[t + 1], S)


def test_bf16_window_boundaries_are_bf16_and_outputs_exact():
    """Boundary states hold bf16 values; inside a window the outputs are the
    exact recurrence from the boundary (nothing is rounded mid-window)."""
    rng = np.random.default_rng(4200)
    T, n, p = 12, 2, 4
    tok = _rand_tokens(rng, T, n, 128, 128, False)
    S0 = 0.1 * rng.standard_normal((n, 128, 128))
    o_w, bounds = O.run_windowed_bf16(S0, tok, p, O.GATE_GDN)
    for B in bounds:
        np.testing.assert_array_equal(O.round_bf16(B), B)
    for w in range(T // p):
        o_ref, _, _ = O.sequential_exact(bounds[w], {k: v[w * p:(w + 1) * p] for k, v in tok.items()}, O.GATE_GDN)
        np.testing.assert_allclose(o_w[w * p:(w + 1) * p], o_ref, rtol=1e-12, atol=1e-12)


def test_bf16_per_window_error_below_per_step():
    """The qualitative claim behind the row ([EL] Table 2, per-window bf16
    close to fp32): rounding once per window accumulates less state error
    than rounding after every token."""
    rng = np.random.default_rng(4300)
    T, n = 64, 2
    tok = _rand_tokens(rng, T, n, 128, 128, False, alpha_lo=0.9, alpha_hi=1.0)
    S0 = 0.1 * rng.standard_normal((n, 128, 128))
    _, S_exact, _ = O.sequential_exact(S0, tok, O.GATE_GDN)
    _, bw = O.run_windowed_bf16(S0, tok, 16, O.GATE_GDN)
    _, bs = O.run_windowed_bf16(S0, tok, 1, O.GATE_GDN)
    err_w = np.mean((bw[-1] - S_exact) ** 2)
    err_s = np.mean((bs[-1] - S_exact) ** 2)
    assert err_w < err_s, (err_w, err_s)


# ---------------------------------------------------------------------------
# Helpers the GPU comparisons rely on
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dense", [False, True])
def test_prerounding_codes_round_to_the_codes(dense):
    """prerounding_codes gives the values quantize rounds: rounding them
    (half to even, clamped) reproduces the codes exactly, for row and dense
    compensators."""
    rng = np.random.default_rng(4400 + dense)
    S = _random_states(rng, 5, 128, 128)
    b = O.quantize(S, 4, O.DENSE_COMP if dense else 0, 2)
    x = O.prerounding_codes(S, b)
    np.testing.assert_array_equal(np.clip(np.rint(x), -127, 127).astype(np.int8), b["codes"])


@pytest.mark.parametrize("kda", [False, True])
def test_replay_of_window_records_is_the_window_state(kda):
    """Applying a window's buffered records (d_i, k~_i, u_i) to its boundary
    state gives the window's end state: the algebra every GPU test uses to
    build the oracle's state from records."""
    rng = np.random.default_rng(4500 + kda)
    T, n = 7, 3
    tok = _rand_tokens(rng, T, n, 128, 128, kda)
    gate = O.GATE_KDA if kda else O.GATE_GDN
    b = O.quantize(_random_states(rng, n, 128, 128), 4)
    _, recs, S_end, _ = O.window(b, tok, 0, T, gate, 4)
    np.testing.assert_allclose(O.replay(O.dequantize(b), recs), S_end, rtol=1e-12, atol=1e-12)


def test_state_mse_is_bounded_by_the_half_step():
    """state_mse of a fresh split against the state it splits is at most the
    mean squared half step (a s / 2)^2 of the codes (up to fp32 rounding)."""
    rng = np.random.default_rng(4600)
    S = _random_states(rng, 4, 128, 128)
    b = O.quantize(S, 4)
    mse = O.state_mse(b, S.astype(np.float64))
    half = 0.5 * b["row_scale"].astype(np.float64)[:, :, None] * b["col_scale"].astype(np.float64)[:, None, :]
    assert np.all(mse <= (half ** 2).mean(axis=(1, 2)) * (1 + 1e-3))
    assert np.all(mse > 0)
