"""[EL] Figure 3 analogue at the long-decode workload's scale.

[EL] Figure 3 plots the recurrent state's error over 64K tokens for
per-token against per-window quantization, with per-window staying below.
Here all 128 states of the long-decode workload (16 heads x batch 8, 65,536
tokens) run three ways on the GPU:
  * the method: windows of p = 16, r = 4 compensator rows, smoothing;
  * per-token quantization: p = 1, r = 0, no smoothing (the INT8 per-step
    row of [EL] Table 2): the whole state is re-quantized after every token;
  * the exact fp32 recurrence: the dense fp32 per-step kernel.
Every 1,024 tokens the mean squared error of each quantized path's boundary
state (dequantized) against the exact state is taken over all states; the
method's must stay below the per-token path's at every checkpoint.  The
fp32 reference itself is checked against the oracle's fp64 recurrence on
sampled states: its own error must be negligible next to the quantization
error it measures.  Both curves are printed (and logged to
$LQ_PARITY_LOG).  The pages print no values for the figure: only the
ordering is pinned.
"""
import json
import os

import numpy as np
import pytest
import torch

import recurrent_state_quant_amd as lq
from oracle import leapquant_oracle as O
from workloads import generators as G
from workloads.configs import WORKLOADS

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_per_window_state_error_below_per_token_64k():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    cfg = WORKLOADS["gdn_long64k_h16_b8"]
    n, T, every = cfg.n_states, cfg.steps, cfg.snapshot_every
    g = G.make_generator(cfg.seed, DEV)
    S0 = G.initial_state(cfg, n, g, DEV)
    tok = G.token_inputs(cfg, n, T, g, DEV)

    method = lq.LeapQuantState(n, cfg.p, cfg.r, cfg.gate, DEV)
    per_token = lq.LeapQuantState(n, 1, 0, cfg.gate, DEV, lq.LQ_NO_SMOOTH)
    lq.leapquant_quantize_state(method, S0)
    lq.leapquant_quantize_state(per_token, S0)
    exact = S0.clone()
    o_m = torch.empty((n, cfg.dv), device=DEV)
    o_t = torch.empty_like(o_m)
    o_e = torch.empty_like(o_m)
    B = torch.empty((n, cfg.dk, cfg.dv), device=DEV)

    # the oracle's fp64 recurrence on sampled states, for the reference check
    sample = np.array([0, 37, 90, 127])
    sidx = torch.as_tensor(sample, device=DEV)
    S64 = S0.index_select(0, sidx).double().cpu().numpy()

    curve = []
    ref_err = 0.0
    for t in range(T):
        args = (tok["q"][t], tok["k"][t], tok["v"][t], tok["beta"][t], tok["alpha"][t])
        j = t % cfg.p
        if j == cfg.p - 1:
            lq.leapquant_decode_close(method, j, *args, o_m)
        else:
            lq.leapquant_decode_step(method, j, *args, o_m)
        lq.leapquant_decode_close(per_token, 0, *args, o_t)
        lq.leapquant_dense_step(exact, cfg.gate, *args, o_e)
        if (t + 1) % every == 0:
            lq.leapquant_dequantize_state(method, B)
            mse_m = ((B - exact) ** 2).mean().item()
            lq.leapquant_dequantize_state(per_token, B)
            mse_t = ((B - exact) ** 2).mean().item()
            curve.append((t + 1, mse_m, mse_t))
        if (t + 1) % (16 * every) == 0:
            # fp64 recurrence for the sampled states up to this token
            t0 = t + 1 - 16 * every
            tk = {k: v[t0:t + 1].index_select(1, sidx).double().cpu().numpy() for k, v in tok.items()}
            _, S64, _ = O.sequential_exact(S64, tk, O.GATE_GDN)
            E = exact.index_select(0, sidx).double().cpu().numpy()
            ref_err = max(ref_err, float(((E - S64) ** 2).mean()))
    torch.cuda.synchronize()

    for tt, mm, mt in curve:
        print(f"tokens {tt:6d}: state MSE per-window {mm:.4e}  per-token {mt:.4e}  ratio {mt / mm:.2f}")
    print(f"fp32 reference vs fp64 oracle on {len(sample)} states: largest MSE {ref_err:.3e}")
    path = os.environ.get("LQ_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps({"what": "fig3 state MSE", "curve": curve, "reference_mse": ref_err}) + "\n")
    smallest = min(mm for _, mm, _ in curve)
    assert ref_err <= 1e-3 * smallest, f"fp32 reference error {ref_err:.3e} is not negligible"
    worse = [(tt, mm, mt) for tt, mm, mt in curve if not mm < mt]
    assert not worse, f"per-window state MSE not below per-token at {worse[:4]}"
