"""Drive the HIP path through the Python binding of the C ABI (GPU tests only)."""
import numpy as np
import torch

import recurrent_state_quant_amd as lq


def to_np(x):
    return x.detach().cpu().numpy()


def boundary_np(state, idx=None):
    """Boundary state of the slab (or of states idx) as numpy arrays, codes
    as row-major matrices."""
    return {k: to_np(v) for k, v in state.boundary(idx).items()}


def upload_boundary(state, b, idx=None):
    """Write boundary arrays (numpy, codes as row-major matrices) into the
    slab, optionally for states idx."""
    state.load_boundary({k: np.ascontiguousarray(b[k]) for k in state.boundary_keys}, idx)


def tokens_np(tok, idx=None, t0=0, t1=None):
    """Host fp64 copies of per-token inputs [T, n, ...] for states idx."""
    out = {}
    for k, v in tok.items():
        x = v[t0:t1]
        if idx is not None:
            x = x.index_select(1, torch.as_tensor(idx, device=x.device, dtype=torch.long))
        out[k] = to_np(x).astype(np.float64)
    return out


def run_window(state, tok, t0, length, out, close=True, lo=0, hi=None, fused=False):
    """Decode tokens t0 .. t0+length-1 of `tok` (device tensors [T, n_total,
    ...]) for the slab's states lo .. hi-1 of the token arrays, writing o into
    out[t] [n_total, dv] (same state range), then close the window; with
    fused=True the last token is decoded and the window closed in one call
    (leapquant_decode_close)."""
    hi = lo + state.n if hi is None else hi
    for j in range(length):
        t = t0 + j
        args = (tok["q"][t, lo:hi], tok["k"][t, lo:hi], tok["v"][t, lo:hi],
                tok["beta"][t, lo:hi], tok["alpha"][t, lo:hi], out[t, lo:hi])
        if fused and close and j == length - 1:
            lq.leapquant_decode_close(state, j, *args)
            return
        lq.leapquant_decode_step(state, j, *args)
    if close:
        lq.leapquant_window_close(state, length)
