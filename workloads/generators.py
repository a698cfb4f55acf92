"""Seeded input generators (draws only; no LeapQuant arithmetic here).

Distributions follow the workload descriptions: q and k are standard normal
vectors scaled to unit L2 norm, v is standard normal, the write strength is
beta = sigmoid(N(0,1)) and the decay is alpha = exp(-softplus(N(0,1))), one per
state (Gated DeltaNet) or one per key channel (Kimi Delta Attention).  The
initial state is 0.02 * N(0,1) with planted outlier rows and columns.

Draw order, from one torch.Generator seeded with the workload seed:
  1. the initial state: the N(0,1) block, then the outlier draws;
  2. for every token t in order: q_t, k_t, v_t, beta_t, alpha_t.
Generation runs on whatever device the caller names; the oracle is given the
exact tensors (copied to the host), so host and device generators need not
agree with each other.
"""
import torch

from .configs import WorkloadConfig


def make_generator(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def initial_state(cfg: WorkloadConfig, n: int, gen: torch.Generator, device) -> torch.Tensor:
    """fp32 [n, dk, dv] initial state with the workload's planted outliers."""
    dk, dv = cfg.dk, cfg.dv
    S = torch.randn((n, dk, dv), generator=gen, device=device, dtype=torch.float32)
    S.mul_(0.02)
    if cfg.outliers == "rows4x20":
        for s in range(n):
            rows = torch.randperm(dk, generator=gen, device=device)[:4]
            S[s, rows, :] *= 20.0
    elif cfg.outliers == "pct1":
        u_row = torch.rand((n, dk), generator=gen, device=device)
        f_row = torch.rand((n, dk), generator=gen, device=device) * 20.0 + 10.0
        u_col = torch.rand((n, dv), generator=gen, device=device)
        f_col = torch.rand((n, dv), generator=gen, device=device) * 20.0 + 10.0
        row_f = torch.where(u_row < 0.01, f_row, torch.ones_like(f_row))
        col_f = torch.where(u_col < 0.01, f_col, torch.ones_like(f_col))
        S.mul_(row_f[:, :, None])
        S.mul_(col_f[:, None, :])
    elif cfg.outliers != "none":
        raise ValueError(f"unknown outlier recipe {cfg.outliers!r}")
    return S


def token_inputs(cfg: WorkloadConfig, n: int, steps: int, gen: torch.Generator, device) -> dict:
    """Per-token inputs for `steps` tokens and `n` states.

    Returns fp32 tensors q [T,n,dk], k [T,n,dk], v [T,n,dv], beta [T,n] and
    alpha [T,n] (gdn) or [T,n,dk] (kda).  For each t the slice [t] is a
    contiguous [n, ...] block, so one decode call can read it directly.
    """
    dk, dv = cfg.dk, cfg.dv
    f32 = torch.float32
    q = torch.empty((steps, n, dk), device=device, dtype=f32)
    k = torch.empty((steps, n, dk), device=device, dtype=f32)
    v = torch.empty((steps, n, dv), device=device, dtype=f32)
    beta = torch.empty((steps, n), device=device, dtype=f32)
    a_shape = (steps, n) if cfg.gate == "gdn" else (steps, n, dk)
    alpha = torch.empty(a_shape, device=device, dtype=f32)
    for t in range(steps):
        torch.randn(q[t].shape, generator=gen, out=q[t])
        torch.randn(k[t].shape, generator=gen, out=k[t])
        torch.randn(v[t].shape, generator=gen, out=v[t])
        torch.randn(beta[t].shape, generator=gen, out=beta[t])
        torch.randn(alpha[t].shape, generator=gen, out=alpha[t])
    q.div_(torch.linalg.vector_norm(q, dim=-1, keepdim=True))
    k.div_(torch.linalg.vector_norm(k, dim=-1, keepdim=True))
    torch.sigmoid_(beta)
    # alpha = exp(-softplus(x)), evaluated chunk-wise to bound temporaries
    flat = alpha.view(-1)
    chunk = 1 << 26
    for s in range(0, flat.numel(), chunk):
        seg = flat[s:s + chunk]
        seg.copy_(torch.exp(-torch.nn.functional.softplus(seg)))
    return {"q": q, "k": k, "v": v, "beta": beta, "alpha": alpha}


def sample_states(tensors: dict, idx, to_host: bool = True) -> dict:
    """Select states `idx` (a list or 1-D tensor) along the state axis.

    Per-token tensors have the state axis at dim 1, the initial state and
    boundary-state arrays at dim 0; pass them in separate dicts.
    """
    out = {}
    for name, x in tensors.items():
        ii = torch.as_tensor(idx, dtype=torch.long, device=x.device)
        y = x.index_select(1 if x.dim() >= 2 and name in ("q", "k", "v", "beta", "alpha") else 0, ii)
        out[name] = y.cpu() if to_host else y
    return out
