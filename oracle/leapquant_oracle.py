"""LeapQuant CPU oracle -- TEST INFRASTRUCTURE ONLY.

This module is the plain, slow, fp64 reference that the HIP decode path is
checked against.  Only the test suite, the package's smoke check and the
benchmark's CPU-baseline leg may import it; the product path never does, and it
shares no code with the HIP kernels or their host library.

Sources (web pages about one preprint; cited by title and section):
  [EL] "LeapQuant: Efficient Linear Attention with Accurate Recurrent State
       Quantization" (paper listing page): Abstract, Figure 2, Figure 4,
       Appendix Table 4.
  [NL] "LeapQuant: Near-Lossless 8-Bit Recurrent State Quantization for Linear
       Attention LLMs" (summary card): Key points.
  [TM] "LeapQuant trims the memory burden of linear-attention models" (news
       write-up): section "Quantize less often, protect the outliers".

What is computed (all floating point in fp64 unless a step says fp32):

* The delta-rule recurrence, one instance per row of [EL] Appendix Table 4
  (the equation it instantiates is not printed; the only form that fits every
  row and its record size is used):
      u_t = v_t - S_{t-1}^T b_t,   S_t = D_t S_{t-1} + k~_t u_t^T,   o_t = S_t^T q_t
  with S in R^{dk x dv}.  Gated DeltaNet: D_t = alpha_t I, k~_t = beta_t k_t,
  b_t = alpha_t k_t.  Kimi Delta Attention (named in [EL] Abstract, absent from
  the table): D_t = Diag(alpha_t), k~_t = beta_t k_t, b_t = alpha_t * k_t.

* Per-window quantization ([EL] Abstract, Figure 2; [TM]): the quantized
  boundary state stays fixed for a window of p tokens; within the window the
  state evolves exactly from it (outputs are the exact recurrence started at
  the boundary state, which is what the buffered high-precision updates
  reproduce); after the p-th token the whole state is quantized once.  The
  oracle writes that definition out densely: no buffer algebra.

* Compensator Tokens ([EL] Abstract, Figure 4; [NL] Key points): r rows of the
  state kept in fp32; they are part of the boundary state, so they follow the
  same recurrence as everything else.  Extraction rule (not given by the
  pages; the reading taken here): the r rows of largest L2 norm, ties to the
  lower row index, stored in descending-norm order.

* Dense Compensator Tokens (flag DENSE_COMP; a second reading of the same
  passages): a compensator is a token (k_c, w_c) with a dense unit key k_c,
  entering the state as k_c w_c^T and updated exactly like the window's own
  tokens.  The keys approximate the span of the state's leading left
  singular vectors (the largest components, which [EL] Figure 4 assigns to
  the compensators): subspace iteration started from the one-hot keys of the
  r largest-norm rows, `iters` rounds of Y = S S^T K, K = MGS(Y) (modified
  Gram-Schmidt in compensator order; a column whose projected norm is at
  most 2e-2 of its norm before projection, or zero, becomes the zero key: a
  column kept with less would carry the rounding of S S^T K amplified by
  more than 50).
  Values w_c = S^T k_c from the fp32 keys, residual R = S - sum_c k_c w_c^T.
  With iters = 0 this is exactly the row extraction above.

* Residual smoothing ([EL] Abstract; [TM]): not specified by the pages; this
  build's reading is a per-value-column absmax scale s_j of the residual
  (after extraction), 1 for an all-zero column.

* 8-bit quantizer ([EL] Abstract, 8-bit state): symmetric int8 in [-127, 127]
  with one fp32 scale per row of the smoothed residual.  Every step that
  decides a code runs in fp32 (the format's precision and the kernel's), with
  correctly rounded IEEE operations in this exact order:
      sigma_j = 1/s_j;  q_ij = R_ij*sigma_j;  m_i = max_j |q_ij|;
      a_i = m_i/127;    inv_i = 127/m_i;      c_ij = clamp(rne(q_ij*inv_i), +-127)
  (a_i = inv_i = 0 and c_i = 0 for an all-zero row).  Dequantized value:
  c_ij * a_i * s_j (evaluated in fp64 here).

Parity pins (tests/test_oracle_pins.py): Table 4 closed forms for every row,
hand-derived quantizer fixtures (tests/golden/), the half-step error bound,
extraction/smoothing invariants, exact recurrence when quantization is off,
the p=1 reduction to per-token quantization, and a brute-force dense
implementation on tiny heads.  Dense compensator tokens
(tests/test_oracle_dense_comp.py): zero iterations equal the row
extraction, orthonormal keys and an orthogonal residual, convergence to the
SVD's leading subspace, LAPACK Householder QR of the same iterates on tiny
heads, the half-step bound of the reconstruction, rank-deficient states.  Parity unpinned: agreement with the authors'
own extraction and smoothing rules, which the pages do not state.
"""
import numpy as np

GATE_GDN = 0   # D_t = alpha_t I           (Gated DeltaNet row of Table 4)
GATE_KDA = 1   # D_t = Diag(alpha_t)       (Kimi Delta Attention reading)
NO_SMOOTH = 1  # flag: s_j = 1 (ablation of residual smoothing)
NO_DELTA = 2   # flag: b_t = 0, so u_t = v_t (the rows of Table 4 without the
               # delta correction: linear attention, RetNet, Mamba2, GLA family)
DENSE_COMP = 4  # flag: compensator tokens with dense keys (subspace iteration)
MGS_DROP = 2e-2  # relative projected norm at or below which a key is dropped

_F32 = np.float32


# --------------------------------------------------------------------------
# Recurrence ([EL] Appendix Table 4)
# --------------------------------------------------------------------------
def transition(gate, k, beta, alpha, dk, flags=0):
    """Return (d, k~, b) for a batch of states.

    d is the diagonal of D_t as an [n, dk] array.  Shapes: k [n, dk],
    beta [n], alpha [n] (GDN) or [n, dk] (KDA).  With NO_DELTA, b = 0.  The
    rows of [EL] Appendix Table 4 are: linear attention (alpha = 1, beta = 1,
    NO_DELTA), RetNet (alpha = gamma, beta = 1, NO_DELTA), Mamba2 (scalar
    alpha_t, beta = 1, NO_DELTA), GLA / RWKV6 / HGRN2 (per-channel alpha_t,
    beta = 1, NO_DELTA), DeltaNet (alpha = 1), Gated DeltaNet.
    """
    k = np.asarray(k, np.float64)
    beta = np.asarray(beta, np.float64)
    alpha = np.asarray(alpha, np.float64)
    n = k.shape[0]
    if gate == GATE_GDN:
        d = np.broadcast_to(alpha.reshape(n, 1), (n, dk))
    elif gate == GATE_KDA:
        d = alpha.reshape(n, dk)
    else:
        raise ValueError("unknown gate")
    kt = beta.reshape(n, 1) * k
    b = np.zeros_like(k) if flags & NO_DELTA else d * k
    return d, kt, b


def step(S, q, k, v, beta, alpha, gate, flags=0):
    """One exact token update on dense fp64 states S [n, dk, dv].

    Returns (o [n, dv], S_new [n, dk, dv], record) where record = (d, k~, u),
    the buffered update of [EL] Table 4's last column.
    """
    n, dk, dv = S.shape
    d, kt, b = transition(gate, k, beta, alpha, dk, flags)
    u = np.asarray(v, np.float64) - np.einsum("nij,ni->nj", S, b)
    S_new = d[:, :, None] * S + kt[:, :, None] * u[:, None, :]
    o = np.einsum("nij,ni->nj", S_new, np.asarray(q, np.float64))
    return o, S_new, (d.copy(), kt, u)


def replay(B, records):
    """State after applying buffered records (d_i, k~_i, u_i) to B in order."""
    S = np.array(B, np.float64, copy=True)
    for d, kt, u in records:
        S = np.asarray(d)[:, :, None] * S + np.asarray(kt)[:, :, None] * np.asarray(u)[:, None, :]
    return S


def sequential_exact(S0, tokens, gate, keep_every=0, flags=0):
    """Unquantized recurrence over all tokens (fp64).

    tokens: dict of arrays q [T,n,dk], k, v [T,n,dv], beta [T,n], alpha.
    Returns (outputs [T,n,dv], final state, {t: state after t tokens}) where
    states are kept every `keep_every` tokens (0: none).
    """
    S = np.array(S0, np.float64, copy=True)
    T = tokens["q"].shape[0]
    outs = np.empty((T,) + (S.shape[0], S.shape[2]))
    kept = {}
    for t in range(T):
        o, S, _ = step(S, tokens["q"][t], tokens["k"][t], tokens["v"][t],
                       tokens["beta"][t], tokens["alpha"][t], gate, flags)
        outs[t] = o
        if keep_every and (t + 1) % keep_every == 0:
            kept[t + 1] = S.copy()
    return outs, S, kept


# --------------------------------------------------------------------------
# Quantized boundary state ([EL] Abstract, Figure 4; [TM])
# --------------------------------------------------------------------------
def mgs(Y, ratios=None, keep=None):
    """Modified Gram-Schmidt on the columns of Y [dk, r] (fp64), in column
    order.  A column whose norm after projection is zero or at most MGS_DROP
    times its norm before projection gives a zero column.  If `ratios` is a
    list, the ratio (norm after projection) / (norm before) of every column
    is appended to it (0 for a zero column): a diagnostic only, the result
    does not depend on it.  `keep` ({column: bool}) overrides the decision
    for the columns it names (a nonzero projected column only): a test
    forces it where the ratio lies within rounding of the threshold, so
    either decision is correct."""
    dk, r = Y.shape
    K = np.zeros((dk, r))
    for c in range(r):
        v = Y[:, c].copy()
        n0 = np.sqrt(v @ v)
        for c2 in range(c):
            v = v - (K[:, c2] @ v) * K[:, c2]
        nv = np.sqrt(v @ v)
        if ratios is not None:
            ratios.append(nv / n0 if n0 > 0 else 0.0)
        kept = nv > 0 and nv > MGS_DROP * n0
        if keep is not None and c in keep and nv > 0:
            kept = bool(keep[c])
        if kept:
            K[:, c] = v / nv
    return K


def dense_keys(S64, start_rows, iters, ratios=None, keep=None):
    """Keys of the dense compensator tokens of one state: subspace iteration
    on S S^T from the one-hot keys of `start_rows` (fp64, [dk, r]).  With a
    list `ratios`, each round appends its list of MGS ratios (see mgs).
    `keep` ({(round, column): bool}) forces keep / drop decisions of mgs."""
    dk = S64.shape[0]
    K = np.zeros((dk, len(start_rows)))
    K[start_rows, np.arange(len(start_rows))] = 1.0
    for it in range(iters):
        rr = None if ratios is None else []
        kk = None if keep is None else {c: v for (i, c), v in keep.items() if i == it}
        K = mgs(S64 @ (S64.T @ K), rr, kk)
        if ratios is not None:
            ratios.append(rr)
    return K


def quantize(S, r, flags=0, iters=0, keys=None, rows=None, keep=None):
    """Split an fp32 state into compensator tokens + smoothed int8 residual.

    S: [n, dk, dv], values taken as fp32 (the reconstructed FP32 state of
    [EL] Figure 4).  Returns a dict with codes int8 [n,dk,dv], row_scale
    fp32 [n,dk], col_scale fp32 [n,dv], comp_idx int32 [n,r], comp_val fp32
    [n,r,dv]; with DENSE_COMP also comp_key fp32 [n,r,dk] (comp_idx then
    holds the rows the subspace iteration started from).  `keys` (fp32
    [n,r,dk], DENSE_COMP only) replaces the subspace iteration: the split
    into values, residual and codes is then made with these keys.  `rows`
    (int [n,r]) replaces the top-r selection of step 2 by the given rows, in
    the given order (the extraction is then forced; when two row norms are
    within rounding of each other, either choice is a correct top-r, and a
    test forces the oracle to the choice it checks).  `keep` (a list of one
    {(round, column): bool} per state, DENSE_COMP only) forces keep / drop
    decisions of the key iteration in the same way (see mgs).
    """
    S32 = np.asarray(S, dtype=_F32)
    n, dk, dv = S32.shape
    if not 0 <= r <= dk:
        raise ValueError("r out of range")
    # 1. row L2 norms (squared, fp64 sum of exact fp32 squares)
    S64 = S32.astype(np.float64)
    norm2 = np.einsum("nij,nij->ni", S64, S64)
    # 2. top-r rows: descending norm, ties to the lower index (stable sort)
    comp_idx = np.argsort(-norm2, axis=1, kind="stable")[:, :r].astype(np.int32)
    if rows is not None:
        comp_idx = np.array(rows, dtype=np.int32).reshape(n, r)
        if r and (comp_idx.min() < 0 or comp_idx.max() >= dk or
                  any(len(set(c.tolist())) != r for c in comp_idx)):
            raise ValueError("rows must be r distinct row indices per state")
    if flags & DENSE_COMP:
        # 3'. dense keys, values w_c = S^T k_c from the fp32 keys, and the
        # residual S - sum_c k_c w_c^T (fp64, rounded once to fp32)
        comp_key = np.zeros((n, r, dk), _F32)
        comp_val = np.zeros((n, r, dv), _F32)
        R = np.zeros_like(S32)
        for s in range(n):
            if keys is not None:
                K32 = np.asarray(keys[s], _F32).T
            else:
                K32 = dense_keys(S64[s], comp_idx[s], iters,
                                 keep=None if keep is None else keep[s]).astype(_F32)
            K = K32.astype(np.float64)
            W32 = (K.T @ S64[s]).astype(_F32)
            comp_key[s] = K32.T
            comp_val[s] = W32
            R[s] = (S64[s] - K @ W32.astype(np.float64)).astype(_F32)
    else:
        # 3. compensator rows keep their fp32 values
        comp_val = np.take_along_axis(S32, comp_idx[:, :, None].astype(np.int64), axis=1).copy()
        # 4. residual: extracted rows zeroed
        R = S32.copy()
        for s in range(n):
            R[s, comp_idx[s], :] = 0
    # 5. smoothing scale per value column (absmax of the residual column)
    if flags & NO_SMOOTH:
        col_scale = np.ones((n, dv), _F32)
    else:
        col_scale = np.abs(R).max(axis=1).astype(_F32)
        col_scale[col_scale == 0] = _F32(1)
    # 6. smoothed residual, fp32 multiply by the fp32 reciprocal
    sigma = (_F32(1) / col_scale).astype(_F32)
    Q = (R * sigma[:, None, :]).astype(_F32)
    # 7. per-row absmax scale and its reciprocal, fp32 divisions
    m = np.abs(Q).max(axis=2).astype(_F32)
    nz = m > 0
    row_scale = np.zeros((n, dk), _F32)
    inv = np.zeros((n, dk), _F32)
    row_scale[nz] = (m[nz] / _F32(127)).astype(_F32)
    inv[nz] = (_F32(127) / m[nz]).astype(_F32)
    # 8. codes: round half to even, clamp to the symmetric range
    X = (Q * inv[:, :, None]).astype(_F32)
    codes = np.clip(np.rint(X), -127, 127).astype(np.int8)
    out = {"codes": codes, "row_scale": row_scale, "col_scale": col_scale,
           "comp_idx": comp_idx, "comp_val": comp_val}
    if flags & DENSE_COMP:
        out["comp_key"] = comp_key
    return out


def prerounding_codes(S, boundary):
    """fp32 values that step 8 of `quantize` rounds, for a given selection.

    Used by tests to tell a code decided at a rounding boundary from a wrong
    one; the selection, scales and zeroed rows are taken from `boundary`.
    """
    S32 = np.asarray(S, dtype=_F32)
    n = S32.shape[0]
    if "comp_key" in boundary:
        K = boundary["comp_key"].astype(np.float64)
        W = boundary["comp_val"].astype(np.float64)
        R = (S32.astype(np.float64) - np.einsum("nci,ncj->nij", K, W)).astype(_F32)
    else:
        R = S32.copy()
        for s in range(n):
            R[s, boundary["comp_idx"][s], :] = 0
    sigma = (_F32(1) / boundary["col_scale"]).astype(_F32)
    Q = (R * sigma[:, None, :]).astype(_F32)
    m = np.abs(Q).max(axis=2).astype(_F32)
    inv = np.zeros_like(m)
    inv[m > 0] = (_F32(127) / m[m > 0]).astype(_F32)
    return (Q * inv[:, :, None]).astype(_F32)


def dequantize(boundary):
    """Boundary state B = deQ(codes, a, s) + compensator tokens, in fp64."""
    c = boundary["codes"].astype(np.float64)
    a = boundary["row_scale"].astype(np.float64)
    s = boundary["col_scale"].astype(np.float64)
    B = c * a[:, :, None] * s[:, None, :]
    if "comp_key" in boundary:
        K = boundary["comp_key"].astype(np.float64)
        W = boundary["comp_val"].astype(np.float64)
        return B + np.einsum("nci,ncj->nij", K, W)
    idx = boundary["comp_idx"]
    w = boundary["comp_val"].astype(np.float64)
    n, r = idx.shape
    for st in range(n):
        for c_ in range(r):
            B[st, idx[st, c_], :] += w[st, c_]
    return B


def copy_boundary(b, sel=None):
    """Deep copy of a boundary-state dict, optionally restricted to states `sel`."""
    if sel is None:
        return {k: np.array(v, copy=True) for k, v in b.items()}
    return {k: np.array(v[sel], copy=True) for k, v in b.items()}


# --------------------------------------------------------------------------
# Per-window decode ([EL] Figure 2) and the per-token baseline
# --------------------------------------------------------------------------
def window(boundary, tokens, t0, length, gate, r, flags=0, quantizer=True, iters=0):
    """Decode `length` tokens from `boundary`, then close the window.

    Tokens t0 .. t0+length-1 of `tokens` are used.  Returns
    (outputs [length, n, dv], records, S_end fp64, next boundary).  With
    quantizer=False the next boundary is the exact fp64 state instead of a
    quantized split (used to check that windowing alone changes nothing).
    """
    B = dequantize(boundary) if quantizer else np.array(boundary, np.float64, copy=True)
    S = B
    outs = []
    records = []
    for t in range(t0, t0 + length):
        o, S, rec = step(S, tokens["q"][t], tokens["k"][t], tokens["v"][t],
                         tokens["beta"][t], tokens["alpha"][t], gate, flags)
        outs.append(o)
        records.append(rec)
    nxt = quantize(S, r, flags, iters) if quantizer else S
    return np.stack(outs), records, S, nxt


def run_windowed(S_init, tokens, p, r, gate, flags=0, quantizer=True, keep=None, iters=0):
    """Free-running per-window quantized decode over all tokens.

    Returns (outputs [T, n, dv], boundaries) where boundaries[w] is the
    boundary state at the start of window w (w = 0 is Quantize(S_init));
    `keep` optionally limits which window indices are stored (plus the last).
    A final partial window (T not a multiple of p) is closed after its
    last token.
    """
    T = tokens["q"].shape[0]
    b = quantize(S_init, r, flags, iters) if quantizer else np.array(S_init, np.float64, copy=True)
    outs = []
    bounds = {}
    w = 0
    t0 = 0
    while True:
        if keep is None or w in keep:
            bounds[w] = b
        if t0 >= T:
            break
        length = min(p, T - t0)
        o, _, _, b = window(b, tokens, t0, length, gate, r, flags, quantizer, iters)
        outs.append(o)
        t0 += length
        w += 1
    bounds[w] = b
    return np.concatenate(outs, axis=0), bounds


def run_per_token(S_init, tokens, r, gate, flags=0, iters=0):
    """Per-token quantization baseline ([EL] Figure 2, left): the whole state
    is re-quantized after every update; the token's output is read from the
    updated state before it is quantized."""
    T = tokens["q"].shape[0]
    b = quantize(S_init, r, flags, iters)
    outs = []
    for t in range(T):
        S = dequantize(b)
        o, S, _ = step(S, tokens["q"][t], tokens["k"][t], tokens["v"][t],
                       tokens["beta"][t], tokens["alpha"][t], gate, flags)
        outs.append(o)
        b = quantize(S, r, flags, iters)
    return np.stack(outs), b


def round_bf16(x):
    """Round to bfloat16 (8 significant bits), to nearest with ties to even,
    through the fp32 value: the storage of the dense "BF16 per-step" state of
    [EL] Table 2.  Returns fp64 arrays holding bf16-representable values."""
    f = np.ascontiguousarray(np.asarray(x, np.float64).astype(np.float32))
    bits = f.view(np.uint32).astype(np.uint64)
    upper, lower = bits >> 16, bits & 0xFFFF
    up = (lower > 0x8000) | ((lower == 0x8000) & ((upper & 1) == 1))
    out = ((upper + up) << 16).astype(np.uint32).view(np.float32)
    return out.astype(np.float64)


def step_dense_bf16(S, q, k, v, beta, alpha, gate, flags=0):
    """One token of the "BF16 per-step" baseline of [EL] Table 2: the exact
    update of a bf16 state, the new state rounded to bf16.  Returns (o, S_new)
    with o read from the updated state before rounding."""
    o, S_new, _ = step(S, q, k, v, beta, alpha, gate, flags)
    return o, round_bf16(S_new)


def window_bf16(B, tokens, t0, length, gate, flags=0):
    """One window of the "BF16 + per-window" row of [EL] Table 2: the
    boundary state B (fp64 array of bf16 values) stays fixed, the window's
    tokens are the exact recurrence from it (what the fp32 buffered records
    reproduce), and the state after the window's last token is stored rounded
    to bf16.  Returns (outputs [length, n, dv], records, S_end, next B)."""
    S = np.array(B, np.float64, copy=True)
    outs, records = [], []
    for t in range(t0, t0 + length):
        o, S, rec = step(S, tokens["q"][t], tokens["k"][t], tokens["v"][t],
                         tokens["beta"][t], tokens["alpha"][t], gate, flags)
        outs.append(o)
        records.append(rec)
    return np.stack(outs), records, S, round_bf16(S)


def run_windowed_bf16(S_init, tokens, p, gate, flags=0):
    """Free-running "BF16 + per-window" decode: B_0 = bf16(S_init), then
    windows of p tokens (a final partial window is closed after its last
    token).  Returns (outputs [T, n, dv], list of boundary states)."""
    T = tokens["q"].shape[0]
    B = round_bf16(S_init)
    outs, bounds = [], [B]
    for t0 in range(0, T, p):
        o, _, _, B = window_bf16(B, tokens, t0, min(p, T - t0), gate, flags)
        outs.append(o)
        bounds.append(B)
    return np.concatenate(outs, axis=0), bounds


def state_mse(boundary, S_exact):
    """mean((B - S_exact)^2) per state, B the dequantized boundary state."""
    B = dequantize(boundary)
    return ((B - S_exact) ** 2).mean(axis=(1, 2))
