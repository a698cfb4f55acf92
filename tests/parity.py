"""Comparison rules between the HIP path and the oracle (host side).

Tolerances:
  * outputs o_t, buffered u_t, compensator rows, row and column scales:
    |gpu - ref| <= 1e-4 + 1e-3 |ref| elementwise;
  * int8 codes: identical, except entries off by one where the oracle's
    pre-rounding value lies within HALF_BAND of a half-integer, at most 0.1%
    of a slab's codes per boundary (a code at a rounding boundary is decided
    by the last bits of the fp32 rebuilt state, which the GPU sums in a
    different order);
  * compensator selection: identical row sets, unless the oracle's r-th and
    (r+1)-th row norms are a near tie (relative gap < 1e-5), in which case
    that state's boundary is reported as a tie and checked by invariants;
  * dense compensator keys: the leading keys that the fp32 state determines
    (every Gram-Schmidt ratio of the oracle's iteration outside
    (RATIO_DROPPED, RATIO_OK)) within KEY_ATOL; every GPU key unit or zero
    and orthogonal to the others within a bound scaled by the keys'
    conditioning; the rest of a dense boundary is compared with the
    oracle's split under the GPU's keys, except for states of numerical
    rank <= r, whose residual is rounding noise: those must reconstruct the
    state to NOISE_RESIDUAL of its largest entry.
"""
import numpy as np

from oracle import leapquant_oracle as O

RTOL, ATOL = 1e-3, 1e-4
FLIP_FRACTION = 1e-3
HALF_BAND = 1e-2
TIE_GAP = 1e-5
# Dense compensator keys (unit vectors), fp32 iteration against fp64: a
# relative perturbation of S by one ulp moves the oracle's keys by up to
# ~2.5e-6 (r = 16, the last keys in the noise bulk, measured); the fp32
# products and Gram-Schmidt sums amount to tens of ulps.  An algorithmic
# mistake moves keys by O(0.1).
KEY_ATOL = 1e-3
NOISE_RESIDUAL = 1e-4  # residual / state magnitude below which a dense split is rank-exhausted
# A Gram-Schmidt step that leaves a fraction rho of a column's norm amplifies
# the error of that column by 1/rho.  The fp32 evaluation of S S^T K carries
# up to about 1.5e-5 of |S S^T k| (two 128-term sums); below RATIO_OK that
# error can exceed KEY_ATOL in the normalized key, and later keys inherit it
# through their projections.  Columns below RATIO_DROPPED (a tenth of the
# drop threshold) are dropped on both sides with margin.
RATIO_OK = 2e-2
RATIO_DROPPED = 1e-4
# Loss of orthogonality between the GPU's nonzero keys c < d: the same
# error, amplified by 1 / (the smallest ratio, at least the drop threshold,
# among the kept keys 0..d, which key d was projected against), with a
# floor for well-conditioned keys.
KEY_ORTHO_EPS = 1.5e-5
KEY_ORTHO_FLOOR = 1e-4


def assert_close(gpu, ref, what, rtol=RTOL, atol=ATOL):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    err = np.abs(gpu - ref)
    bad = err > atol + rtol * np.abs(ref)
    if bad.any():
        i = np.unravel_index(np.argmax(err - (atol + rtol * np.abs(ref))), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} entries out of tolerance; "
                             f"worst at {i}: gpu={gpu[i]!r} ref={ref[i]!r}")
    lim = atol + rtol * np.abs(ref)
    return float(np.divide(err, lim, out=np.zeros_like(err), where=lim > 0).max()) if err.size else 0.0


def near_tie(S32, r):
    """Per state: True when two of the oracle's top r + 1 row norms differ,
    but by less than TIE_GAP relative.  Exactly equal norms are not a near
    tie: both sides break them by the lower row index."""
    S = np.asarray(S32, np.float32).astype(np.float64)
    n2 = np.sort(np.einsum("nij,nij->ni", S, S), axis=1)[:, ::-1]
    if r == 0:
        return np.zeros(S.shape[0], bool)
    top = n2[:, :r + 1]
    gaps = (top[:, :-1] - top[:, 1:]) / np.maximum(top[:, :-1], 1e-300)
    return ((gaps > 0) & (gaps < 2 * TIE_GAP)).any(axis=1)


def compare_boundary(gpu, ref, S_ref, r, what, exact=False, band=None):
    """Compare a GPU boundary state with the oracle's.

    gpu, ref: dicts of arrays (codes, row_scale, col_scale, comp_idx,
    comp_val) for the same states; S_ref: the oracle's fp32 state that `ref`
    quantizes (used to locate rounding boundaries).  exact=True demands
    bit-identity (both sides quantized the same fp32 input).  band: optional
    per-code widening of the rounding band (code units), for residuals whose
    fp32 evaluation error is known to exceed the rebuilt state's.
    Returns a dict of statistics.
    """
    n = ref["codes"].shape[0]
    ties = near_tie(S_ref, r)
    ok = ~ties
    stats = {"states": n, "ties": int(ties.sum()), "flips": 0, "codes": 0, "max_half_dist": 0.0}
    if r:
        same_sel = np.all(gpu["comp_idx"] == ref["comp_idx"], axis=1)
        bad = ok & ~same_sel
        assert not bad.any(), f"{what}: compensator rows differ without a near tie in states {np.nonzero(bad)[0][:8]}"
    if not ok.any():
        return stats
    g = {k: np.asarray(v)[ok] for k, v in gpu.items()}
    o = {k: np.asarray(v)[ok] for k, v in ref.items()}
    if exact:
        for k in ("codes", "row_scale", "col_scale", "comp_idx", "comp_val", "comp_key"):
            if k in o:
                np.testing.assert_array_equal(g[k], o[k], err_msg=f"{what}: {k}")
        stats["codes"] = int(o["codes"].size)
        return stats
    if r:
        assert_close(g["comp_val"], o["comp_val"], f"{what}: comp_val")
    assert_close(g["col_scale"], o["col_scale"], f"{what}: col_scale")
    assert_close(g["row_scale"], o["row_scale"], f"{what}: row_scale")
    d = g["codes"].astype(np.int32) - o["codes"].astype(np.int32)
    assert np.abs(d).max(initial=0) <= 1, f"{what}: a code differs by {np.abs(d).max()}"
    flips = np.nonzero(d)
    nflip = len(flips[0])
    stats["flips"] = nflip
    stats["codes"] = int(d.size)
    if nflip:
        pre = O.prerounding_codes(np.asarray(S_ref)[ok], o)
        x = pre[flips].astype(np.float64)
        dist = np.abs(np.abs(x - np.floor(x)) - 0.5)
        stats["max_half_dist"] = float(dist.max())
        extra = 0.0 if band is None else np.asarray(band)[ok][flips]
        assert np.all(dist <= HALF_BAND + extra), \
            f"{what}: code flip away from a rounding boundary (distance {dist.max()})"
        allowed = FLIP_FRACTION * d.size
        if band is not None:
            # codes whose value lies inside the widened band flip at most
            # with the band's width (uniform fractional parts), 4x margin
            allowed += 4 * float(np.minimum(0.5, np.asarray(band)[ok]).sum())
        assert nflip <= allowed, f"{what}: {nflip} flipped codes of {d.size}"
    return stats


def key_ratios(S32, r, iters):
    """Gram-Schmidt ratios of the oracle's dense-key iteration: [n, iters, r]
    (see oracle mgs), for the states S32 started from their top-r rows."""
    S32 = np.asarray(S32, np.float32)
    out = np.ones((len(S32), iters, r))
    for s in range(len(S32)):
        S64 = S32[s].astype(np.float64)
        start = np.argsort(-np.einsum("ij,ij->i", S64, S64), kind="stable")[:r]
        ratios = []
        O.dense_keys(S64, start, iters, ratios)
        if iters:
            out[s] = np.array(ratios)
    return out


def determined_keys(ratios):
    """Per state, the number of leading dense keys that the fp32 state
    determines to KEY_ATOL: keys up to the first one whose ratio, in any
    round, lies between RATIO_DROPPED and RATIO_OK (key c depends only on
    keys 0..c of this and earlier rounds)."""
    bad = ((ratios > RATIO_DROPPED) & (ratios < RATIO_OK)).any(axis=1)  # [n, r]
    r = ratios.shape[2]
    return np.where(bad.any(axis=1), bad.argmax(axis=1), r)


def compare_dense_boundary(gpu, S_ref, r, iters, flags, what):
    """Dense compensator tokens.

    The keys come from an fp32 iteration on the GPU and an fp64 one in the
    oracle.  A key that survives a Gram-Schmidt step with a small fraction
    of its norm carries the fp32 error amplified by the inverse of that
    fraction, and so do the keys after it; the leading keys up to the first
    such one agree to KEY_ATOL and are compared, every GPU key is checked
    for unit norm (or zero) and orthogonality to the others.  Given the
    keys, the values follow.
    The residual S - sum_c k_c w_c^T is evaluated in fp32 on the GPU; in rows
    that the tokens mostly carry it is small next to the terms it is computed
    from, so its rounding error (bounded below) is large in code units and
    moves row and column scales too.  Codes are therefore checked against
    the GPU's own scales: every GPU code must round the oracle's residual
    (under the GPU's keys) divided by the GPU's a_i s_j, up to the rounding
    band plus that bound; the scales themselves are compared with the
    oracle's.  States of numerical rank <= r, whose residual is rounding
    noise, must reconstruct the state to NOISE_RESIDUAL of its largest entry.
    Near ties of the starting rows are exempt, as for row extraction.
    """
    S_ref = np.asarray(S_ref, np.float32)
    S64 = S_ref.astype(np.float64)
    g_all = {k: np.asarray(v) for k, v in gpu.items()}
    ok = ~near_tie(S_ref, r)
    ref = O.quantize(S_ref, r, flags | O.DENSE_COMP, iters)
    stats = {"states": len(S_ref), "ties": int((~ok).sum()), "flips": 0, "codes": 0, "low_rank": 0,
             "max_excess": 0.0, "keys_compared": 0, "keys_undetermined": 0}
    if r and ok.any():
        np.testing.assert_array_equal(g_all["comp_idx"][ok], ref["comp_idx"][ok], err_msg=f"{what}: start rows")
        # keys the fp32 state determines: against the oracle's; the rest:
        # unit or zero and orthogonal (checked below for every key)
        rat = key_ratios(S_ref[ok], r, iters)
        det = determined_keys(rat)
        mask = np.arange(r)[None, :] < det[:, None]
        assert_close(g_all["comp_key"][ok][mask], ref["comp_key"][ok][mask], f"{what}: comp_key",
                     rtol=0, atol=KEY_ATOL)
        stats["keys_compared"] = int(mask.sum())
        stats["keys_undetermined"] = int((~mask).sum())
        Kg = g_all["comp_key"][ok].astype(np.float64)
        G = np.einsum("nci,ndi->ncd", Kg, Kg)
        nz = np.linalg.norm(Kg, axis=2) > 0.5
        both = nz[:, :, None] & nz[:, None, :]
        dev = np.abs(G - np.eye(r)[None])
        if iters:
            # per key, its smallest ratio over the rounds in which it was kept
            kept = rat > RATIO_DROPPED
            rk = np.where(kept, np.maximum(rat, O.MGS_DROP), 1.0).min(axis=1)
            cum = np.minimum.accumulate(rk, axis=1)          # over keys 0..d
        else:
            cum = np.ones((len(Kg), r))
        later = np.maximum(np.arange(r)[:, None], np.arange(r)[None, :])
        tol = np.maximum(KEY_ORTHO_FLOOR, KEY_ORTHO_EPS / cum[:, later])
        if not np.all(dev[both] <= tol[both]):
            i = np.unravel_index(np.argmax(np.where(both, dev - tol, -np.inf)), dev.shape)
            raise AssertionError(f"{what}: GPU keys not orthonormal: state {i[0]}, keys {i[1]}, {i[2]}: "
                                 f"{dev[i]:.3g} > {tol[i]:.3g}")
        assert np.all(Kg[~nz] == 0), f"{what}: a dropped GPU key is not zero"
    ref_g = O.quantize(S_ref, r, flags | O.DENSE_COMP, iters, keys=g_all["comp_key"])
    K = g_all["comp_key"].astype(np.float64)
    W = ref_g["comp_val"].astype(np.float64)
    R = S64 - np.einsum("nci,ncj->nij", K, W)
    smax = np.abs(S64).max(axis=(1, 2))
    noise = ok & (smax > 0) & (np.abs(R).max(axis=(1, 2)) <= NOISE_RESIDUAL * smax)
    if noise.any():
        B = O.dequantize({k: v[noise] for k, v in g_all.items()})
        err = np.abs(B - S64[noise]).max(axis=(1, 2))
        assert np.all(err <= NOISE_RESIDUAL * smax[noise]), f"{what}: low-rank states not reconstructed"
        stats["low_rank"] = int(noise.sum())
    keep = ok & ~noise
    if not keep.any():
        return stats
    g = {k: v[keep] for k, v in g_all.items()}
    o = {k: np.asarray(v)[keep] for k, v in ref_g.items()}
    if r:
        assert_close(g["comp_val"], o["comp_val"], f"{what}: comp_val")
    assert_close(g["col_scale"], o["col_scale"], f"{what}: col_scale")
    assert_close(g["row_scale"], o["row_scale"], f"{what}: row_scale")
    # fp32 evaluation error of the residual: the FMA chain over c and the
    # sums forming w_c (depth <= 8) each round at 2^-24 of the magnitudes
    # involved; 2^-20 bounds their total (and the rebuilt state's own error)
    Kk, Sk, Rk = np.abs(K[keep]), np.abs(S64[keep]), R[keep]
    mag = Sk + np.einsum("nci,ncj->nij", Kk, np.abs(W[keep])) + \
        np.einsum("nci,ncj->nij", Kk, np.einsum("ncl,nlj->ncj", Kk, Sk))
    unit = g["row_scale"].astype(np.float64)[:, :, None] * g["col_scale"].astype(np.float64)[:, None, :]
    pos = unit > 0
    safe = np.where(pos, unit, 1.0)
    x = np.where(pos, np.clip(Rk / safe, -127, 127), 0.0)
    band = np.where(pos, 2.0 ** -20 * mag / safe, 0.0)
    c = g["codes"].astype(np.float64)
    excess = np.abs(x - c) - (0.5 + HALF_BAND + band)
    stats["max_excess"] = float(excess.max())
    assert excess.max() <= 0, f"{what}: a code is not the rounded residual under its own scales " \
                              f"(excess {excess.max()})"
    off = int((c != np.rint(x)).sum())
    allowed = FLIP_FRACTION * c.size + 4 * float(np.minimum(0.5, band).sum())
    assert off <= allowed, f"{what}: {off} codes at rounding boundaries of {c.size} (allowed {allowed:.0f})"
    stats["flips"] = off
    stats["differ_from_oracle_codes"] = int((g["codes"] != o["codes"]).sum())
    stats["codes"] = int(c.size)
    return stats
