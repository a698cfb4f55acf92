"""Comparison rules between the HIP path and the oracle (host side).

Tolerances:
  * outputs o_t, buffered u_t, compensator rows, row and column scales:
    |gpu - ref| <= 1e-4 + 1e-3 |ref| elementwise;
  * int8 codes: identical, except entries off by one where the oracle's
    pre-rounding value lies within a band of a half-integer, at most 0.1%
    of a slab's codes per boundary (a code at a rounding boundary is decided
    by the last bits of the fp32 rebuilt state, which the GPU sums in a
    different order).  The band is HALF_BAND plus two measured or bounded
    terms per code: the shift that the GPU's own row and column scales
    (compared above) cause at that code, |x| (|da|/a + |ds|/s), and, when
    the caller passes the magnitudes the fp32 rebuild sums (`mag`), that
    rebuild's rounding error in code units, REBUILD_EPS mag / (a s);
  * compensator selection: the GPU's rows must be a top-r of the oracle's
    norms up to fp32 rounding of those norms (TIE_GAP relative).  Where
    they differ from the oracle's own choice (a near tie), the oracle is
    forced to the GPU's rows and the whole boundary is compared against
    that split under the same rules: no state is left out;
  * dense compensator keys: every key within KEY_ATOL of the oracle's.  A
    key is kept only if its Gram-Schmidt ratio exceeds the drop threshold
    (2e-2), which bounds the amplification of fp32 rounding; a keep / drop
    decision may differ only where the oracle's ratio lies within
    DECISION_BAND of the threshold, and the oracle is then forced to the
    GPU's decision.  Every GPU key is unit or zero and orthogonal to the
    others; the rest of a dense boundary is compared with the oracle's
    split under the GPU's keys, except for states of numerical rank <= r,
    whose residual is rounding noise: those must reconstruct the state to
    NOISE_RESIDUAL of its largest entry.
"""
import json
import os

import numpy as np

from oracle import leapquant_oracle as O

RTOL, ATOL = 1e-3, 1e-4
FLIP_FRACTION = 1e-3
# Distance from a half-integer within which the oracle's fp32 pre-rounding
# code value may round the other way on the GPU, before the per-code terms
# below (scale shift, rebuild error) are added.
HALF_BAND = 1e-3
# fp32 error of the rebuilt state relative to the magnitudes it sums:
# Gamma (a product of up to 64 fp32 gates), the dequantized code (two
# products), the compensator add, the suffix products of the records' key
# decays (up to 64 factors) and the fp32 MFMA / FMA accumulation over up to
# 64 + 16 terms, each rounding at 2^-24: below 2^-16 in total.
REBUILD_EPS = 2.0 ** -16
# Relative gap within which two fp32 row norms (128 squares summed in a
# different order) may order two rows differently: the sum of n = 128
# non-negative terms carries at most (n - 1) 2^-24 = 7.6e-6 relative error.
TIE_GAP = 1e-5
# Dense compensator keys (unit vectors), fp32 iteration against fp64: a
# relative perturbation of S by one ulp moves the oracle's keys by up to
# ~2.5e-6 (r = 16, the last keys in the noise bulk, measured); the fp32
# products and Gram-Schmidt sums amount to tens of ulps, amplified at most
# 1 / MGS_DROP = 50-fold in a kept key (simulated fp32 iterations: below
# 1e-5).  An algorithmic mistake moves keys by O(0.1).
KEY_ATOL = 1e-3
NOISE_RESIDUAL = 1e-4  # residual / state magnitude below which a dense split is rank-exhausted
# A keep / drop decision is taken in fp32 on the GPU: the ratio carries an
# absolute error of about 1e-5 (1.5e-5 of |S S^T k| through the projected
# norm), i.e. 5e-4 of the threshold; decisions whose oracle ratio lies within
# this relative band of the threshold may go either way.
DECISION_BAND = 1e-2
# Loss of orthogonality between the GPU's nonzero keys: the same error,
# amplified by 1 / (the smallest ratio among the kept keys a key was
# projected against, at least the drop threshold), with a floor.
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


def _log(stats, what):
    """Append a comparison's statistics to $LQ_PARITY_LOG (JSON lines), if set."""
    path = os.environ.get("LQ_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps({"what": what, **stats}) + "\n")


def row_norms2(S32):
    """Squared row norms of fp32 states, fp64 sums of exact fp32 squares."""
    S = np.asarray(S32, np.float32).astype(np.float64)
    return np.einsum("nij,nij->ni", S, S)


def check_selection(idx, S32, r, what):
    """The GPU's compensator rows idx [n, r] must be a top-r selection of the
    oracle's fp32 state up to fp32 rounding of the row norms: r distinct rows
    in range, every chosen norm at least (1 - TIE_GAP) times every unchosen
    one, stored in descending order up to the same gap.  Returns the mask of
    states whose selection differs from the oracle's own (near ties)."""
    n2 = row_norms2(S32)
    n = n2.shape[0]
    if r == 0:
        return np.zeros(n, bool)
    idx = np.asarray(idx).astype(np.int64)
    assert idx.shape == (n, r), (what, idx.shape)
    assert idx.min() >= 0 and idx.max() < n2.shape[1], f"{what}: compensator row out of range"
    for s in range(n):
        assert len(set(idx[s].tolist())) == r, f"{what}: state {s} repeats a compensator row"
    chosen = np.take_along_axis(n2, idx, axis=1)
    mask = np.ones_like(n2, bool)
    np.put_along_axis(mask, idx, False, axis=1)
    rest_max = np.where(mask, n2, -np.inf).max(axis=1)
    lo = chosen.min(axis=1)
    bad = lo < (1 - TIE_GAP) * rest_max
    assert not bad.any(), f"{what}: compensator rows are not a top-{r} in states {np.nonzero(bad)[0][:8]}"
    dec = chosen[:, 1:] <= chosen[:, :-1] * (1 + TIE_GAP)
    assert dec.all(), f"{what}: compensator rows not in descending-norm order"
    own = np.argsort(-n2, axis=1, kind="stable")[:, :r]
    return ~np.all(idx == own, axis=1)


def _infer_flags(ref, flags):
    if flags is not None:
        return flags
    return O.NO_SMOOTH if np.all(np.asarray(ref["col_scale"]) == 1) else 0


def compare_boundary(gpu, ref, S_ref, r, what, exact=False, band=None, flags=None, mag=None):
    """Compare a GPU boundary state with the oracle's.

    gpu, ref: dicts of arrays (codes, row_scale, col_scale, comp_idx,
    comp_val) for the same states; S_ref: the oracle's fp32 state that `ref`
    quantizes (used to locate rounding boundaries and to re-split near
    ties).  exact=True demands bit-identity (both sides quantized the same
    fp32 input).  band: optional per-code widening of the rounding band
    (code units).  flags: the quantizer flags `ref` was made with (None:
    NO_SMOOTH when every column scale of `ref` is 1).  mag: optional
    [n, dk, dv] magnitudes that the GPU's fp32 rebuild of S_ref summed
    (Gamma |B| + sum_i |K_i| |u_i|), for the rebuild-error term of the band.
    Every state is compared; states whose GPU rows differ from the oracle's
    (a near tie, validated by check_selection) are compared against the
    oracle's split under the GPU's rows.  Returns a dict of statistics,
    also appended to $LQ_PARITY_LOG.
    """
    n = ref["codes"].shape[0]
    S_ref = np.asarray(S_ref, np.float32)
    gpu = {k: np.asarray(v) for k, v in gpu.items()}
    ref = {k: np.asarray(v) for k, v in ref.items()}
    ties = check_selection(gpu["comp_idx"], S_ref, r, what)
    stats = {"states": n, "ties": int(ties.sum()), "flips": 0, "codes": 0, "max_half_dist": 0.0,
             "max_band_use": 0.0}
    if ties.any():
        # the oracle's split of the same fp32 state under the GPU's rows
        forced = O.quantize(S_ref[ties], r, _infer_flags(ref, flags), rows=gpu["comp_idx"][ties])
        ref = {k: v.copy() for k, v in ref.items()}
        for k in forced:
            ref[k][ties] = forced[k]
    np.testing.assert_array_equal(gpu["comp_idx"], ref["comp_idx"], err_msg=f"{what}: comp_idx")
    if exact:
        for k in ("codes", "row_scale", "col_scale", "comp_idx", "comp_val", "comp_key"):
            if k in ref:
                np.testing.assert_array_equal(gpu[k], ref[k], err_msg=f"{what}: {k}")
        stats["codes"] = int(ref["codes"].size)
        _log(stats, what)
        return stats
    g, o = gpu, ref
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
        pre = O.prerounding_codes(S_ref, o)
        x = pre[flips].astype(np.float64)
        dist = np.abs(np.abs(x - np.floor(x)) - 0.5)
        stats["max_half_dist"] = float(dist.max())
        extra = np.zeros_like(x) if band is None else np.asarray(band, np.float64)[flips]
        # the GPU's own scales shift every code of a row / column
        a_g, a_o = g["row_scale"].astype(np.float64), o["row_scale"].astype(np.float64)
        s_g, s_o = g["col_scale"].astype(np.float64), o["col_scale"].astype(np.float64)
        ra = np.abs(a_g - a_o) / np.where(a_o > 0, a_o, 1.0)
        rs = np.abs(s_g - s_o) / np.where(s_o > 0, s_o, 1.0)
        extra = extra + np.abs(x) * (ra[flips[0], flips[1]] + rs[flips[0], flips[2]])
        if mag is not None:
            unit = a_o[flips[0], flips[1]] * s_o[flips[0], flips[2]]
            m = np.asarray(mag, np.float64)[flips]
            extra = extra + np.where(unit > 0, REBUILD_EPS * m / np.where(unit > 0, unit, 1.0), 0.0)
        lim = HALF_BAND + extra
        stats["max_band_use"] = float((dist / lim).max())
        assert np.all(dist <= lim), \
            f"{what}: code flip away from a rounding boundary (distance {dist.max()}, band {lim[np.argmax(dist / lim)]})"
        allowed = FLIP_FRACTION * d.size
        if band is not None:
            # codes whose value lies inside the widened band flip at most
            # with the band's width (uniform fractional parts), 4x margin
            allowed += 4 * float(np.minimum(0.5, np.asarray(band)).sum())
        assert nflip <= allowed, f"{what}: {nflip} flipped codes of {d.size}"
    _log(stats, what)
    return stats


def rebuild_magnitude(boundary, records):
    """Magnitudes that a rebuild of the state from `boundary` and the window's
    records sums, |Gamma B| + sum_i |Gamma_p / Gamma_i k~_i| |u_i|: the replay
    of the records on |B| with |k~| and |u| (decays are non-negative)."""
    B = np.abs(O.dequantize(boundary))
    return O.replay(B, [(d, np.abs(kt), np.abs(u)) for d, kt, u in records])


def oracle_keys(S32, rows, iters, keep=None):
    """The oracle's keys [r, dk] and Gram-Schmidt ratios [iters, r] of one
    state started from `rows`, with keep / drop decisions forced by `keep`
    ({(round, key): bool})."""
    ratios = []
    K = O.dense_keys(np.asarray(S32, np.float32).astype(np.float64), rows, iters, ratios, keep)
    return K.T, (np.array(ratios) if iters else np.ones((0, len(rows))))


def match_decisions(K_gpu, S32, rows, iters, what):
    """Force the oracle's keep / drop decisions to the GPU's where the GPU
    kept a key the oracle dropped, or dropped one it kept; each such
    decision must sit within DECISION_BAND of the threshold in some round.
    Returns (forced decisions, oracle keys, ratios)."""
    r = len(rows)
    nz_g = np.linalg.norm(np.asarray(K_gpu, np.float64), axis=1) > 0.5
    keep = {}
    for _ in range(r + 1):
        K, rat = oracle_keys(S32, rows, iters, keep)
        nz_o = np.linalg.norm(K, axis=1) > 0.5
        diff = np.nonzero(nz_o != nz_g)[0]
        if not len(diff):
            return keep, K, rat
        c = int(diff[0])
        near = [it for it in range(iters)
                if rat[it, c] > 0 and abs(rat[it, c] / O.MGS_DROP - 1) <= DECISION_BAND and (it, c) not in keep]
        assert near, (f"{what}: GPU {'kept' if nz_g[c] else 'dropped'} key {c} away from the threshold "
                      f"(oracle ratios {rat[:, c]})")
        keep[(near[0], c)] = bool(nz_g[c])
    raise AssertionError(f"{what}: keep / drop decisions do not settle")


def compare_dense_boundary(gpu, S_ref, r, iters, flags, what):
    """Dense compensator tokens.

    The keys come from an fp32 iteration on the GPU and an fp64 one in the
    oracle.  A key that survives a Gram-Schmidt step with a fraction rho of
    its norm carries the fp32 error amplified by 1 / rho; keys are kept only
    with rho above the drop threshold, so every key agrees to KEY_ATOL and
    is compared, after forcing the oracle's keep / drop decisions that lie
    within rounding of the threshold to the GPU's.  Every GPU key is checked
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
    Near ties of the starting rows force the oracle to the GPU's rows, as
    for row extraction.
    """
    S_ref = np.asarray(S_ref, np.float32)
    S64 = S_ref.astype(np.float64)
    g_all = {k: np.asarray(v) for k, v in gpu.items()}
    n = len(S_ref)
    # the starting rows are a top-r selection; near ties force the oracle's
    # iteration to start from the GPU's rows
    ties = check_selection(g_all["comp_idx"], S_ref, r, what)
    ok = np.ones(n, bool)
    stats = {"states": n, "ties": int(ties.sum()), "flips": 0, "codes": 0, "low_rank": 0,
             "max_excess": 0.0, "keys_compared": 0, "decisions_forced": 0, "max_key_err": 0.0}
    if r and ok.any():
        # every key against the oracle's, with keep / drop decisions at the
        # threshold forced to the GPU's
        Ko = np.zeros((n, r, 128))
        rat = np.ones((n, iters, r))
        for s_ in range(n):
            keep, Ko[s_], rat[s_] = match_decisions(g_all["comp_key"][s_], S_ref[s_], g_all["comp_idx"][s_],
                                                    iters, f"{what} state {s_}")
            stats["decisions_forced"] += len(keep)
        Kg = g_all["comp_key"].astype(np.float64)
        assert_close(Kg, Ko.astype(np.float32), f"{what}: comp_key", rtol=0, atol=KEY_ATOL)
        stats["keys_compared"] = int(n * r)
        stats["max_key_err"] = float(np.abs(Kg - Ko.astype(np.float32)).max())
        G = np.einsum("nci,ndi->ncd", Kg, Kg)
        nz = np.linalg.norm(Kg, axis=2) > 0.5
        both = nz[:, :, None] & nz[:, None, :]
        dev = np.abs(G - np.eye(r)[None])
        if iters:
            # per key, its smallest ratio over the rounds (at least the
            # threshold: a kept key's ratio is above it up to the band)
            rk = np.where(nz, np.maximum(rat, O.MGS_DROP * (1 - DECISION_BAND)).min(axis=1), 1.0)
            cum = np.minimum.accumulate(rk, axis=1)          # over keys 0..d
        else:
            cum = np.ones((n, r))
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
        _log(stats, what)
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
    _log(stats, what)
    return stats
