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
    that state's boundary is reported as a tie and checked by invariants.
"""
import numpy as np

from oracle import leapquant_oracle as O

RTOL, ATOL = 1e-3, 1e-4
FLIP_FRACTION = 1e-3
HALF_BAND = 1e-2
TIE_GAP = 1e-5


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
    return float((err / (atol + rtol * np.abs(ref))).max()) if err.size else 0.0


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


def compare_boundary(gpu, ref, S_ref, r, what, exact=False):
    """Compare a GPU boundary state with the oracle's.

    gpu, ref: dicts of arrays (codes, row_scale, col_scale, comp_idx,
    comp_val) for the same states; S_ref: the oracle's fp32 state that `ref`
    quantizes (used to locate rounding boundaries).  exact=True demands
    bit-identity (both sides quantized the same fp32 input).
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
        for k in ("codes", "row_scale", "col_scale", "comp_idx", "comp_val"):
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
        assert dist.max() <= HALF_BAND, f"{what}: code flip away from a rounding boundary (distance {dist.max()})"
        assert nflip <= FLIP_FRACTION * d.size, f"{what}: {nflip} flipped codes of {d.size}"
    return stats
