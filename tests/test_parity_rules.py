"""The dense-key comparison rule rejects plausible GPU mistakes (CPU).

compare_dense_boundary compares every key with the oracle's (keep / drop
decisions within rounding of the threshold forced to the GPU's), checks
every key's orthonormality with a conditioning-scaled bound, and checks
values and codes under the GPU's own keys.  Here a
stand-in for the GPU result is built from the oracle: unchanged it passes,
and with each planted mistake (keys iterated on S^T S instead of S S^T,
keys not orthogonalized, keys not normalized, the residual's sign) it
fails.
"""
import numpy as np
import pytest

from oracle import leapquant_oracle as O
from tests import parity as P

R, ITERS = 4, 2


def _states(seed, n=6):
    rng = np.random.default_rng(seed)
    S = (0.02 * rng.standard_normal((n, 128, 128))).astype(np.float32)
    for s in range(n):
        rows = rng.choice(128, 3, replace=False)
        S[s, rows] *= rng.uniform(10, 30, (3, 1)).astype(np.float32)
    return S


def _keys(S, mistake):
    out = np.zeros((len(S), R, 128), np.float32)
    for s in range(len(S)):
        S64 = S[s].astype(np.float64)
        start = np.argsort(-np.einsum("ij,ij->i", S64, S64), kind="stable")[:R]
        K = np.zeros((128, R))
        K[start, np.arange(R)] = 1.0
        for _ in range(ITERS):
            Y = (S64.T @ (S64 @ K)) if mistake == "wrong side" else S64 @ (S64.T @ K)
            if mistake == "no projection":
                K = Y / np.linalg.norm(Y, axis=0)
            elif mistake == "no normalization":
                K = O.mgs(Y) * np.linalg.norm(Y, axis=0)
            else:
                K = O.mgs(Y)
        out[s] = K.T
    return out


def _gpu_standin(S, mistake=None):
    b = O.quantize(S, R, O.DENSE_COMP, ITERS, keys=_keys(S, mistake))
    if mistake == "residual sign":
        # codes of S + sum_c k_c w_c^T instead of S - sum_c k_c w_c^T
        K = b["comp_key"].astype(np.float64)
        W = b["comp_val"].astype(np.float64)
        wrong = (S.astype(np.float64) + np.einsum("nci,ncj->nij", K, W)).astype(np.float32)
        b2 = O.quantize(wrong, 0)   # that residual smoothed and quantized as it stands
        b = dict(b, codes=b2["codes"], row_scale=b2["row_scale"], col_scale=b2["col_scale"])
    return b


def test_oracle_standin_passes():
    S = _states(11)
    stats = P.compare_dense_boundary(_gpu_standin(S), S, R, ITERS, 0, "stand-in")
    assert stats["keys_compared"] == len(S) * R


@pytest.mark.parametrize("mistake", ["wrong side", "no projection", "no normalization", "residual sign"])
def test_planted_mistakes_fail(mistake):
    S = _states(12)
    with pytest.raises(AssertionError):
        P.compare_dense_boundary(_gpu_standin(S, mistake), S, R, ITERS, 0, mistake)
