"""Pins of the oracle's dense Compensator Tokens (flag DENSE_COMP).

In the pages, compensators are a few high-precision tokens that hold the
state's largest components and are updated like real tokens ([EL] Abstract,
Figure 4).  The dense reading keeps r tokens
(k_c, w_c) with unit keys from subspace iteration on S S^T started at the
one-hot keys of the largest-norm rows.  What mathematics fixes, and what is
checked here without a GPU:
  * zero iterations are exactly the row extraction;
  * the keys are orthonormal and the residual is orthogonal to them;
  * many iterations reach the dominant left singular subspace (LAPACK SVD);
  * on tiny heads the keys equal those of a Householder QR (LAPACK) of the
    same iterates, with the signs fixed to a positive R diagonal;
  * the reconstruction keeps the quantizer's half-step bound;
  * rank-deficient and zero states give zero keys past their rank.
"""
import numpy as np
import pytest

from oracle import leapquant_oracle as O

DENSE = O.DENSE_COMP


def _states(rng, n, dk=128, dv=128, outliers=True):
    S = (0.02 * rng.standard_normal((n, dk, dv))).astype(np.float32)
    if outliers:
        for s in range(n):
            rows = rng.choice(dk, 3, replace=False)
            cols = rng.choice(dv, 2, replace=False)
            S[s, rows] *= rng.uniform(10, 30, (3, 1)).astype(np.float32)
            S[s, :, cols] *= rng.uniform(10, 30, (2, 1)).astype(np.float32)
    return S


@pytest.mark.parametrize("r,flags", [(0, 0), (4, 0), (8, 0), (4, O.NO_SMOOTH)])
def test_zero_iterations_are_row_extraction(r, flags):
    rng = np.random.default_rng(500 + r + flags)
    S = _states(rng, 5)
    rows = O.quantize(S, r, flags)
    dense = O.quantize(S, r, flags | DENSE, iters=0)
    for k in ("codes", "row_scale", "col_scale", "comp_idx", "comp_val"):
        np.testing.assert_array_equal(dense[k], rows[k], err_msg=k)
    onehot = np.zeros((5, r, 128), np.float32)
    for s in range(5):
        onehot[s, np.arange(r), rows["comp_idx"][s]] = 1
    np.testing.assert_array_equal(dense["comp_key"], onehot)
    np.testing.assert_array_equal(O.dequantize(dense), O.dequantize(rows))


@pytest.mark.parametrize("r,iters", [(1, 1), (4, 1), (4, 2), (8, 3), (16, 2)])
def test_keys_orthonormal_and_residual_orthogonal(r, iters):
    rng = np.random.default_rng(600 + 10 * r + iters)
    S = _states(rng, 4)
    b = O.quantize(S, r, DENSE, iters=iters)
    for s in range(4):
        K = b["comp_key"][s].astype(np.float64)          # [r, dk]
        # kept keys orthonormal, dropped keys exactly zero
        kept = np.linalg.norm(K, axis=1) > 0.5
        assert kept[0] and np.all(K[~kept] == 0)
        np.testing.assert_allclose(K @ K.T, np.diag(kept.astype(np.float64)), atol=2e-6)
        W = b["comp_val"][s].astype(np.float64)
        S64 = S[s].astype(np.float64)
        np.testing.assert_allclose(W, K @ S64, rtol=1e-6, atol=1e-6 * np.abs(S64).max())
        R = S64 - K.T @ W
        assert np.abs(K @ R).max() <= 1e-5 * np.abs(S64).max()


def test_many_iterations_reach_the_svd_subspace():
    """A state with r well separated singular values above a noise bulk:
    the projector onto the keys equals that of the r leading left singular
    vectors from LAPACK's SVD."""
    rng = np.random.default_rng(700)
    dk = dv = 128
    r = 4
    for trial in range(3):
        U, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
        V, _ = np.linalg.qr(rng.standard_normal((dv, dv)))
        sig = np.array([9.0, 7.0, 5.0, 4.0])
        S = (U[:, :r] * sig) @ V[:, :r].T + 0.02 * rng.standard_normal((dk, dv))
        S = S.astype(np.float32)[None]
        b = O.quantize(S, r, DENSE, iters=12)
        K = b["comp_key"][0].astype(np.float64)
        Us, _, _ = np.linalg.svd(S[0].astype(np.float64))
        P_svd = Us[:, :r] @ Us[:, :r].T
        np.testing.assert_allclose(K.T @ K, P_svd, atol=1e-5)


@pytest.mark.parametrize("dk,dv,r,iters", [(8, 8, 2, 3), (6, 5, 3, 2), (4, 7, 1, 4), (8, 4, 4, 1)])
def test_tiny_heads_against_householder_qr(dk, dv, r, iters):
    rng = np.random.default_rng(800 + dk * dv + r + iters)
    S = rng.standard_normal((3, dk, dv)).astype(np.float32)
    b = O.quantize(S, r, DENSE, iters=iters)
    for s in range(3):
        S64 = S[s].astype(np.float64)
        norms = (S64 ** 2).sum(axis=1)
        start = np.argsort(-norms, kind="stable")[:r]
        Q = np.eye(dk)[:, start]
        for _ in range(iters):
            Q, Rq = np.linalg.qr(S64 @ S64.T @ Q)
            Q = Q * np.sign(np.diag(Rq))
        np.testing.assert_allclose(b["comp_key"][s].astype(np.float64), Q.T, atol=1e-6)
        np.testing.assert_array_equal(b["comp_idx"][s], start)


@pytest.mark.parametrize("r,iters", [(4, 1), (4, 2), (8, 2)])
def test_reconstruction_half_step_bound(r, iters):
    """|S - B| <= (a s / 2)(1 + 1e-4) + 2^-23 (|S| + |K^T W|): the quantizer's
    half step on the residual, plus the one fp32 rounding of the residual."""
    rng = np.random.default_rng(900 + r + iters)
    S = _states(rng, 4)
    b = O.quantize(S, r, DENSE, iters=iters)
    B = O.dequantize(b)
    for s in range(4):
        K = b["comp_key"][s].astype(np.float64)
        W = b["comp_val"][s].astype(np.float64)
        S64 = S[s].astype(np.float64)
        step_ = b["row_scale"][s][:, None].astype(np.float64) * b["col_scale"][s][None, :].astype(np.float64)
        bound = 0.5 * step_ * (1 + 1e-4) + 2.0 ** -23 * (np.abs(S64) + np.abs(K.T @ W))
        assert np.all(np.abs(S64 - B[s]) <= bound)


def test_rank_deficient_and_zero_states():
    rng = np.random.default_rng(1000)
    a = rng.standard_normal((128, 2))
    c = rng.standard_normal((2, 128))
    S = np.stack([(a @ c).astype(np.float32), np.zeros((128, 128), np.float32)])
    b = O.quantize(S, 4, DENSE, iters=2)
    K = b["comp_key"].astype(np.float64)
    np.testing.assert_allclose(K[0, :2] @ K[0, :2].T, np.eye(2), atol=2e-6)
    np.testing.assert_array_equal(K[0, 2:], 0)        # past the rank: zero keys
    np.testing.assert_array_equal(b["comp_val"][0, 2:], 0)
    np.testing.assert_array_equal(K[1], 0)            # zero state: zero keys, values, codes
    np.testing.assert_array_equal(b["comp_val"][1], 0)
    np.testing.assert_array_equal(b["codes"][1], 0)
    # the rank-2 state is carried almost entirely by its two tokens
    B = O.dequantize(b)
    assert np.abs(B[0] - S[0]).max() <= 1e-5 * np.abs(S[0]).max()


def test_dense_tokens_follow_the_update_path():
    """A window from a dense boundary equals the plain recurrence started at
    the dequantized boundary, compensator tokens included, and the next
    boundary carries fresh dense tokens."""
    rng = np.random.default_rng(1100)
    n, T, r = 2, 5, 4
    S0 = _states(rng, n)
    b0 = O.quantize(S0, r, DENSE, iters=2)
    q = rng.standard_normal((T, n, 128)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((T, n, 128)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    tok = {"q": q, "k": k, "v": rng.standard_normal((T, n, 128)),
           "beta": rng.uniform(0.05, 1, (T, n)), "alpha": rng.uniform(0.05, 1, (T, n))}
    o_w, _, S_end, b1 = O.window(b0, tok, 0, T, O.GATE_GDN, r, DENSE, iters=2)
    o_ref, S_ref, _ = O.sequential_exact(O.dequantize(b0), tok, O.GATE_GDN)
    np.testing.assert_allclose(o_w, o_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S_end, S_ref, rtol=1e-12, atol=1e-12)
    assert b1["comp_key"].shape == (n, r, 128)
