"""Planted mistakes in the CPU oracle, for checking that its pins bite.

Each mutant names one function of oracle/leapquant_oracle.py, a snippet of
its source and the mistaken snippet that replaces it: a plausible slip in
transcribing the method (a dropped term, a wrong sign or index, a
transposed operand, a wrong rounding).  `apply(name)` recompiles the
function from the edited source inside the oracle module, so every caller
in the module and in the tests sees the mistake.  A mutant whose snippet no
longer occurs in the oracle raises, so the list cannot silently go stale.

Used by tests/conftest.py when LQ_ORACLE_MUTANT names a mutant (only in the
subprocesses that tests/test_oracle_mutants.py starts).
"""
import inspect
import textwrap

from oracle import leapquant_oracle as O

# name -> (function, original snippet, mistaken snippet)
MUTANTS = {
    # the recurrence ([EL] Appendix Table 4)
    "dropped_decay": ("step", "S_new = d[:, :, None] * S + ", "S_new = S + "),
    "u_sign": ("step", "u = np.asarray(v, np.float64) - np.einsum", "u = np.asarray(v, np.float64) + np.einsum"),
    "b_is_k": ("transition", "else d * k", "else k"),
    "output_before_update": ("step", 'o = np.einsum("nij,ni->nj", S_new,', 'o = np.einsum("nij,ni->nj", S,'),
    "decay_on_wrong_axis": ("step", "S_new = d[:, :, None] * S", "S_new = d[:, None, :] * S"),
    # the split of the boundary state ([EL] Abstract, Figure 4; [TM])
    "smooth_before_extraction": ("quantize", "col_scale = np.abs(R).max(axis=1)", "col_scale = np.abs(S32).max(axis=1)"),
    "smallest_norm_rows": ("quantize", "np.argsort(-norm2,", "np.argsort(norm2,"),
    "truncating_rounding": ("quantize", "np.clip(np.rint(X),", "np.clip(np.trunc(X),"),
    "round_half_up": ("quantize", "np.clip(np.rint(X),", "np.clip(np.floor(X + 0.5),"),
    "row_scale_over_columns": ("quantize", "m = np.abs(Q).max(axis=2)", "m = np.abs(Q).max(axis=1)"),
    "extracted_rows_kept": ("quantize", "R[s, comp_idx[s], :] = 0", "R[s, comp_idx[s], :] = R[s, comp_idx[s], :]"),
    "dequantize_transposed_scales": ("dequantize", "B = c * a[:, :, None] * s[:, None, :]",
                                     "B = c * a[:, None, :] * s[:, :, None]"),
    # windows ([EL] Figure 2)
    "window_one_token_long": ("run_windowed", "length = min(p, T - t0)", "length = min(p + 1, T - t0)"),
    # dense compensator tokens (second reading of [EL] Figure 4)
    "iteration_on_wrong_side": ("dense_keys", "K = mgs(S64 @ (S64.T @ K), rr, kk)", "K = mgs(S64.T @ (S64 @ K), rr, kk)"),
    "keys_not_normalized": ("mgs", "K[:, c] = v / nv", "K[:, c] = v"),
    "keys_not_projected": ("mgs", "v = v - (K[:, c2] @ v) * K[:, c2]", "v = v"),
    "no_drop_threshold": ("mgs", "kept = nv > 0 and nv > MGS_DROP * n0", "kept = nv > 0"),
    "one_iteration_too_many": ("dense_keys", "for it in range(iters):", "for it in range(iters + 1):"),
    "values_from_rows": ("quantize", "W32 = (K.T @ S64[s])", "W32 = (K.T @ S64[s].T)"),
    "residual_sign": ("quantize", "R[s] = (S64[s] - K @ W32", "R[s] = (S64[s] + K @ W32"),
    "residual_outer_transposed": ("quantize", "R[s] = (S64[s] - K @ W32.astype(np.float64))",
                                  "R[s] = (S64[s] - (K @ W32.astype(np.float64)).T)"),
}


def apply(name):
    """Replace the named function of the oracle module by its mutated copy."""
    func_name, old, new = MUTANTS[name]
    src = textwrap.dedent(inspect.getsource(getattr(O, func_name)))
    if src.count(old) != 1:
        raise RuntimeError(f"mutant {name}: snippet not found exactly once in oracle.{func_name}")
    code = compile(src.replace(old, new), f"<mutant {name}>", "exec")
    exec(code, O.__dict__)  # rebinds O.<func_name> in the module namespace
