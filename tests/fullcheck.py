"""Every-element comparison of a device result with the oracle, in row chunks.

The oracle's reference and bound for a full 8192 x 8192 output take 1 GiB of
float64 each; computing them a block of rows at a time keeps host memory
small while still checking every element.
"""

import numpy as np

import oracle


def check_all_rows(out, oracle_rows, fmt="f32", chunk=1024):
    """Assert the acceptance rule on every element of ``out`` (a 2-D device tensor).

    ``oracle_rows(r0, r1)`` returns the oracle's (ref, bound) for rows
    [r0, r1); ``fmt`` is the output format ('f32', 'f16' or 'bf16').
    Returns the worst error over its allowance.
    """
    M = out.shape[0]
    worst = 0.0
    for r0 in range(0, M, chunk):
        r1 = min(M, r0 + chunk)
        got = out[r0:r1].float().double().cpu().numpy()
        ref, bound = oracle_rows(r0, r1)
        ok, w, n_bad = oracle.within_bound_out(got, ref, bound, fmt)
        assert ok, f"rows {r0}..{r1 - 1}: {n_bad} elements outside the bound (worst {w:.3g})"
        worst = max(worst, w)
    return worst


def rows_of(X, r0, r1):
    return np.asarray(X)[r0:r1]
