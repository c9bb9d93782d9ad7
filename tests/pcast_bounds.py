"""Error bound for the E4M3 P-cast path, used by oracle pins and GPU tests.

With exact attention weights a_j (row-normalised) and p_j = a_j / max(a) the
probability relative to the row's final maximum, casting S*p to E4M3 with
round-to-nearest-even perturbs each weight by a relative amount r_j:
  r_j = 2^-4                     if S*p_j >= 2^-6 (normal: half an ulp of a
                                 3-bit mantissa),
  r_j = min(1, 2^-10 / (S*p_j))  otherwise (subnormal grid 2^-9, half step
                                 2^-10; a flushed value loses all of it).
A running maximum never exceeds the final one, so the p the kernel casts is
at least p_j and the same r_j bounds its error.  The normaliser is the sum of
the uncast p, so  |O_pcast - O| <= sum_j a_j r_j |v_j|  per output element;
`slack` adds fp32 rounding of logits, exponentials and sums.  The MSE bound is
the mean of the squared per-element bounds.
"""
import numpy as np


def pcast_bound(a_rows: np.ndarray, v_rows: np.ndarray, S: float, slack: float = 2e-5):
    """a_rows: [R, Nk] exact weights; v_rows: [R, Nk, d] (or [Nk, d] shared).
    Returns the per-element bound [R, d]."""
    mx = a_rows.max(axis=1, keepdims=True)
    p = np.divide(a_rows, mx, out=np.zeros_like(a_rows, dtype=np.float64), where=mx > 0)
    sp = S * p
    with np.errstate(divide="ignore"):
        r = np.where(sp >= 2.0 ** -6, 2.0 ** -4, np.minimum(1.0, 2.0 ** -10 / sp))
    r = np.where(a_rows > 0, r, 0.0)
    av = np.abs(v_rows.astype(np.float64))
    if av.ndim == 2:
        core = (a_rows * r) @ av
        scale = a_rows @ av
    else:
        core = np.einsum("rj,rjc->rc", a_rows * r, av)
        scale = np.einsum("rj,rjc->rc", a_rows, av)
    return core + slack * scale + 1e-7
