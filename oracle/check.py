"""Tolerance check of a GPU result against the fp64 oracle.

TEST INFRASTRUCTURE (see oracle/__init__.py).

Bars (applied per call, to whatever block of outputs was computed):

* no NaN or Inf anywhere in the GPU output;
* per element: |y - y_ref| <= ELEM_TOL * max |y_ref|;
* per row:     ||y_row - y_ref_row||_2 <= ROW_TOL * ||y_ref_row||_2
  (a row whose reference is all zero must come back all zero).

Why these bars separate right from wrong: an fp32 sum of K terms carries a
relative error of at most about K * 2^-24 of sum |x_k w_k| (Higham, Accuracy and
Stability of Numerical Algorithms, ch. 3), and the fp16 output adds at most
2^-11 |y|.  A swapped nibble, a wrong group index or a dropped group instead
gives an O(1) relative error in the rows it touches.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

ELEM_TOL = 4e-3
ROW_TOL = 1e-3


@dataclass
class Report:
    ok: bool
    max_abs_err: float
    elem_bound: float
    worst_row_rel_l2: float
    first_bad: tuple | None
    message: str

    def __bool__(self):
        return self.ok


def compare(y, y_ref, elem_tol: float = ELEM_TOL, row_tol: float = ROW_TOL) -> Report:
    y = np.asarray(y).astype(np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    if y.shape != y_ref.shape:
        return Report(False, np.inf, 0.0, np.inf, None, f"shape {y.shape} != {y_ref.shape}")
    if y.size == 0:
        return Report(True, 0.0, 0.0, 0.0, None, "empty")
    finite = np.isfinite(y)
    if not finite.all():
        idx = tuple(int(i) for i in np.argwhere(~finite)[0])
        return Report(False, np.inf, 0.0, np.inf, idx, f"non-finite output at {idx}")
    y2 = y.reshape(-1, y.shape[-1])
    r2 = y_ref.reshape(-1, y_ref.shape[-1])
    err = np.abs(y2 - r2)
    bound = elem_tol * float(np.max(np.abs(r2)))
    max_err = float(err.max())
    row_err = np.sqrt(np.sum((y2 - r2) ** 2, axis=1))
    row_ref = np.sqrt(np.sum(r2 ** 2, axis=1))
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(row_ref > 0, row_err / np.where(row_ref > 0, row_ref, 1.0),
                       np.where(row_err > 0, np.inf, 0.0))
    worst = float(rel.max())
    bad_elem = np.argwhere(err > bound)
    bad_rows = np.flatnonzero(rel > row_tol)
    if bad_elem.size:
        r, c = (int(v) for v in bad_elem[0])
        return Report(False, max_err, bound, worst, (r, c),
                      f"element ({r},{c}): |err| {err[r, c]:.3e} > {bound:.3e} "
                      f"(got {y2[r, c]!r}, want {r2[r, c]!r})")
    if bad_rows.size:
        r = int(bad_rows[0])
        return Report(False, max_err, bound, worst, (r, None),
                      f"row {r}: rel L2 {rel[r]:.3e} > {row_tol:.1e}")
    return Report(True, max_err, bound, worst, None,
                  f"ok: max|err| {max_err:.3e} <= {bound:.3e}, worst row rel L2 {worst:.3e}")
