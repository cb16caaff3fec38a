"""Normwise error metrics and the output tolerance (test infrastructure only).

The tolerance for floating-point GEMM outputs is max relative error 1e-2 and
RMS relative error 2e-3.  Element-wise relative error is ill-posed where the
reference is near zero, so both are normwise over one output tensor:

    max_rel = max_i |y_i - r_i| / max_i |r_i|
    rms_rel = ||y - r||_2 / ||r||_2
"""

import numpy as np

MAX_REL_TOL = 1e-2
RMS_REL_TOL = 2e-3


def normwise_errors(y, ref):
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert y.shape == ref.shape, (y.shape, ref.shape)
    diff = y - ref
    ref_max = np.max(np.abs(ref)) if ref.size else 0.0
    ref_norm = np.linalg.norm(ref.ravel())
    max_rel = float(np.max(np.abs(diff)) / ref_max) if ref_max > 0 else float(np.max(np.abs(diff), initial=0.0))
    rms_rel = float(np.linalg.norm(diff.ravel()) / ref_norm) if ref_norm > 0 else float(np.linalg.norm(diff.ravel()))
    return max_rel, rms_rel


def within_tolerance(y, ref, max_rel_tol=MAX_REL_TOL, rms_rel_tol=RMS_REL_TOL):
    max_rel, rms_rel = normwise_errors(y, ref)
    return (max_rel <= max_rel_tol and rms_rel <= rms_rel_tol), max_rel, rms_rel
