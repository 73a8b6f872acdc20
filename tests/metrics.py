"""Error measures used by the parity tests.

Outputs of linear attention are convex combinations of zero-mean values, so single
elements can sit near zero and an elementwise relative error is ill-conditioned.  The bar
is therefore normwise per head slice:

    err = max over heads of  max_{i,c} |g - r|  /  max_{i,c} |r|

with r the fp64 oracle and g the GPU result decoded exactly to fp64.  An elementwise error
with a floor, |g - r| / max(|r|, 1e-3 max|r|), is reported alongside for information.

Causal outputs are not of one size along a head: out_i averages i + 1 values, so its size
falls like 1/sqrt(i + 1) for zero-mean values (row 0 of a 65,536-token head is about 300 times
row 65,535).  A bar relative to the whole head would then check late rows hardly at all, so
the causal forms are measured per row, each row against its own size:

    err = max over rows (b, h, i) of  max_c |g - r|  /  max_c |r|
"""
import numpy as np

TOL_F32 = 1e-4
TOL_BF16 = 2e-2


def normwise_err(g, r, head_axes_last=2):
    g = np.asarray(g, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    if g.shape != r.shape:
        raise ValueError("shape mismatch %s vs %s" % (g.shape, r.shape))
    if g.size == 0:
        return 0.0
    lead = g.shape[:-head_axes_last] if g.ndim > head_axes_last else ()
    gg = g.reshape((int(np.prod(lead)) if lead else 1, -1))
    rr = r.reshape(gg.shape)
    if not np.all(np.isfinite(gg)):
        return float("inf")
    num = np.abs(gg - rr).max(axis=1)
    den = np.abs(rr).max(axis=1)
    return float(np.max(num / den))


def floored_elementwise_err(g, r, floor=1e-3):
    g = np.asarray(g, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    if g.size == 0:
        return 0.0
    m = np.abs(r).max()
    return float(np.max(np.abs(g - r) / np.maximum(np.abs(r), floor * m)))


def rowwise_err(g, r):
    """Max over rows (the last axis holds one output row) of max_c |g - r| / max_c |r|; a row
    whose reference is exactly zero must match exactly."""
    g = np.asarray(g, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    if g.shape != r.shape:
        raise ValueError("shape mismatch %s vs %s" % (g.shape, r.shape))
    if g.size == 0:
        return 0.0
    gg = g.reshape(-1, g.shape[-1])
    rr = r.reshape(gg.shape)
    if not np.all(np.isfinite(gg)):
        return float("inf")
    num = np.abs(gg - rr).max(axis=1)
    den = np.abs(rr).max(axis=1)
    zero = den == 0
    if np.any(num[zero] != 0):
        return float("inf")
    return float(np.max(num[~zero] / den[~zero])) if np.any(~zero) else 0.0


def form_err(form, g, r):
    """The measure of a form: per row for causal outputs, per head otherwise."""
    return rowwise_err(g, r) if form == "causal" else normwise_err(g, r)
