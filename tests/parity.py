"""Parity metric between a GPU result and the fp64 oracle.

For each (sequence, value head) slice s of a tensor (outputs or final
states), e_s = max_i |x_i - r_i| / max_i |r_i|; a tensor passes when
max_s e_s <= tol and it holds no NaN or Inf. The tolerance is 2e-2 for
bf16 inputs and 1e-4 for fp32 inputs. Normalising by the slice's largest
reference value (rather than element by element) keeps the metric defined
where outputs cross zero.
"""
import numpy as np

from gdn_synth import bf16_to_f32

TOL = {"bf16": 2e-2, "f32": 1e-4}


def as_f64(x):
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return bf16_to_f32(x).astype(np.float64)
    return x.astype(np.float64)


def slice_error(x, r):
    """x, r: arrays of one slice. Returns e_s (0 when r is all zero and x == r)."""
    x = as_f64(x)
    r = as_f64(r)
    if not np.all(np.isfinite(x)):
        return float("inf")
    den = np.max(np.abs(r)) if r.size else 0.0
    num = np.max(np.abs(x - r)) if r.size else 0.0
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)


def max_error(x, r, slice_axes):
    """Max of slice errors; slices are indexed by the axes in slice_axes
    (e.g. (0, 2) for outputs [B,T,Hv,D]: sequence and head)."""
    x = as_f64(x)
    r = as_f64(r)
    axes = list(slice_axes)
    rest = [a for a in range(x.ndim) if a not in axes]
    xp = np.transpose(x, axes + rest).reshape([np.prod([x.shape[a] for a in axes], dtype=int), -1])
    rp = np.transpose(r, axes + rest).reshape(xp.shape)
    worst = 0.0
    for i in range(xp.shape[0]):
        worst = max(worst, slice_error(xp[i], rp[i]))
    return worst
