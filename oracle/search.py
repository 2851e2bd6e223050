"""Smooth-factor grid search of one layer (test infrastructure only).

AutoRound doc, "Smooth search": with G grid points the candidate exponent
pairs are (alpha, beta) = (0, 0), then (a/G, 0) for a = 1 .. G-1, then
(a/G, 1 - a/G) for the same a: 2G - 1 pairs, 39 at the default G = 20.
Each candidate sets lambda = x_span^alpha / w_span^beta, prepares the layer
with it, and is scored by how far the layer's output on the calibration
inputs lands from the floating-point output X W; the finite smallest score
wins.

Readings (the pages leave these open):
S1  x_span / w_span are the per-input-channel absolute maxima of the
    calibration activations and of the weight rows, the statistics Eq. (4)
    of the Zhou notes uses.
S2  The candidate output is the deployed layer's output, W4A4 with the
    low-rank branch (activations quantized, Y rounded to bf16), without the
    bias, which both sides share.
S3  The score is the relative Frobenius error ||Y - X W||_F / ||X W||_F
    (any monotone function of the squared error selects the same pair);
    ties keep the earlier candidate in the order above.

Pins (tests/test_oracle_search.py): the candidate set against the pages'
count and description, the selection rule on hand-made score lists, an
exactly representable layer for which only (0, 0) is lossless, and an
outlier-activation layer for which smoothing must win.
"""

import numpy as np

from . import forward as F
from . import prepare as P
from .rounding import round_bf16


def candidates(grids=20):
    """The (alpha, beta) pairs in the pages' order."""
    g = int(grids)
    if g < 2:
        raise ValueError("grids must be >= 2")
    out = [(0.0, 0.0)]
    out += [(a / g, 0.0) for a in range(1, g)]
    out += [(a / g, 1.0 - a / g) for a in range(1, g)]
    return out


def output_error(y, y_ref):
    """S3: relative Frobenius error in fp64."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    return float(np.linalg.norm(y - y_ref) / np.linalg.norm(y_ref))


def select(errors):
    """Index of the smallest finite score (first on ties); None if none is finite."""
    best = None
    for i, e in enumerate(errors):
        if np.isfinite(e) and (best is None or e < errors[best]):
            best = i
    return best


def smooth_search(w, x_cal, rank, fmt, grids=20, residual_iters=1):
    """Score every candidate on x_cal ([M, K] bf16 values); returns
    (best index, list of (alpha, beta), list of scores)."""
    w = np.asarray(w, dtype=np.float64)
    x = np.asarray(x_cal, dtype=np.float64)
    amax = P.calib_amax(x)
    y_ref = x @ w
    pairs = candidates(grids)
    errors = []
    for alpha, beta in pairs:
        layer = P.prepare(w, amax, alpha, rank, fmt, beta=beta, residual_iters=residual_iters)
        y = F.forward(x, layer)["y"]
        errors.append(output_error(round_bf16(y), y_ref))
    return select(errors), pairs, errors
