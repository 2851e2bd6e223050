"""Smooth-factor grid search of one layer (test infrastructure only).

AutoRound doc, "Smooth search": with G grid points the candidate exponent
pairs are (alpha, beta) = (0, 0), then (a/G, 0) for a = 1 .. G-1, then
(a/G, 1 - a/G) for the same a: 2G - 1 pairs, 39 at the default G = 20.
Each candidate sets lambda = x_span^alpha / w_span^beta, prepares the layer
with it, and is scored by how far the layer's output on the calibration
inputs lands from the floating-point output X W; the finite smallest score
wins.

With residual iteration on (the doc: "Residual iteration"), each
candidate's iterations are scored by that same calibration output error,
not by the weight error the doc names for runs without smooth search, and
the candidate's score is that of its kept iteration.

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

The doc caps the calibration calls each group keeps by reservoir sampling.
S4  Reading: Algorithm R (Vitter, "Random sampling with a reservoir", ACM
    TOMS 1985): the first k calls fill the reservoir; call i >= k draws j
    uniform in 0..i and replaces slot j when j < k.  The draws come from
    SplitMix64 (Steele, Lea and Flood, OOPSLA 2014) seeded with the caller's
    seed, one output per call i >= k, mapped to 0..i by the high 64 bits of
    the 128-bit product output * (i + 1).  The kept call indices are returned
    in increasing order.

Pins (tests/test_oracle_search.py): the candidate set against the pages'
count and description, the selection rule on hand-made score lists, an
exactly representable layer for which only (0, 0) is lossless, an
outlier-activation layer for which smoothing must win, the reservoir's
inclusion frequencies (k / n for every call) over many seeds, and SplitMix64
against its published first outputs for two seeds (tests/golden/splitmix64.json).
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


MASK64 = (1 << 64) - 1


def splitmix64(state):
    """One SplitMix64 step: (next state, output), 64-bit unsigned ints."""
    state = (state + 0x9E3779B97F4A7C15) & MASK64
    z = state
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return state, z ^ (z >> 31)


def reservoir_select(n_calls, k, seed):
    """S4: indices of the calls kept by a reservoir of size k."""
    n_calls, k = int(n_calls), int(k)
    if k <= 0 or n_calls <= 0:
        return []
    slots = list(range(min(k, n_calls)))
    state = int(seed) & MASK64
    for i in range(k, n_calls):
        state, r = splitmix64(state)
        j = (r * (i + 1)) >> 64
        if j < k:
            slots[j] = i
    return sorted(slots)


def candidate_score(x, y_ref):
    """S2 + S3 as a function of a deployable layer: the relative error of
    its bf16-rounded output on the calibration rows."""
    return lambda layer: output_error(round_bf16(F.forward(x, layer)["y"]), y_ref)


def smooth_search(w, x_cal, rank, fmt, grids=20, residual_iters=1, early_stop=False, details=None):
    """Score every candidate on x_cal ([M, K] bf16 values); returns
    (best index, list of (alpha, beta), list of scores).  `details`, if a
    list, receives per candidate the prepared layer's kept iteration and its
    per-iteration scores."""
    w = np.asarray(w, dtype=np.float64)
    x = np.asarray(x_cal, dtype=np.float64)
    amax = P.calib_amax(x)
    y_ref = x @ w
    score = candidate_score(x, y_ref)
    pairs = candidates(grids)
    errors = []
    for alpha, beta in pairs:
        layer = P.prepare(w, amax, alpha, rank, fmt, beta=beta, residual_iters=residual_iters,
                          early_stop=early_stop, score=score)
        errors.append(min(layer["iter_errors"]))
        if details is not None:
            details.append({"best_iter": layer["best_iter"], "iter_scores": list(layer["iter_errors"])})
    return select(errors), pairs, errors
