"""Offline preparation of one SVDQuant layer (test infrastructure only).

Orientation: X is [M, K] (tokens x in-features), W is [K, N] and Y = X W
(Zhou notes, sec. 2.1).  The msModelSlim doc and the MindStudio entry use
PyTorch's [out, in] weight; their V^T / U*S pair maps to our L1 / L2 up to
where Sigma sits.

Steps, in the order of Algorithm 1 of the Zhou notes (sec. 5):

O1 smoothing factor (Zhou notes sec. 3.1, Eq. (4); msModelSlim doc stage 1):
       lambda_i = amaxX_i**alpha / amaxW_i**(1 - alpha),
   amaxX_i the calibration per-channel max |X[:, i]|, amaxW_i = max_j |W[i, j]|
   over the whole row (for a grouped QKV weight: across Q, K and V).  The
   pages leave zero statistics open; reading taken: lambda_i = 1 when either
   statistic is 0.  lambda is stored as fp32 and the runtime uses
   inv_lambda = fp32(1 / lambda32).
O2 W~ = diag(lambda32) W (Zhou notes Eq. (3); D left-multiplies W, the notes
   flag the paper's W diag(lambda) as a dimension error).
O3 W~ = U S V^T, L1 = U[:, :r] S[:r], L2 = V[:, :r]^T (Zhou notes sec. 5,
   Eq. (10)).  Exact SVD, Sigma on the down side (the Zhou notes are the
   authority; the msModelSlim doc's randomized svd_lowrank with Sigma on the
   up side differs only by where the bf16 rounding falls).
O4 L1b = bf16(L1), L2b = bf16(L2), R = W~ - L1b L2b in fp64, R32 = fp32(R)
   (AutoRound doc, "Residual iteration": the factors are materialized in
   low_rank_dtype, bf16 by default, before R = W - U @ V).
O5 LoRA attach (Zhou notes sec. 7, Eq. (13)): L1' = [L1b | bf16(D A)],
   L2' = [L2b ; bf16(s B)]; R and its codes are untouched, no re-truncation.
O6 weight packing: the quantizer of the chosen format applied to R32^T
   ([N, K], grouped along K).

O-RI residual iterations (AutoRound doc, "Residual iteration"): refit the
   branch to W~ - Q(R_prev), keep the candidate with the smallest score,
   optionally stop at the first worse one.  The doc scores candidates by
   the weight reconstruction error ||W~ - L1b L2b - Q(R)||_F when smooth
   search is off and by the calibration output error when it is on; the
   second is passed in by the smooth search (oracle.search) as `score`.

Pins (tests/test_oracle_prepare.py): Eq. (3) smoothing invariance (bit
identical for power-of-two lambda), Eckart-Young tail energy, R = 0 at full
rank, optimality against random rank-r competitors, a hand-computed lambda,
QKV column-block equality, the Eq. (13) LoRA identity.
"""

import numpy as np

from .rounding import round_bf16, to_f32
from .quantizers import quantize


def calib_amax(x_cal):
    """Per-input-channel max |X| over calibration rows (Algorithm 1, step 1).

    x_cal: [rows, K] values.  Returns fp32 [K].
    """
    return np.max(np.abs(np.asarray(x_cal, dtype=np.float64)), axis=0).astype(np.float32)


def smoothing_factors(act_amax, w, alpha, beta=None):
    """O1: lambda32 and inv_lambda (both fp32 [K]).  The weight exponent is
    beta (AutoRound doc, "Smooth search": lambda = x_span^alpha /
    w_span^beta); None means 1 - alpha, Eq. (4) of the notes."""
    ax = np.asarray(act_amax, dtype=np.float64)
    aw = np.max(np.abs(np.asarray(w, dtype=np.float64)), axis=1)
    b = 1.0 - alpha if beta is None else beta
    with np.errstate(divide="ignore", invalid="ignore"):
        lam = ax ** alpha / aw ** b
    lam = np.where((ax == 0) | (aw == 0), 1.0, lam)
    lam32 = to_f32(lam)
    inv = (np.float32(1.0) / lam32).astype(np.float32)
    return lam32, inv


def smooth_weight(w, lam32):
    """O2: diag(lambda32) W in fp64 (exact: 24-bit times bf16 values)."""
    return np.asarray(lam32, dtype=np.float64)[:, None] * np.asarray(w, dtype=np.float64)


def truncated_svd(wt, rank):
    """O3: rank-r factors (fp64) and all singular values."""
    u, s, vt = np.linalg.svd(wt, full_matrices=False)
    l1 = u[:, :rank] * s[:rank]
    l2 = vt[:rank, :]
    return l1, l2, s


def _candidate(wt, target, rank, fmt):
    """One low-rank fit of `target` and the residual of wt it leaves (steps
    O3-O6 with the fit taken on `target`)."""
    l1, l2, sig = truncated_svd(target, rank)
    l1b = round_bf16(l1)
    l2b = round_bf16(l2)
    r = wt - l1b @ l2b
    r32 = to_f32(r)
    q = quantize(r32.T.copy(), fmt)
    err = float(np.linalg.norm(wt - l1b @ l2b - q["deq"].T))
    return {"l1": l1, "l2": l2, "sigma": sig, "l1b": l1b, "l2b": l2b, "r": r, "r32": r32, "q": q, "err": err}


def residual_iterations(wt, rank, fmt, iters=1, early_stop=False, keep_all=False, score=None):
    """Residual iteration (AutoRound doc, "Residual iteration"; Zhou notes
    sec. 5, the alternating update of the protected branch).

    Iteration 1 fits the rank-r branch to W~ itself.  Every further
    iteration fits it to W~ - Q(R_prev), Q the deployment RTN
    quantize-dequantize of the previous residual, then takes the new
    residual R = W~ - L1b L2b.  A candidate's score is score(candidate)
    when a scoring function is given (the smooth search passes the
    calibration output error), else its weight reconstruction error
    ||W~ - L1b L2b - Q(R)||_F in smoothed coordinates (the doc's objective
    without smooth search).  The candidate with the smallest score is kept
    (the earlier on ties; a non-finite score never displaces a finite one);
    with early_stop the loop ends at the first iteration whose score is
    larger than the best so far.
    Returns (best candidate, list of scores per iteration run, all
    candidates if keep_all).
    """
    cands, errors = [], []
    best = None
    target = wt
    for it in range(max(1, int(iters))):
        c = _candidate(wt, target, rank, fmt)
        c["iteration"] = it
        c["score"] = c["err"] if score is None else float(score(c))
        errors.append(c["score"])
        if keep_all:
            cands.append(c)
        if (best is None or c["score"] < best["score"]
                or (not np.isfinite(best["score"]) and np.isfinite(c["score"]))):
            best = c
        elif early_stop and c["score"] > best["score"]:
            break
        target = wt - c["q"]["deq"].T
    return best, errors, cands


def candidate_layer(c, lam32, inv, fmt, rank, lora=None):
    """The deployable layer (the dict oracle.forward reads) of one residual
    iteration candidate."""
    l1p, l2p = c["l1b"], c["l2b"]
    if lora is not None:
        l1p, l2p = attach_lora(l1p, l2p, lam32, lora["A"], lora["B"], lora.get("strength", 1.0))
    return {"fmt": fmt, "rank": rank, "lam32": lam32, "inv_lambda": inv, "l1p": l1p, "l2p": l2p,
            "wq_packed": c["q"]["packed"], "ws": c["q"]["scales"]}


def prepare(w, act_amax, alpha, rank, fmt, lora=None, residual_iters=1, early_stop=False, beta=None,
            score=None):
    """Prepare one layer.

    w: [K, N] weight values, act_amax: [K], alpha in [0, 1], rank r >= 0,
    fmt 'int4' | 'mxfp4', lora: optional dict(A=[K, k], B=[k, N], strength=s),
    residual_iters / early_stop: see residual_iterations (1 = one SVD),
    beta: weight exponent of lambda (None: 1 - alpha), score: optional
    function of a candidate's deployable layer (candidate_layer) that
    scores residual iterations in place of the weight error.
    Returns a dict of every intermediate the pins and the forward need.
    """
    w = np.asarray(w, dtype=np.float64)
    lam32, inv = smoothing_factors(act_amax, w, alpha, beta)
    wt = smooth_weight(w, lam32)
    sc = None if score is None else (lambda c: score(candidate_layer(c, lam32, inv, fmt, rank, lora)))
    c, errors, _ = residual_iterations(wt, rank, fmt, residual_iters, early_stop, score=sc)
    l1, l2, sig = c["l1"], c["l2"], c["sigma"]
    l1b, l2b = c["l1b"], c["l2b"]
    r_exact = wt - l1 @ l2
    wq = c["q"]
    l1p, l2p = l1b, l2b
    if lora is not None:
        l1p, l2p = attach_lora(l1b, l2b, lam32, lora["A"], lora["B"], lora.get("strength", 1.0))
    return {
        "lam32": lam32, "inv_lambda": inv, "w_tilde": wt, "sigma": sig,
        "l1": l1, "l2": l2, "l1b": l1b, "l2b": l2b,
        "l1p": l1p, "l2p": l2p,
        "r_exact": r_exact, "r": c["r"], "r32": c["r32"],
        "wq_packed": wq["packed"], "ws": wq["scales"], "wq_codes": wq["codes"],
        "w_deq": wq["deq"], "fmt": fmt, "rank": rank,
        "iter_errors": errors, "best_iter": c["iteration"],
    }


def attach_lora(l1b, l2b, lam32, a, b, strength=1.0):
    """O5: concatenate a LoRA adapter A B into the low-rank branch.

    In smoothed coordinates the adapter is D A B (Zhou notes Eq. (13)); the
    strength is absorbed into B.
    """
    da = np.asarray(lam32, dtype=np.float64)[:, None] * np.asarray(a, dtype=np.float64)
    sb = float(strength) * np.asarray(b, dtype=np.float64)
    return (np.concatenate([l1b, round_bf16(da)], axis=1),
            np.concatenate([l2b, round_bf16(sb)], axis=0))


def prepare_grouped(ws, act_amax, alpha, rank, fmt):
    """QKV grouping (AutoRound doc, processing flow): the projections that
    read the same input are processed as one group with one shared down
    factor and separate up factors.  Reading taken: one lambda and one SVD of
    the column concatenation [Wq | Wk | Wv]; the separate up factors are the
    column blocks of L2.  Returns the layer dict plus 'splits'.
    """
    w = np.concatenate([np.asarray(x, dtype=np.float64) for x in ws], axis=1)
    out = prepare(w, act_amax, alpha, rank, fmt)
    edges = np.cumsum([0] + [x.shape[1] for x in ws])
    out["splits"] = [(int(a), int(b)) for a, b in zip(edges[:-1], edges[1:])]
    return out
