"""Pins of the oracle's smooth-factor grid search (AutoRound doc, "Smooth
search"): the candidate set the section describes, the finite-minimum
selection, and two layers whose winner is fixed by the mathematics."""
import numpy as np
import pytest

from oracle import search as SR
from oracle import prepare as P
from rank_gemm_svdq_amd import synthetic as S


def test_candidate_set_default_grid():
    c = SR.candidates(20)
    assert len(c) == 39                                    # the count the section states for G = 20
    assert c[0] == (0.0, 0.0)
    assert len(set(c)) == 39
    beta0 = [a for a, b in c[1:] if b == 0.0]
    paired = [(a, b) for a, b in c[1:] if b != 0.0]
    assert beta0 == [k / 20 for k in range(1, 20)]
    assert [a for a, _ in paired] == beta0
    assert all(abs(a + b - 1.0) < 1e-15 for a, b in paired)
    assert len(SR.candidates(2)) == 3
    with pytest.raises(ValueError):
        SR.candidates(1)


def test_select_finite_minimum():
    assert SR.select([0.3, 0.1, 0.2]) == 1
    assert SR.select([np.nan, 0.5, np.inf, 0.5, 0.4]) == 4
    assert SR.select([0.2, 0.2]) == 0                      # ties keep the earlier candidate
    assert SR.select([np.nan, np.inf]) is None


def test_exactly_representable_layer_selects_no_smoothing():
    # X and W hold exact INT4 grid values with a full-scale element in every
    # group of 64, so with lambda = 1 and no branch both quantize without
    # loss and only the bf16 rounding of Y remains.  Channel ranges differ,
    # so every other candidate has a non-uniform lambda and moves values off
    # the grid.
    rng = np.random.default_rng(3)
    M, K, N = 64, 256, 128
    cx = rng.integers(1, 8, K)                              # per-channel code range
    cw = rng.integers(1, 8, K)
    x = np.round(rng.uniform(-1, 1, (M, K)) * cx).astype(np.float64)
    x[:, ::64] = 7.0
    w = np.round(rng.uniform(-1, 1, (K, N)) * cw[:, None]) / 64.0
    w[::64, :] = 7.0 / 64.0
    best, pairs, errs = SR.smooth_search(w, x, 0, "int4", grids=4)
    y_ref = x @ w
    bf16_only = np.linalg.norm(P.round_bf16(y_ref) - y_ref) / np.linalg.norm(y_ref)
    assert best == 0 and pairs[best] == (0.0, 0.0)
    assert errs[0] == pytest.approx(bf16_only, rel=1e-12)
    assert min(errs[1:]) > 2 * errs[0]


def test_outlier_activations_select_smoothing():
    # a few activation channels 40x larger than the rest: lambda = 1 leaves
    # them to crush every other channel's 4-bit grid, so some alpha > 0 wins
    s = S.spec("tiny", M=128, K=512, N=256, rank=16)
    d = S.make_layer(s)
    best, pairs, errs = SR.smooth_search(d["W"], d["X"], 16, "int4", grids=4)
    assert pairs[best][0] > 0.0
    assert errs[best] < 0.8 * errs[0]
    assert all(np.isfinite(errs))


def _plain_output_error(x, w, layer):
    """The score written out from its definition: the layer's output on the
    calibration rows (quantized main path plus low-rank branch, no bias),
    rounded to bf16, against X W."""
    from oracle.forward import forward
    y_ref = x @ w
    y = P.round_bf16(forward(x, layer)["y"])
    return float(np.linalg.norm(y - y_ref) / np.linalg.norm(y_ref))


def test_residual_iterations_under_search_score_the_output():
    """AutoRound doc, "Residual iteration": with smooth search on, the
    residual iterations are scored by the calibration output error.  Every
    iterate is scored on its own (brute force over the iteration sequence),
    the kept iteration is the first minimum of those scores, and on this
    layer (16 calibration rows) it is not the iteration the weight error
    would keep, so the reading is observable."""
    s = S.spec("tiny", M=32, K=256, N=128, rank=16, fmt="int4")
    d = S.make_layer(s)
    x = d["X"][:16].astype(np.float64)
    w = d["W"].astype(np.float64)
    amax = P.calib_amax(x)
    lam32, inv = P.smoothing_factors(amax, w, 0.5)
    wt = P.smooth_weight(w, lam32)
    _, weight_err, cands = P.residual_iterations(wt, 16, "int4", iters=8, keep_all=True)
    brute = [_plain_output_error(x, w, P.candidate_layer(c, lam32, inv, "int4", 16)) for c in cands]
    score = SR.candidate_score(x, x @ w)
    lo = P.prepare(w, amax, 0.5, 16, "int4", residual_iters=8, score=score)
    assert lo["iter_errors"] == pytest.approx(brute, rel=1e-12)
    assert lo["best_iter"] == int(np.argmin(brute))
    assert lo["best_iter"] != int(np.argmin(weight_err))
    # the search itself reports that candidate's kept iteration and score
    det = []
    _, pairs, errs = SR.smooth_search(w, x, 16, "int4", grids=2, residual_iters=8, details=det)
    k = pairs.index((0.5, 0.5))
    assert det[k]["best_iter"] == lo["best_iter"]
    assert errs[k] == pytest.approx(min(brute), rel=1e-12)
    # early stop: the scored run cut at its first rise above the best so far
    le = P.prepare(w, amax, 0.5, 16, "int4", residual_iters=8, score=score, early_stop=True)
    stop = next((t for t in range(1, 8) if brute[t] > min(brute[:t])), 7)
    assert le["iter_errors"][:stop + 1] == pytest.approx(brute[:stop + 1], rel=1e-12)
    assert len(le["iter_errors"]) == stop + 1


def test_search_without_residual_iteration_scores_the_prepared_layer():
    s = S.spec("tiny", M=64, K=256, N=128, rank=16, fmt="mxfp4")
    d = S.make_layer(s)
    x = d["X"].astype(np.float64)
    w = d["W"].astype(np.float64)
    _, pairs, errs = SR.smooth_search(w, x, 16, "mxfp4", grids=2)
    amax = P.calib_amax(x)
    for (a, b), e in zip(pairs, errs):
        assert e == pytest.approx(_plain_output_error(x, w, P.prepare(w, amax, a, 16, "mxfp4", beta=b)), rel=1e-12)


def test_reservoir_small_cases():
    assert SR.reservoir_select(5, 8, 1) == [0, 1, 2, 3, 4]      # fewer calls than slots: all kept
    assert SR.reservoir_select(8, 8, 1) == list(range(8))
    assert SR.reservoir_select(0, 4, 1) == [] and SR.reservoir_select(4, 0, 1) == []
    got = SR.reservoir_select(1000, 128, 7)
    assert len(got) == 128 and len(set(got)) == 128 and all(0 <= i < 1000 for i in got)
    assert got == SR.reservoir_select(1000, 128, 7)               # deterministic per seed
    assert got != SR.reservoir_select(1000, 128, 8)


def test_reservoir_inclusion_is_uniform():
    # Algorithm R keeps every call with probability k / n; over many seeds
    # each call's inclusion count is Binomial(trials, k / n)
    n, k, trials = 40, 10, 4000
    counts = np.zeros(n)
    for seed in range(trials):
        for i in SR.reservoir_select(n, k, seed):
            counts[i] += 1
    p = k / n
    sd = np.sqrt(trials * p * (1 - p))
    assert np.all(np.abs(counts - trials * p) < 5 * sd)
    # the late calls are not favoured or starved relative to the early ones
    assert abs(counts[:20].mean() - counts[20:].mean()) < 3 * sd / np.sqrt(20) * np.sqrt(2) + 1


def test_splitmix64_is_a_bijective_mixer_on_small_states():
    # distinct states give distinct outputs (the finaliser is invertible)
    outs = {SR.splitmix64(s)[1] for s in range(5000)}
    assert len(outs) == 5000
    # and the output bits are balanced
    bits = np.array([[(SR.splitmix64(s)[1] >> b) & 1 for b in range(64)] for s in range(2000)])
    assert np.all(np.abs(bits.mean(0) - 0.5) < 0.06)


def test_splitmix64_reproduces_the_published_outputs():
    # tests/golden/splitmix64.json: the generator's first outputs for two
    # seeds as published with its reference implementations
    import json, os
    with open(os.path.join(os.path.dirname(__file__), "golden", "splitmix64.json")) as fh:
        golden = json.load(fh)
    for seed, outs in golden["outputs"].items():
        state = int(seed)
        for want in outs:
            state, got = SR.splitmix64(state)
            assert got == int(want, 0), (seed, hex(got), want)
