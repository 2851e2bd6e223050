"""GPU parity of the smooth-factor grid search (AutoRound doc, "Smooth
search") against the oracle's search on the same calibration rows.

The library scores a candidate with the device forward, the oracle with its
fp64 forward.  By the triangle inequality a candidate's two scores differ by
at most ||Y_dev - Y_oracle||_F / ||X W||_F, which the forward parity bounds
by its 5e-3 tolerance (scaled by ||Y|| / ||X W||, about 1 here), so every
score must agree within that bound, and the library's winner must score,
under the oracle, within twice the bound of the oracle's winner."""
import numpy as np
import pytest

import rank_gemm_svdq_amd as B
from rank_gemm_svdq_amd import synthetic as S
from oracle import search as SR

pytestmark = pytest.mark.gpu
TOL = 5e-3


def _xdev(x):
    import torch
    return torch.from_numpy(S.bf16_bits_of(x).view(np.int16)).cuda()


def _search(w, x, rank, fmt, grids):
    r = B.smooth_search(w, _xdev(x), rank, fmt, grids=grids)
    ob, pairs, oerr = SR.smooth_search(w, x, rank, fmt, grids=grids)
    assert B.smooth_candidates(grids) == pairs
    assert np.all(np.abs(r["errors"] - np.asarray(oerr)) <= TOL), (r["errors"], oerr)
    assert oerr[r["best"]] <= oerr[ob] + 2 * TOL
    assert (r["alpha"], r["beta"]) == pairs[r["best"]]
    # the returned layer is the winner prepared by svdq_prepare
    amax = B.calib_absmax(S.bf16_bits_of(x))
    p = B.prepare(w, amax, r["alpha"], rank, fmt, beta=r["beta"])
    for k in ("lambda", "smooth_inv", "wq", "ws", "l1", "l2"):
        assert np.array_equal(r["prepared"][k], p[k]), k
    return r, ob, oerr


@pytest.mark.parametrize("fmt", ["int4", "mxfp4", "w8a8"])
def test_search_small_grid(fmt):
    s = S.spec("tiny", M=128, K=512, N=256, rank=16, fmt=fmt)
    d = S.make_layer(s)
    r, ob, _ = _search(d["W"], d["X"], 16, fmt, 4)
    assert r["alpha"] > 0.0          # the outlier channels make smoothing win


def test_search_default_grid_39_candidates():
    s = S.spec("tiny", M=96, K=384, N=256, rank=16, fmt="int4")
    d = S.make_layer(s)
    r, _, _ = _search(d["W"], d["X"], 16, "int4", 20)
    assert len(r["errors"]) == 39 and np.isfinite(r["errors"]).all()


def test_search_exact_layer_keeps_unsmoothed():
    # exact INT4-grid operands (see the oracle pin): only (0, 0) is lossless
    rng = np.random.default_rng(3)
    M, K, N = 64, 256, 128
    cx, cw = rng.integers(1, 8, K), rng.integers(1, 8, K)
    x = np.round(rng.uniform(-1, 1, (M, K)) * cx)
    x[:, ::64] = 7.0
    w = np.round(rng.uniform(-1, 1, (K, N)) * cw[:, None]) / 64.0
    w[::64, :] = 7.0 / 64.0
    r, ob, oerr = _search(w.astype(np.float32), x, 0, "int4", 4)
    assert r["best"] == ob == 0
    assert r["errors"][0] == pytest.approx(oerr[0], rel=1e-9)


@pytest.mark.parametrize("fmt,rows,rank", [("int4", 2, 32), ("w8a8", 4, 16)])
def test_search_scores_residual_iterations_by_output(fmt, rows, rank):
    """AutoRound doc, "Residual iteration": with smooth search on, each
    residual iteration is scored by the calibration output error.  The
    library's search is checked against the oracle's search (every
    candidate's score within the forward tolerance) and against its own
    parts composed independently: the winner's iterate t is what
    svdq_prepare returns with t + 1 iterations when the weight error falls
    at every iteration, each iterate runs through the device forward on the
    calibration rows, and the kept iteration must be the first minimum of
    those output errors, with the winner's score equal to that minimum."""
    import torch
    T = 8
    s = S.spec("tiny", M=64, K=256, N=128, rank=rank, fmt=fmt)
    d = S.make_layer(s)
    x = d["X"][:rows]
    w = d["W"]
    r = B.smooth_search(w, _xdev(x), rank, fmt, grids=2, residual_iters=T)
    det = []
    ob, pairs, oerr = SR.smooth_search(w, x, rank, fmt, grids=2, residual_iters=T, details=det)
    assert np.all(np.abs(r["errors"] - np.asarray(oerr)) <= TOL), (r["errors"], oerr)
    assert 0 <= r["best_iter"] < T
    alpha, beta = pairs[r["best"]]
    amax = B.calib_absmax(S.bf16_bits_of(x))
    xd = _xdev(x)
    y_ref = x.astype(np.float64) @ w.astype(np.float64)
    scores = []
    for t in range(T):
        p = B.prepare(w, amax, alpha, rank, fmt, beta=beta, residual_iters=t + 1)
        assert t == 0 or p["iter_errors"][t] < p["iter_errors"][t - 1]   # so p holds iterate t
        assert p["best_iter"] == t
        lay = B.DeviceLayer(p)
        Y = torch.empty((rows, s.N), dtype=torch.int16, device="cuda")
        B.linear_forward(lay, xd, Y, lay.workspace(rows))
        torch.cuda.synchronize()
        y = (Y.cpu().numpy().view(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        scores.append(np.linalg.norm(y - y_ref) / np.linalg.norm(y_ref))
        if t == r["best_iter"]:
            for k in ("lambda", "smooth_inv", "wq", "ws", "l1", "l2"):
                assert np.array_equal(r["prepared"][k], p[k]), k
    assert r["best_iter"] == int(np.argmin(scores)), (r["best_iter"], scores)
    # the device reference X W is fp32, the one here fp64
    assert r["errors"][r["best"]] == pytest.approx(min(scores), rel=1e-5)
    # against the oracle's kept iteration where the oracle's own scores of
    # that candidate separate it from every other iteration by 1 %
    it = np.asarray(det[r["best"]]["iter_scores"])
    k = det[r["best"]]["best_iter"]
    if np.all(np.delete(it, k) > it[k] * 1.01):
        assert r["best_iter"] == k
