"""Pins of the oracle's offline preparation: Eq. (4) special cases, Eq. (3)
invariance, Eckart-Young (Eq. (10)), full-rank exactness, optimality, QKV
grouping, the Eq. (13) LoRA identity (Zhou notes sec. 3, 5, 7; AutoRound
doc processing flow), and residual iteration (AutoRound doc, "Residual
iteration": each refit is the top-r part of W~ - Q(R_prev), checked through
an eigen-decomposition; rank 0 reduces to plain RTN; early stop cuts the full
sequence at its first rise)."""
import numpy as np
import pytest

from oracle import prepare as P
from oracle import forward as F
from oracle import quantizers as Q
from oracle.rounding import round_bf16
from rank_gemm_svdq_amd import synthetic as S


def test_smoothing_factor_special_cases():
    w = np.array([[1.0, -0.5], [2.0, 0.25], [0.0, 0.0], [0.5, -0.125]])
    ax = np.array([4.0, 0.0, 9.0, 8.0], dtype=np.float32)
    lam, inv = P.smoothing_factors(ax, w, 0.5)
    # sqrt(4)/sqrt(1) = 2; zero activation stat -> 1; zero weight row -> 1;
    # sqrt(8)/sqrt(0.5) = 4
    assert list(lam) == [2.0, 1.0, 1.0, 4.0]
    assert list(inv) == [0.5, 1.0, 1.0, 0.25]
    lam0, _ = P.smoothing_factors(ax, w, 0.0)      # alpha 0: 1 / amaxW
    assert lam0[0] == 1.0 and lam0[3] == 2.0
    lam1, _ = P.smoothing_factors(ax, w, 1.0)      # alpha 1: amaxX
    assert lam1[0] == 4.0 and lam1[3] == 8.0


def test_smoothing_invariance_eq3():
    rng = np.random.default_rng(0)
    x = S.to_bf16_values(rng.standard_normal((64, 96)))
    w = S.to_bf16_values(rng.standard_normal((96, 80)))
    # power-of-two lambda: both scalings are exact, so the products agree bit for bit
    lam = np.ldexp(1.0, rng.integers(-6, 7, 96)).astype(np.float32)
    inv = (np.float32(1) / lam).astype(np.float32)
    xh = F.smooth_activations(x, inv).astype(np.float64)
    wt = P.smooth_weight(w, lam)
    assert np.array_equal(xh @ wt, x.astype(np.float64) @ w.astype(np.float64))
    # general lambda: X D^-1 (fp64) times D W equals X W to rounding
    lam, inv = P.smoothing_factors(np.abs(x).max(0) + 1, w, 0.5)
    xd = x.astype(np.float64) / lam.astype(np.float64)
    ref = x.astype(np.float64) @ w.astype(np.float64)
    got = xd @ P.smooth_weight(w, lam)
    assert np.linalg.norm(got - ref) <= 1e-13 * np.linalg.norm(ref)


def _layer(seed, K, N, rank, fmt="int4", alpha=0.5, outliers=4):
    rng = np.random.default_rng(seed)
    w = S.to_bf16_values(rng.standard_normal((K, N)) / np.sqrt(K))
    xc = rng.standard_normal((128, K))
    xc[:, rng.choice(K, outliers, replace=False)] *= 40
    ax = P.calib_amax(S.to_bf16_values(xc))
    return w, ax, P.prepare(w, ax, alpha, rank, fmt)


def test_eckart_young_tail_energy():
    _, _, L = _layer(1, 192, 256, 16)
    r2 = np.sum(L["r_exact"] ** 2)
    tail = np.sum(L["sigma"][16:] ** 2)
    assert abs(r2 - tail) <= 1e-10 * tail
    assert abs(np.sum(L["w_tilde"] ** 2) - np.sum(L["sigma"][:16] ** 2) - r2) <= 1e-10 * np.sum(L["w_tilde"] ** 2)


def test_full_rank_residual_vanishes():
    _, _, L = _layer(2, 64, 96, 64)
    assert np.linalg.norm(L["r_exact"]) <= 1e-12 * np.linalg.norm(L["w_tilde"])


def test_truncation_is_optimal_against_random_rank_r():
    _, _, L = _layer(3, 128, 160, 8)
    best = np.linalg.norm(L["r_exact"])
    rng = np.random.default_rng(4)
    wt = L["w_tilde"]
    for _ in range(20):
        q, _ = np.linalg.qr(rng.standard_normal((128, 8)))
        assert np.linalg.norm(wt - q @ (q.T @ wt)) >= best
    # also against a perturbation of the optimal subspace
    u = L["l1"] / np.linalg.norm(L["l1"], axis=0)
    q, _ = np.linalg.qr(u + 1e-3 * rng.standard_normal(u.shape))
    assert np.linalg.norm(wt - q @ (q.T @ wt)) >= best


def test_bf16_factors_and_residual_reassemble_w_tilde():
    _, _, L = _layer(5, 128, 192, 16)
    assert np.array_equal(L["l1b"], round_bf16(L["l1"]))
    assert np.array_equal(L["l2b"], round_bf16(L["l2"]))
    recon = L["l1b"] @ L["l2b"] + L["r"]
    assert np.allclose(recon, L["w_tilde"], rtol=0, atol=1e-15 * np.abs(L["w_tilde"]).max())
    # the residual absorbs the bf16 factor error: it differs from r_exact
    assert not np.array_equal(L["r"], L["r_exact"])
    assert np.linalg.norm(L["r"] - L["r_exact"]) < 1e-2 * np.linalg.norm(L["r_exact"])


def test_smoothing_moves_outliers_to_low_rank():
    # with the outlier channels migrated, the top singular directions carry
    # the scaled rows and the residual's group maxima shrink
    w, ax, L = _layer(6, 256, 256, 16, outliers=4)
    assert L["sigma"][0] > 3 * L["sigma"][20]
    assert np.abs(L["r_exact"]).max() < np.abs(L["w_tilde"]).max()


def test_qkv_grouping_shares_lambda_and_down_factor():
    rng = np.random.default_rng(7)
    K = 128
    ws = [S.to_bf16_values(rng.standard_normal((K, 96)) / np.sqrt(K)) for _ in range(3)]
    ws[1][5, :] *= 10          # row 5's maximum lives in Wk
    ax = np.abs(rng.standard_normal(K)).astype(np.float32) + 0.5
    L = P.prepare_grouped(ws, ax, 0.5, 16, "int4")
    assert L["splits"] == [(0, 96), (96, 192), (192, 288)]
    amax_w = np.maximum.reduce([np.abs(x).max(1) for x in ws])
    lam_ref, _ = P.smoothing_factors(ax, amax_w[:, None], 0.5)
    assert np.array_equal(L["lam32"], lam_ref)
    assert L["l1b"].shape == (K, 16) and L["l2b"].shape == (16, 288)
    # Eckart-Young on the concatenated smoothed weight
    assert abs(np.sum(L["r_exact"] ** 2) - np.sum(L["sigma"][16:] ** 2)) <= 1e-10 * np.sum(L["sigma"] ** 2)
    # the separate up factors are column blocks of one L2: each block of Y
    # equals the forward through that block alone
    x = S.to_bf16_values(rng.standard_normal((32, K)))
    y = F.forward(x, L)["y"]
    for (a, b) in L["splits"]:
        sub = dict(L, l2p=L["l2p"][:, a:b], wq_packed=L["wq_packed"][a:b], ws=L["ws"][a:b])
        assert np.allclose(F.forward(x, sub)["y"], y[:, a:b], rtol=1e-13, atol=1e-13)


def test_lora_attach_eq13():
    rng = np.random.default_rng(8)
    K, N, k = 128, 160, 16
    w, ax, L = _layer(9, K, N, 16)
    a = S.to_bf16_values(rng.standard_normal((K, k)) / np.sqrt(K))
    b = S.to_bf16_values(rng.standard_normal((k, N)) * 0.1)
    La = P.prepare(w, ax, 0.5, 16, "int4", lora={"A": a, "B": b, "strength": 0.75})
    assert np.array_equal(La["wq_packed"], L["wq_packed"]) and np.array_equal(La["ws"], L["ws"])
    assert La["l1p"].shape == (K, 32) and La["l2p"].shape == (32, N)
    x = S.to_bf16_values(rng.standard_normal((64, K)))
    dy = F.forward(x, La)["y"] - F.forward(x, L)["y"]
    want = x.astype(np.float64) @ a @ (0.75 * b)
    # equal up to the bf16 rounding of D A and s B
    assert np.linalg.norm(dy - want) <= 5e-3 * np.linalg.norm(want)
    # dropping D (using A instead of D A) would be far off when lambda != 1
    wrong = x.astype(np.float64) @ (a / La["lam32"][:, None].astype(np.float64)) @ (0.75 * b)
    assert np.linalg.norm(dy - wrong) > 0.1 * np.linalg.norm(want)


def test_calib_amax():
    x = np.array([[1.0, -3.0], [-2.0, 0.5]])
    assert list(P.calib_amax(x)) == [2.0, 3.0]


# ---------------------------------------------------------------- residual iteration
# AutoRound doc, "Residual iteration": every outer iteration after the first
# refits the rank-r branch to W~ - Q(R_prev) and re-quantizes the new
# residual; the best candidate by weight reconstruction error is kept.

def _ri_layer(seed, K=128, N=64, scale=1.0):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((K, N)) * scale).astype(np.float32)
    ax = (np.abs(rng.standard_normal(K)) + 0.1).astype(np.float32)
    return w, ax


def _top_r_projection(a, r):
    """Best rank-r approximation of a through the eigenvectors of a^T a
    (a different route from the SVD the oracle takes)."""
    ev, vec = np.linalg.eigh(a.T @ a)
    v = vec[:, np.argsort(ev)[::-1][:r]]
    return a @ v @ v.T


@pytest.mark.parametrize("fmt", ["int4", "mxfp4"])
def test_residual_iteration_targets_and_errors(fmt):
    w, ax = _ri_layer(11)
    lam, _ = P.smoothing_factors(ax, w, 0.5)
    wt = P.smooth_weight(w, lam)
    best, errors, cands = P.residual_iterations(wt, 16, fmt, iters=4, keep_all=True)
    assert len(errors) == len(cands) == 4
    prev_deq = None
    for t, c in enumerate(cands):
        # the fit of iteration t is the top-r part of W~ (t = 0) or of W~ - Q(R_{t-1})
        target = wt if t == 0 else wt - prev_deq
        ref = _top_r_projection(target, 16)
        assert np.linalg.norm(c["l1"] @ c["l2"] - ref) <= 1e-9 * np.linalg.norm(ref)
        # residual and its quantization, decoded from the packed codes
        np.testing.assert_array_equal(c["r"], wt - c["l1b"] @ c["l2b"])
        sc = c["q"]["scales"]
        deq_t = Q.dequantize_packed(c["q"]["packed"], sc, fmt).T
        # error: explicit sum of squares over the columns
        e2 = sum(float(np.dot(col, col)) for col in (wt - c["l1b"] @ c["l2b"] - deq_t).T)
        assert abs(errors[t] - np.sqrt(e2)) <= 1e-12 * errors[t]
        prev_deq = deq_t
    assert best["err"] == min(errors) and best["iteration"] == int(np.argmin(errors))


def test_residual_iteration_rank0_is_plain_rtn():
    # with no branch every iteration leaves R = W~, so all errors are ||W~ - Q(W~)||
    w, ax = _ri_layer(3)
    lam, _ = P.smoothing_factors(ax, w, 0.5)
    wt = P.smooth_weight(w, lam)
    best, errors, _ = P.residual_iterations(wt, 0, "int4", iters=3, early_stop=True)
    rtn = np.linalg.norm(wt - Q.quantize(P.to_f32(wt).T.copy(), "int4")["deq"].T)
    assert errors == [errors[0]] * 3 and abs(errors[0] - rtn) <= 1e-12 * rtn
    assert best["iteration"] == 0


def test_residual_iteration_early_stop_is_prefix_of_full_run():
    # a layer whose error sequence rises at iteration 5 and later falls below
    # its earlier best: early stop must cut the full sequence right there
    w, ax = _ri_layer(0)
    lam, _ = P.smoothing_factors(ax, w, 0.5)
    wt = P.smooth_weight(w, lam)
    _, full, _ = P.residual_iterations(wt, 48, "mxfp4", iters=10)
    best_es, es, _ = P.residual_iterations(wt, 48, "mxfp4", iters=10, early_stop=True)
    rise = next(t for t in range(1, len(full)) if full[t] > min(full[:t]))
    assert es == full[:rise + 1]
    assert best_es["err"] == min(full[:rise + 1]) > min(full)


def test_residual_iteration_reduces_error_on_outlier_layer():
    # the point of iterating: the kept error is below the one-shot split
    w, ax, L1 = _layer(2, 256, 192, 16)
    L = P.prepare(w, ax, 0.5, 16, "int4", residual_iters=6)
    assert L["iter_errors"][0] == pytest.approx(np.linalg.norm(L1["r"] - L1["w_deq"].T), rel=1e-12)
    assert min(L["iter_errors"]) < 0.97 * L["iter_errors"][0]
    assert L["best_iter"] > 0


def test_beta_weight_exponent():
    # Smooth search candidates: (alpha, 0) gives lambda = amaxX^alpha, and
    # beta = 1 - alpha is Eq. (4)
    rng = np.random.default_rng(0)
    w = rng.standard_normal((8, 5))
    ax = np.abs(rng.standard_normal(8)) + 0.5
    lam0, _ = P.smoothing_factors(ax, w, 0.3, beta=0.0)
    np.testing.assert_array_equal(lam0, np.float32(ax ** 0.3))
    a, _ = P.smoothing_factors(ax, w, 0.3, beta=0.7)
    b, _ = P.smoothing_factors(ax, w, 0.3)
    np.testing.assert_array_equal(a, b)
    lam00, _ = P.smoothing_factors(ax, w, 0.0, beta=0.0)
    np.testing.assert_array_equal(lam00, np.ones(8, np.float32))
