"""Pins of the oracle's offline preparation: Eq. (4) special cases, Eq. (3)
invariance, Eckart-Young (Eq. (10)), full-rank exactness, optimality, QKV
grouping and the Eq. (13) LoRA identity (Zhou notes sec. 3, 5, 7; AutoRound
doc processing flow)."""
import numpy as np
import pytest

from oracle import prepare as P
from oracle import forward as F
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
