"""Pins of the oracle forward: the Eq. (8) error identity, the
no-quantization identity of the msModelSlim doc, a brute-force int64
per-group GEMM, the Eq. (5)/(6) decomposition and bound, and lower error than
plain W4A4 on outlier inputs (Zhou notes sec. 4; msModelSlim doc)."""
import numpy as np
import pytest

from oracle import forward as F
from oracle import prepare as P
from oracle import quantizers as Q
from rank_gemm_svdq_amd import synthetic as S


def _tiny(fmt="int4", **kw):
    s = S.spec("tiny", fmt=fmt, **kw)
    d = S.make_layer(s)
    L = P.prepare(d["W"], P.calib_amax(d["X_cal"]), s.alpha, s.rank, fmt)
    return s, d, L


@pytest.mark.parametrize("fmt", ["int4", "mxfp4", "w8a8"])
def test_eq8_error_identity(fmt):
    s, d, L = _tiny(fmt)
    x = d["X"].astype(np.float64)
    out = F.forward(d["X"], L)
    xh = x * L["inv_lambda"].astype(np.float64)
    r32 = L["r32"].astype(np.float64)
    w_eff = L["l1b"] @ L["l2b"] + r32
    lhs = xh @ w_eff - out["y"]
    a_q = Q.quantize(F.smooth_activations(d["X"], L["inv_lambda"]), fmt)["deq"]
    b_q = Q.quantize(L["r32"].T.copy(), fmt)["deq"]
    rhs = xh @ r32 - a_q @ b_q.T
    assert np.linalg.norm(lhs - rhs) <= 1e-12 * np.linalg.norm(rhs)


def test_no_quantization_identity():
    # x D^-1 R_exact + (x D^-1 L1) L2 = x W  (msModelSlim doc, forward equivalence)
    s, d, L = _tiny()
    x = d["X"].astype(np.float64)
    xd = x / L["lam32"].astype(np.float64)
    got = xd @ L["r_exact"] + (xd @ L["l1"]) @ L["l2"]
    ref = x @ d["W"].astype(np.float64)
    assert np.linalg.norm(got - ref) <= 1e-12 * np.linalg.norm(ref)


def test_gemm_equals_int64_brute_force():
    s, d, L = _tiny()
    out = F.forward(d["X"], L)
    qx = out["xq_codes"].astype(np.int64)
    qw = L["wq_codes"].astype(np.int64)
    M, K = qx.shape
    G = K // 64
    y = np.zeros((M, qw.shape[0]))
    for g in range(G):
        ig = qx[:, 64 * g:64 * g + 64] @ qw[:, 64 * g:64 * g + 64].T   # exact int64
        y += out["xs"][:, g][:, None] * L["ws"][:, g][None, :] * ig
    assert np.linalg.norm(y - out["y_main"]) <= 1e-13 * np.linalg.norm(y)


def test_w8a8_gemm_equals_int64_brute_force():
    # per-token x per-channel scales factor out of the whole K sum
    s, d, L = _tiny("w8a8")
    out = F.forward(d["X"], L)
    qx = out["xq_codes"].astype(np.int64)
    qw = L["wq_codes"].astype(np.int64)
    y = np.empty((qx.shape[0], qw.shape[0]))
    for m in range(qx.shape[0]):
        for n in range(0, qw.shape[0], 64):
            acc = qw[n:n + 64] @ qx[m]                                 # exact int64 dot products
            y[m, n:n + 64] = acc * (float(out["xs"][m]) * L["ws"][n:n + 64].astype(np.float64))
    assert np.linalg.norm(y - out["y_main"]) <= 1e-13 * np.linalg.norm(y)
    # and the 8-bit layer is far closer to X W than the 4-bit one
    L4 = P.prepare(d["W"], P.calib_amax(d["X_cal"]), s.alpha, s.rank, "int4")
    ref = d["X"].astype(np.float64) @ d["W"].astype(np.float64)
    e8 = np.linalg.norm(out["y"] - ref)
    e4 = np.linalg.norm(F.forward(d["X"], L4)["y"] - ref)
    assert e8 < 0.1 * e4


def test_forward_terms_and_bias():
    s, d, L = _tiny()
    out = F.forward(d["X"], L, bias=d["bias"])
    assert np.allclose(out["y"], out["y_main"] + out["z"] @ L["l2p"] + d["bias"][None, :], rtol=0, atol=1e-12)
    z = (d["X"].astype(np.float64) * L["inv_lambda"].astype(np.float64)) @ L["l1b"]
    assert np.allclose(out["z"], z, rtol=1e-14, atol=0)
    # rows are independent (equal up to BLAS summation order)
    sub = F.forward(d["X"][17:40], L, bias=d["bias"])
    assert np.allclose(sub["y"], out["y"][17:40], rtol=1e-13, atol=1e-13)
    assert np.array_equal(sub["xq"], out["xq"][17:40]) and np.array_equal(sub["xs"], out["xs"][17:40])


def test_eq5_decomposition_and_eq6_bound():
    s, d, L = _tiny()
    x = d["X"].astype(np.float64)
    w = d["W"].astype(np.float64)
    qx = Q.quantize(d["X"], "int4")["deq"]
    qw = Q.quantize(d["W"].T.copy(), "int4")["deq"].T
    dx, dw = x - qx, w - qw
    lhs = x @ w - qx @ qw
    assert np.allclose(lhs, x @ dw + dx @ qw, rtol=0, atol=1e-10 * np.abs(lhs).max())
    nf = np.linalg.norm
    assert nf(lhs) <= nf(x) * nf(dw) + nf(dx) * (nf(w) + nf(dw))


def _quality_case(name, **shape):
    s = S.spec(name, **shape)
    d = S.make_layer(s)
    L = P.prepare(d["W"], P.calib_amax(d["X_cal"]), s.alpha, s.rank, s.fmt)
    x = d["X"].astype(np.float64)
    ref = x @ d["W"].astype(np.float64)
    e_svdq = np.linalg.norm(ref - F.forward(d["X"], L)["y"])
    e_rtn = np.linalg.norm(ref - F.plain_w4a4(d["X"], d["W"], s.fmt))
    return e_svdq, e_rtn, np.linalg.norm(ref)


@pytest.mark.parametrize("name,shape", [
    ("tiny", {}),
    ("tiny", {"fmt": "mxfp4"}),
    ("flux_qkv", {"M": 256, "K": 768, "N": 1152}),
    ("flux_mlp_down", {"M": 256, "K": 1536, "N": 384}),
])
# Not pinned here: the Student-t(3) MLP-up workload has no outlier channels
# (its tails are per element), and there the SVDQuant error equals plain RTN
# to within 0.1 %; the direction claim is about channel outliers.
def test_lower_error_than_plain_w4a4_on_outliers(name, shape):
    e_svdq, e_rtn, ref = _quality_case(name, **shape)
    assert e_svdq < e_rtn, (e_svdq / ref, e_rtn / ref)
