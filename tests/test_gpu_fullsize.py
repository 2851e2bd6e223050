"""Parity of the device path at the full FLUX-shaped layer sizes, through the
same entry point and launch configuration the benchmark times.

The oracle cannot run the whole layer in seconds, so it checks sampled token
rows: every row's quantisation and output depend on that row alone, so the
oracle's forward on the sampled rows is the exact reference for them.  The
oracle prepares the weights with its own LAPACK SVD; the device layer uses
the library's preparation, so Y is compared within the 5e-3 relative
Frobenius tolerance while the activation codes and scales (which do not
depend on the SVD) must match bit for bit.

Every row is then checked through a property that holds at any size: Y is
the bf16 rounding of the exact product of the decoded 4-bit operands the
device wrote (codes decoded by the oracle's decoders, multiplied in fp32 on
the GPU by torch) plus Z L2' plus bias, so every element lies within half a
bf16 ulp plus the fp32 accumulation slack of that reference.

Kernel-isolated parity: the same kernels then run on the oracle's own
prepared layer (its lambda, bf16 factors, codes and scales, laid out by the
library's kernel-layout conversion), and every element of the sampled rows
must lie within the element-wise bound of the oracle's fp64 forward of those
rows (tests/gpu_util.elementwise_bound: half a bf16 ulp plus the fp32
accumulation slack of the main and low-rank sums).
"""
import numpy as np
import pytest

from rank_gemm_svdq_amd import synthetic as S
from oracle import forward as F
from oracle import quantizers as Q
from tests.gpu_util import (GpuRun, assert_elementwise, bf16_to_f64, elementwise_bound, oracle_layer,
                            oracle_scales_bits, rel_fro, run_on_oracle_layer)

pytestmark = pytest.mark.gpu
Y_TOL = 5e-3


def _rows(M, seed=0):
    rng = np.random.default_rng(seed)
    edges = [0, 1, 255, 256, M - 257, M - 256, M - 1]          # both sides of 256-row tile edges
    return np.unique(np.concatenate([[e for e in edges if 0 <= e < M], rng.choice(M, 57, replace=False)]))


def _check(name, fmt, alpha=None, lora=False):
    s = S.spec(name, fmt=fmt) if alpha is None else S.spec(name, fmt=fmt, alpha=alpha)
    d = S.make_layer(s)
    lo = {"A": d["lora_A"], "B": d["lora_B"], "strength": 1.0} if lora else None
    run = GpuRun(d, fmt, s.rank, s.alpha, lora=lo).forward()
    po = oracle_layer(d, fmt, s.rank, s.alpha, lora=lo)
    assert np.array_equal(run.prep["smooth_inv"], po["inv_lambda"])
    rows = _rows(s.M)
    of = F.forward(d["X"][rows], po, d["bias"])
    xq, xs, z = run.activations()
    assert np.array_equal(xq[rows], of["xq"]), f"{name}/{fmt}: activation codes differ"
    assert np.array_equal(xs[rows], oracle_scales_bits(of["xs"], fmt)), f"{name}/{fmt}: activation scales differ"
    zl2 = z[rows].astype(np.float64) @ bf16_to_f64(run.prep["l2"])
    assert rel_fro(zl2, of["z"] @ po["l2p"]) <= 1e-4
    err = rel_fro(run.y(rows), of["y"])
    assert err <= Y_TOL, f"{name}/{fmt}: rel_fro {err:.3e}"
    # all rows: decoded operands, fp32 product on the GPU, against Y
    import torch
    sc = lambda v: v.view(np.float16).astype(np.float64) if fmt == "int4" else v   # E8M0 bytes / fp32 as is
    xd = torch.from_numpy(Q.dequantize_packed(xq, sc(xs), fmt).astype(np.float32)).cuda()
    wd = torch.from_numpy(Q.dequantize_packed(run.prep["wq"], sc(run.prep["ws"]), fmt).astype(np.float32)).cuda()
    l2 = torch.from_numpy(bf16_to_f64(run.prep["l2"]).astype(np.float32)).cuda()
    zt = torch.from_numpy(z.astype(np.float32)).cuda()
    bias = torch.from_numpy(np.asarray(d["bias"], np.float32)).cuda()
    prev = torch.backends.cuda.matmul.allow_tf32
    torch.backends.cuda.matmul.allow_tf32 = False
    try:
        ref = xd @ wd.T + zt @ l2 + bias
        # the reference's own fp32 sums carry the same slack as the device's
        e = (2 * (s.K / 32 + 16) * 2.0**-24) * (xd.abs() @ wd.abs().T) + 2.0**-15 * (zt.abs() @ l2.abs())
        e += 8 * 2.0**-24 * ref.abs()
    finally:
        torch.backends.cuda.matmul.allow_tf32 = prev
    ydev = (run.Y.to(torch.int32) << 16).view(torch.float32)
    assert bool(torch.isfinite(ydev).all())
    full_err = float(torch.linalg.norm(ydev - ref) / torch.linalg.norm(ref))
    assert full_err <= 2.5e-3, f"{name}/{fmt}: all-row rel_fro {full_err:.3e} against the decoded-operand product"
    bound = 2.0**-8 * (ref.abs() + e) + e
    over = (ydev - ref).abs() > bound
    n_over = int(over.sum())
    assert n_over == 0, f"{name}/{fmt}: {n_over} elements outside the element-wise bound (first {over.nonzero()[:4].tolist()})"
    del xd, wd, ref, e, bound, over, ydev
    # kernel-isolated: the oracle's own layer through the same kernels
    y_iso = run_on_oracle_layer(po, d["X"], d["bias"])
    assert_elementwise(y_iso[rows], of["y"], elementwise_bound(d["X"][rows], po, d["bias"]),
                       f"{name}/{fmt} oracle layer, sampled rows")
    return err


def test_flux_qkv_int4():
    _check("flux_qkv", "int4")


def test_flux_mlp_up_mxfp4():
    _check("flux_mlp_up", "mxfp4")


def test_flux_mlp_up_mxfp4_ocp_rule():
    # the OCP shared-exponent rule (saturating) on the same layer
    _check("flux_mlp_up", "mxfp4_ocp")


@pytest.mark.parametrize("alpha", [0.3, 0.5, 0.7])
def test_flux_mlp_down_int4_alpha(alpha):
    _check("flux_mlp_down", "int4", alpha=alpha)


def test_flux_qkv_w8a8():
    # the 8-bit setting: rank 16, per-token activations, per-channel weights
    _check("flux_qkv_w8a8", "w8a8")


@pytest.mark.parametrize("fmt", ["mxfp4", "int4"])
def test_flux_lora_two_image_batch(fmt):
    _check("flux_lora", fmt, lora=True)
