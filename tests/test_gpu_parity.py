"""GPU parity of the device path (K-A + K-B through the C ABI) against the
fp64 oracle: activation codes and scales bit-exact, the down projection Z to
fp32 accumulation accuracy, Y within 5e-3 relative Frobenius error (the
tolerance the method's target states)."""
import numpy as np
import pytest

import rank_gemm_svdq_amd as B
from rank_gemm_svdq_amd import synthetic as S
from oracle import forward as F
from oracle import prepare as P
from oracle import quantizers as Q
from tests.gpu_util import (GpuRun, bf16_to_f64, check_elementwise_on_oracle_layer, oracle_layer,
                            oracle_scales_bits, rel_fro)

pytestmark = pytest.mark.gpu
Y_TOL = 5e-3


def _check_full(run, po, x, bias, z_tol=2e-5):
    of = F.forward(x, po, bias)
    assert np.array_equal(run.prep["smooth_inv"], po["inv_lambda"])
    xq, xs, z = run.activations()
    assert np.array_equal(xq, of["xq"]), f"codes differ at {np.argwhere(xq != of['xq'])[:5]}"
    assert np.array_equal(xs, oracle_scales_bits(of["xs"], run.fmt))
    if run.rank:
        # Z itself depends on the sign of each singular vector; Z L2' does not
        zl2 = z.astype(np.float64) @ bf16_to_f64(run.prep["l2"])
        assert rel_fro(zl2, of["z"] @ po["l2p"]) <= z_tol
    err = rel_fro(run.y(), of["y"])
    assert err <= Y_TOL, err
    # kernel-isolated: the same kernels on the oracle's own prepared layer,
    # every element of Y within its bf16 + fp32-accumulation bound
    check_elementwise_on_oracle_layer(po, x, bias, f"{run.fmt} M={run.M} K={run.K} N={run.N} rank={run.rank}")
    return err


@pytest.mark.parametrize("fmt", ["int4", "mxfp4", "w8a8", "mxfp4_ocp"])
@pytest.mark.parametrize("use_bias", [True, False])
def test_tiny_layer(fmt, use_bias):
    s = S.spec("tiny", fmt=fmt)
    d = S.make_layer(s)
    run = GpuRun(d, fmt, s.rank, s.alpha, use_bias=use_bias).forward()
    po = oracle_layer(d, fmt, s.rank, s.alpha)
    _check_full(run, po, d["X"], d["bias"] if use_bias else None)


@pytest.mark.parametrize("fmt", ["int4", "mxfp4", "w8a8"])
@pytest.mark.parametrize("M,K,N,rank", [
    (1, 512, 512, 16), (17, 512, 512, 16), (255, 512, 512, 16),   # ragged token counts
    (300, 1024, 400, 32),                                          # several tiles, ragged N
    (130, 128, 144, 0),                                            # one K step, plain W4A4
    (64, 768, 272, 48),                                            # rank 48 (padded to 64)
    (96, 640, 320, 32), (40, 1152, 272, 64), (33, 384, 160, 16),   # odd numbers of 128-wide K steps
    (70, 640, 384, 96), (257, 512, 400, 128),                      # ranks 96 and 128 (the maximum)
    (50, 512, 160, 80), (70, 384, 144, 112),                       # ranks 80 and 112 (odd 16-column tiles)
    (4200, 256, 160, 48),                                          # more 16-row blocks than compute units
    (4200, 256, 160, 64),                                          # the same at rank 64 (4 fragment tiles in the ring)
    (4200, 16512, 64, 32),                                         # the same with 1/lambda not staged in LDS
    (24, 16384, 64, 16),                                           # K = 16384: 16 steps of 1/lambda staged per wave
    (40, 16512, 64, 16),                                           # K above 16384: 1/lambda not staged in LDS
    (3, 65536, 16, 16),                                            # the largest K with the smallest N
    (20, 128, 262144, 16),                                         # the largest N with the smallest K
])
def test_shapes_and_tails(fmt, M, K, N, rank):
    s = S.spec("tiny", M=M, K=K, N=N, rank=rank, fmt=fmt)
    d = S.make_layer(s)
    run = GpuRun(d, fmt, rank, s.alpha).forward()
    po = oracle_layer(d, fmt, rank, s.alpha)
    _check_full(run, po, d["X"], d["bias"])


@pytest.mark.parametrize("fmt", ["int4", "mxfp4", "w8a8", "mxfp4_ocp"])
def test_lora_rank48(fmt):
    s = S.spec("flux_lora", M=200, K=512, N=640, fmt=fmt)
    d = S.make_layer(s)
    lora = {"A": d["lora_A"], "B": d["lora_B"], "strength": 1.0}
    run = GpuRun(d, fmt, s.rank, s.alpha, lora=lora).forward()
    po = oracle_layer(d, fmt, s.rank, s.alpha, lora=lora)
    _check_full(run, po, d["X"], d["bias"])


@pytest.mark.parametrize("fmt", ["int4", "mxfp4", "w8a8", "mxfp4_ocp"])
def test_quantizer_edge_values(fmt):
    """Zero rows, bf16 subnormals (MXFP4 scale clamped at 2^-127; 8-bit
    scale below 2^-128), huge values (an INT4 scale past the fp16 range,
    saturated at 65504) and exact ties go through K-A; codes and scales
    bit-exact, and Y finite and within its element-wise bound."""
    M, K, N = 48, 512, 64
    x = S.random_bf16(5, (M, K), 2.0)
    x[0] = 0.0
    x[1, :64] = -0.0
    x[2] = S.to_bf16_values(np.full(K, 3e-39))                   # bf16 subnormals
    x[3, :] = S.to_bf16_values(np.linspace(-6, 6, K))
    x[4, :32] = S.to_bf16_values(np.array([7.0, 2.5, -2.5, 0.5, -0.5, 1.5, 3.5, -6.5] * 4))
    x[5] = S.to_bf16_values(S.random_bf16(6, (K,), 1.0) * 1e30)
    x[6, :] = S.to_bf16_values(np.full(K, 1e-36))
    x[7, :32] = 7.0                                                 # OCP rule: a saturated block
    x[7, 32:64] = S.to_bf16_values(np.linspace(-7.9, 7.9, 32))
    d = {"spec": S.spec("tiny"), "X": x, "X_cal": np.abs(x) + 1.0,
         "W": S.random_bf16(7, (K, N), 0.05), "bias": S.random_bf16(8, (N,), 0.1)}
    run = GpuRun(d, fmt, 0, 0.5).forward()
    po = oracle_layer(d, fmt, 0, 0.5)
    of = F.forward(x, po, d["bias"])
    xq, xs, _ = run.activations()
    assert np.array_equal(xq, of["xq"])
    assert np.array_equal(xs, oracle_scales_bits(of["xs"], fmt))
    if fmt == "int4":
        assert np.any(of["xs"] == 65504.0)           # the huge row's groups saturate
    assert np.all(np.isfinite(of["y"])) and np.all(np.isfinite(run.y()))
    check_elementwise_on_oracle_layer(po, x, d["bias"], f"edge values {fmt}")


def test_workspace_reuse_and_determinism():
    s = S.spec("tiny", M=300, K=1024, N=400, rank=32, fmt="mxfp4")
    d = S.make_layer(s)
    run = GpuRun(d, "mxfp4", 32, s.alpha).forward()
    y1 = run.Y.clone()
    run.ws.fill_(0x5A)
    run.forward()
    assert bool((run.Y == y1).all())


def _rows_past_one_block_per_cu():
    # more 16-row K-A blocks than compute units (ragged last block): K-A runs
    # its ring-free variant, two blocks per unit
    import torch
    return 16 * torch.cuda.get_device_properties(0).multi_processor_count + 17


@pytest.mark.parametrize("fmt", ["int4", "mxfp4", "mxfp4_ocp"])
@pytest.mark.parametrize("rank", [16, 32, 48])
def test_more_ka_blocks_than_compute_units(fmt, rank):
    M = _rows_past_one_block_per_cu()
    s = S.spec("tiny", M=M, K=512, N=256, rank=rank, fmt=fmt)
    d = S.make_layer(s)
    run = GpuRun(d, fmt, rank, s.alpha).forward()
    po = oracle_layer(d, fmt, rank, s.alpha)
    _check_full(run, po, d["X"], d["bias"])


@pytest.mark.parametrize("fmt", ["int4", "mxfp4"])
def test_more_ka_blocks_than_compute_units_unfused(fmt):
    """The unfused baseline's separate down-projection pass at the same
    token count."""
    import torch
    M = _rows_past_one_block_per_cu()
    s = S.spec("tiny", M=M, K=384, N=144, rank=32, fmt=fmt)
    d = S.make_layer(s)
    run = GpuRun(d, fmt, 32, s.alpha).forward()
    y_fused = run.y()
    B.linear_forward_unfused(run.layer, run.X, run.Y, run.ws)
    torch.cuda.synchronize()
    po = oracle_layer(d, fmt, 32, s.alpha)
    of = F.forward(d["X"], po, d["bias"])
    assert rel_fro(run.y(), of["y"]) <= Y_TOL
    assert rel_fro(run.y(), y_fused) <= 4e-3


def _n_with_partial_round(M):
    """An N whose 256 x 256 tiles leave a last round at most a quarter full,
    so that K-B runs the last 256-wide columns as 128 x 128 tiles."""
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    tm = (M + 255) // 256
    tn = 2 * cus // tm + max(1, cus // (4 * tm))
    assert 0 < (tm * tn) % cus <= cus // 4
    return 256 * tn


@pytest.mark.parametrize("fmt,M,K,rank", [
    ("mxfp4", 4096, 256, 32), ("mxfp4", 4000, 384, 48),     # ragged token count, odd step count
    ("mxfp4", 4096, 256, 0), ("mxfp4_ocp", 4096, 256, 32), ("w8a8", 4096, 256, 16),
])
def test_partial_last_round_runs_as_small_tiles(fmt, M, K, rank):
    N = _n_with_partial_round(M)
    s = S.spec("tiny", M=M, K=K, N=N, rank=rank, fmt=fmt)
    d = S.make_layer(s)
    run = GpuRun(d, fmt, rank, s.alpha).forward()
    po = oracle_layer(d, fmt, rank, s.alpha)
    _check_full(run, po, d["X"], d["bias"])


@pytest.mark.parametrize("fmt", ["int4", "mxfp4", "w8a8", "mxfp4_ocp"])
@pytest.mark.parametrize("M,K,N,rank", [(300, 1024, 400, 32), (17, 512, 272, 48), (130, 640, 144, 0)])
def test_unfused_baseline(fmt, M, K, N, rank):
    """The four-kernel baseline computes the same layer: within the
    tolerance of the oracle, and close to the fused output (it rounds Y to
    bf16 once more, before the low-rank add)."""
    import torch
    s = S.spec("tiny", M=M, K=K, N=N, rank=rank, fmt=fmt)
    d = S.make_layer(s)
    run = GpuRun(d, fmt, rank, s.alpha).forward()
    y_fused = run.y()
    B.linear_forward_unfused(run.layer, run.X, run.Y, run.ws)
    torch.cuda.synchronize()
    y_unf = run.y()
    po = oracle_layer(d, fmt, rank, s.alpha)
    of = F.forward(d["X"], po, d["bias"])
    assert rel_fro(y_unf, of["y"]) <= Y_TOL
    assert rel_fro(y_unf, y_fused) <= 4e-3
    xq, xs, _ = run.activations()
    assert np.array_equal(xq, of["xq"])


@pytest.mark.parametrize("fmt", ["int4", "mxfp4", "w8a8"])
def test_residual_iterated_layer(fmt):
    """A layer prepared with residual iteration (refits to W~ - Q(R_prev),
    the best of 6 kept) runs through the same device path: codes bit-exact,
    Y within tolerance of the oracle's forward of its own iterated layer."""
    s = S.spec("tiny", M=200, K=512, N=384, rank=32, fmt=fmt)
    d = S.make_layer(s)
    run = GpuRun(d, fmt, s.rank, s.alpha, residual_iters=6).forward()
    po = oracle_layer(d, fmt, s.rank, s.alpha, residual_iters=6)
    assert run.prep["best_iter"] == po["best_iter"]
    np.testing.assert_allclose(run.prep["iter_errors"], po["iter_errors"], rtol=1e-9)
    _check_full(run, po, d["X"], d["bias"])
