"""Parity at the largest shapes the device path accepts: M = 2^20 token rows
and M K = 2^32 elements (8 GiB of X, 2-4 GiB of activation codes), where the
byte offsets into X, the codes, the INT4 code tails and Y pass 2^31 and, for
the 8-bit codes, come within a kilobyte group of 2^32.

The kernels run on the oracle's own prepared layer (its lambda, codes,
scales and bf16 factors in the kernel layouts), X is drawn on the device
(synthetic.device_normal_bf16), and sampled rows - at the ends, at tile and
row-group edges and where the offsets cross 2^30, 2^31 and 2^32 - are
copied back; every element of those rows must lie within the element-wise
bound of the oracle's fp64 forward (tests/gpu_util.elementwise_bound).  Each
output row depends on its own X row only, so the oracle's forward of the
sampled rows is their exact reference.  The weight codes (N K below 2^32 by
the same rule) are addressed by the same offset arithmetic as the activation
codes in both GEMM kernels, so the token side stands for both.
"""
import numpy as np
import pytest

import rank_gemm_svdq_amd as B
from rank_gemm_svdq_amd import synthetic as S
from oracle import forward as F
from tests.gpu_util import (assert_elementwise, bf16_to_f64, elementwise_bound, oracle_canonical,
                            oracle_layer)

pytestmark = pytest.mark.gpu

K, N, RANK = 4096, 256, 16
M_MAX = 1 << 20


def _rows(M):
    rng = np.random.default_rng(M)
    edges = [0, 1, 15, 16, 255, 256, (1 << 18) - 1, 1 << 18, (1 << 19) - 1, 1 << 19, (1 << 19) + 1,
             M - 257, M - 256, M - 33, M - 32, M - 17, M - 16, M - 2, M - 1]
    return np.unique(np.concatenate([[e for e in edges if 0 <= e < M], rng.choice(M, 40, replace=False)]))


@pytest.mark.parametrize("fmt,M", [("mxfp4", M_MAX), ("int4", M_MAX), ("w8a8", M_MAX), ("mxfp4_ocp", M_MAX),
                                   ("mxfp4", M_MAX - 3), ("int4", M_MAX - 3)])
def test_largest_layer(fmt, M):
    import torch
    assert M * K <= 1 << 32
    s = S.spec("tiny", M=1024, K=K, N=N, rank=RANK, fmt=fmt)    # weights, bias and calibration rows
    d = S.make_layer(s, with_x=False)
    po = oracle_layer(d, fmt, RANK, s.alpha)
    layer = B.DeviceLayer(oracle_canonical(po), S.bf16_bits_of(d["bias"]))
    X = S.device_normal_bf16(7, M, K)
    Y = torch.empty((M, N), dtype=torch.int16, device="cuda")
    ws = layer.workspace(M)
    print(f"[maxsize] {fmt} M={M} K={K} N={N} rank={RANK}: X {X.numel() * 2 / 2**30:.1f} GiB, "
          f"workspace {ws.numel() / 2**30:.2f} GiB", flush=True)
    B.linear_forward(layer, X, Y, ws)
    torch.cuda.synchronize()
    rows = _rows(M)
    idx = torch.from_numpy(rows).cuda()
    x = bf16_to_f64(X.index_select(0, idx).cpu().numpy()).astype(np.float32)
    y = bf16_to_f64(Y.index_select(0, idx).cpu().numpy())
    del X, Y, ws, layer
    torch.cuda.empty_cache()
    assert np.all(np.isfinite(y))
    ref = F.forward(x, po, d["bias"])["y"]
    assert_elementwise(y, ref, elementwise_bound(x, po, d["bias"]), f"{fmt} M={M}, sampled rows")
