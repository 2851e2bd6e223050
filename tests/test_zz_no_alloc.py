"""The allocation-free forward (svdq_linear_forward_noalloc, for callers
that cannot allocate device memory) against svdq_linear_forward: the same
kernels, so Y must be bit-identical, on two calls in a row (the second with
a smaller input, which reuses the same per-GPU scratch array), in every
format; and the size limit is enforced before any launch."""
import numpy as np
import pytest

import rank_gemm_svdq_amd as B
from rank_gemm_svdq_amd import synthetic as S
from tests.gpu_util import GpuRun

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fmt", ["int4", "mxfp4", "w8a8"])
def test_noalloc_matches_workspace_forward_twice(fmt):
    import torch
    for M, K, N, rank in [(300, 1024, 400, 32), (70, 640, 272, 48)]:   # second call smaller
        s = S.spec("tiny", M=M, K=K, N=N, rank=rank, fmt=fmt)
        d = S.make_layer(s)
        run = GpuRun(d, fmt, rank, s.alpha).forward()
        y_ref = run.Y.clone()
        Y2 = torch.full_like(run.Y, 0x7FC0)
        B.linear_forward_noalloc(run.layer, run.X, Y2)
        torch.cuda.synchronize()
        assert bool((Y2 == y_ref).all()), f"{fmt} M={M} K={K} N={N} rank={rank}"


def test_noalloc_full_size_and_limit():
    import torch
    s = S.spec("flux_mlp_up")
    d = S.make_layer(s)
    run = GpuRun(d, "mxfp4", s.rank, s.alpha).forward()
    assert B.workspace_bytes(s.M, s.K, s.rank + s.lora_rank, "mxfp4") <= B.NOALLOC_MAX_WORKSPACE
    Y2 = torch.empty_like(run.Y)
    B.linear_forward_noalloc(run.layer, run.X, Y2)
    torch.cuda.synchronize()
    assert bool((Y2 == run.Y).all())
    # a token count whose workspace exceeds the array is rejected, nothing launched
    M = 40000
    assert B.workspace_bytes(M, s.K, s.rank, "mxfp4") > B.NOALLOC_MAX_WORKSPACE
    X = torch.zeros((M, s.K), dtype=torch.int16, device="cuda")
    Y = torch.zeros((M, s.N), dtype=torch.int16, device="cuda")
    with pytest.raises(B.SvdqError) as e:
        B.linear_forward_noalloc(run.layer, X, Y)
    assert e.value.status == 5            # SVDQ_ERR_WORKSPACE
    assert int(Y.abs().max()) == 0
