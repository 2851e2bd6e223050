"""The forward recorded in a HIP graph (torch.cuda.CUDAGraph over HIP
stream capture) and replayed: the workspace forward and the
allocation-free one, each captured once and replayed several times with
other device work and synchronisations between the replays. Every replay's
Y must be bit-identical to the eager forward's on the same input (the same
kernels on the same operands). The forward issues only kernel launches: no
allocation, no memset, no synchronisation."""
import pytest

import rank_gemm_svdq_amd as B
from rank_gemm_svdq_amd import synthetic as S
from tests.gpu_util import GpuRun

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fmt", ["int4", "mxfp4", "w8a8", "mxfp4_ocp"])
@pytest.mark.parametrize("noalloc", [False, True])
def test_graph_replays_match_the_eager_forward(fmt, noalloc):
    import torch
    s = S.spec("tiny", M=300, K=1024, N=400, rank=32, fmt=fmt)
    d = S.make_layer(s)
    run = GpuRun(d, fmt, 32, s.alpha).forward()
    y_ref = run.Y.clone()
    Yg = torch.empty_like(run.Y)
    wsg = run.layer.workspace(run.M)

    def fwd():
        if noalloc:
            B.linear_forward_noalloc(run.layer, run.X, Yg)
        else:
            B.linear_forward(run.layer, run.X, Yg, wsg)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fwd()                      # first calls (device check, scratch lookup) outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert bool((Yg == y_ref).all())

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fwd()
    Y_other = torch.empty_like(run.Y)
    for rep in range(4):
        Yg.fill_(0x7FC0)                                           # eager work between replays
        B.linear_forward(run.layer, run.X, Y_other, run.ws)        # and an eager forward
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert bool((Yg == y_ref).all()), f"{fmt} noalloc={noalloc} replay {rep}"
        assert bool((Y_other == y_ref).all())
    del g
