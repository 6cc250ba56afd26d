"""The entry points capture into a HIP graph: they make no host synchronisation
and allocate nothing, so each call becomes one kernel node.  The graph is
replayed several times, with the program's own eager work and
synchronisations in between, and every replay is compared bit for bit with
the eager result."""

import pytest
import torch

import packed_varlen_rotary_amd as P
import workloads as W

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cfg", [1, 2])
def test_graph_replays_match_eager(cfg):
    w = W.make_workload(cfg)
    dev = "cuda"
    cu = torch.as_tensor(w.cu_seqlens, device=dev)
    src = W.make_tensors(w, ("q", "k", "dq", "dk"), device=dev)
    work = {n: t.clone() for n, t in src.items()}

    def step():
        P.rope_qk_fwd(work["q"], work["k"], cu, w.theta)
        P.rope_qk_bwd(work["dq"], work["dk"], cu, w.theta)

    step()  # eager reference
    torch.cuda.synchronize()
    eager = {n: t.clone() for n, t in work.items()}

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for n in work:
            work[n].copy_(src[n])
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for replay in range(4):
        for n in work:  # eager work between replays: restore the inputs
            work[n].copy_(src[n])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n in work:
            assert torch.equal(work[n].view(torch.int16) if work[n].dtype == torch.bfloat16 else work[n],
                               eager[n].view(torch.int16) if eager[n].dtype == torch.bfloat16 else eager[n]), (replay, n)
