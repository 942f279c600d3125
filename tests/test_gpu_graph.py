"""The layer forward captured in a HIP graph (torch.cuda.CUDAGraph over the
C-ABI calls on the capturing stream) and replayed: every replay equals the
eager forward bit for bit, with eager work and synchronisations between the
replays, and a new input copied into the captured buffer is routed afresh.

The eager forward itself is checked against the dense-masked oracle by the
forward tests; here the replays are checked against it.  Graph capture needs
calls that record no host synchronisation and no memset node: the library
clears memory with fill kernels and its workspaces are allocated by the
caller before capture.
"""
import pytest
import torch

from workloads import Workload, make_inputs

from gpu_helpers import make_layer, need_gpu, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T", [16, 300])
def test_forward_graph_replays_match_eager(T):
    need_gpu()
    # T = 16: the split router, streaming expert GEMMs and the split shared
    # down projection; T = 300: the tile GEMMs
    w = Workload("graph", T=T, H=1024, E=16, k=4, I=128, Is=512, score=0, renorm=False, shared_gated=True,
                 seed=21)
    inp = make_inputs(w, device="cuda")
    layer = make_layer(w, inp)
    x = inp["x"].clone()
    eager = layer.forward(x).clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer.forward(x)   # warm-up on the capture side stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = layer.forward(x)
    other_x = make_inputs(w.with_(seed=22), device="cuda")["x"]
    for i in range(4):
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i}"
        other = layer.forward(other_x)   # eager work between the replays
        torch.cuda.synchronize()
    x.copy_(other_x)
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(out, other)
    assert not torch.equal(out, eager)
    say(f"T={T}: 5 replays equal the eager forward")
