"""The layer forward captured in a HIP graph (torch.cuda.CUDAGraph over the
C-ABI calls on the capturing stream) and replayed: every replay equals the
eager forward bit for bit, with eager work and synchronisations between the
replays, and a new input copied into the captured buffer is routed afresh.

The eager forward itself is checked against the dense-masked oracle by the
forward tests; here the replays are checked against it.  Graph capture needs
calls that record no host synchronisation and no memset node: the library
clears memory with fill kernels and its workspaces are allocated by the
caller before capture.  A second test runs decode-sized forwards from two
host threads on two streams at once (the library's per-device side stream is
shared between them) and checks every result against its serial forward.
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


def test_concurrent_decode_forwards_on_two_streams():
    """Two host threads run decode-sized forwards (whose shared expert goes
    through the library's side stream) on two streams at once: each result
    equals its serial forward bit for bit."""
    import threading
    need_gpu()
    w = Workload("two_streams", T=16, H=1024, E=16, k=4, I=128, Is=512, score=0, renorm=False,
                 shared_gated=True, seed=23)
    inps = [make_inputs(w.with_(seed=23 + i), device="cuda") for i in range(2)]
    layers = [make_layer(w, inp) for inp in inps]
    serial = [layer.forward(inp["x"]).clone() for layer, inp in zip(layers, inps)]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(2)]
    outs = [[None] * 20, [None] * 20]
    errors = []

    def run(i):
        try:
            with torch.cuda.stream(streams[i]):
                for r in range(20):
                    outs[i][r] = layers[i].forward(inps[i]["x"])
            streams[i].synchronize()
        except Exception as e:  # pragma: no cover - reported below
            errors.append(e)

    threads = [threading.Thread(target=run, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    torch.cuda.synchronize()
    for i in range(2):
        for r in range(20):
            assert torch.equal(outs[i][r], serial[i]), f"stream {i} call {r}"
