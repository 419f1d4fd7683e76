"""The layer step recorded once into a HIP graph and replayed over several batches
gives, at every replay, the same bits as the step run eagerly on the same batch
and bias: routing, counts, permutation, output and the updated bias.  Between
the replays the test does eager work of its own (the next batch copied into the
captured input, comparisons on the host after a synchronisation), and the bias
carried from replay to replay is the graph's own."""
import numpy as np
import pytest
import torch

from biased_top_routing_amd.runner import MoeLayerGPU, to_device
from gpu_util import dev_f32, host, say
from workloads import MID, TINY
from workloads.inputs import make_weights, make_x

GRAPH_CASES = [
    ("tiny fp32", TINY, False),
    ("mid bf16 gather", MID.with_(T=2048), True),
    ("mid bf16 copy", MID.with_(T=1000), False),
    ("small fp8", MID.with_(T=700, H=384, E=16, G=4, M=2, k=4, S=1, I=256, wgt="fp8_e4m3", group_topr=2), False),
]


@pytest.mark.gpu
@pytest.mark.parametrize("label,c,gather", GRAPH_CASES, ids=[g[0] for g in GRAPH_CASES])
def test_graph_replay_matches_eager(label, c, gather):
    wts = make_weights(c)
    eager = MoeLayerGPU(c, wts, gather=gather)
    graph = MoeLayerGPU(c, wts, gather=gather)
    bias_e = dev_f32(wts.bias0)
    bias_g = dev_f32(wts.bias0)
    x_g = to_device(make_x(c, 0))
    say(f"graph capture {label}")
    graph.capture(x_g, bias_g, gamma=c.gamma)
    torch.cuda.synchronize()
    assert (host(bias_g).view(np.uint32) == wts.bias0.view(np.uint32)).all()   # capture ran nothing
    for step in range(4):
        say(f"graph replay {label} step {step}")
        xs = to_device(make_x(c, step))
        x_g.copy_(xs)
        y_e = eager.forward(xs, bias_e, gamma=c.gamma)
        torch.cuda.synchronize()
        y_g = graph.replay()
        torch.cuda.synchronize()
        for name in ("topk_idx", "topk_w", "counts", "offsets", "perm", "inv"):
            a, b = host(getattr(eager, name)), host(getattr(graph, name))
            assert (a.view(np.uint32) == b.view(np.uint32)).all(), (name, step)
        assert (host(y_e).view(np.uint32) == host(y_g).view(np.uint32)).all(), step
        assert (host(bias_e).view(np.uint32) == host(bias_g).view(np.uint32)).all(), step
