"""The non-causal forward that allocates nothing (la_forward_noncausal_noalloc) under HIP graph
capture, the use it exists for: captured once into a torch CUDA graph (its kernels on the
capturing stream, no allocation and no memset node), then replayed on new inputs written into
the captured tensors between replays.  Every replay is checked bit for bit against the eager call
that takes a workspace, with eager work and synchronisations between the replays."""
import numpy as np
import pytest

from gpu_util import need_gpu, say, to_dev
from seeded_inputs import random_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ea():
    need_gpu()
    import efficient_attention_amd
    return efficient_attention_amd


@pytest.mark.parametrize("dtype,d,B,H,n", [("bf16", 64, 2, 4, 3000), ("f32", 128, 1, 3, 2000)])
def test_noalloc_graph_replays_equal_eager_calls(ea, dtype, d, B, H, n):
    import torch
    inputs = [random_inputs(700 + 10 * d + r, (B, H, n, d), dtype, 1.0 / np.sqrt(d)) for r in range(5)]
    q, k, v = (to_dev(x, dtype) for x in inputs[0])
    out = torch.empty_like(q)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up: the first call on a device looks up the scratch address
        ea.la_forward_noncausal_noalloc(q, k, v, out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    say("graph capture", dtype, d, B, H, n)
    with torch.cuda.graph(graph):
        ea.la_forward_noncausal_noalloc(q, k, v, out=out)
    for r in range(1, 5):
        for dst, src in zip((q, k, v), inputs[r]):
            dst.copy_(to_dev(src, dtype))
        torch.cuda.synchronize()
        out.fill_(float("nan"))
        say("graph replay", r)
        graph.replay()
        torch.cuda.synchronize()
        ref = ea.la_forward_noncausal(q, k, v)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), (dtype, d, r)
