"""The hot path under HIP graph capture.  The library makes no allocation, copy or memset call, so
a caller that provides the output and the workspace can capture any entry point into a torch
CUDA graph (its kernels on the capturing stream) and replay it on new inputs written into the
captured tensors:
- the non-causal forward that allocates nothing (la_forward_noncausal_noalloc), the use it
  exists for;
- the causal forward with a caller workspace (state sums and chunked kernel, bf16 and fp32);
- the in-place decode step, replayed as consecutive steps on the state it updates.
Every replay is checked bit for bit against eager calls, with eager work and synchronisations
between the replays."""
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


@pytest.mark.parametrize("dtype,d,chunk,B,H,n", [("bf16", 128, 128, 1, 3, 3000), ("f32", 64, 64, 1, 2, 2000)])
def test_causal_graph_replays_equal_eager_calls(ea, dtype, d, chunk, B, H, n):
    import torch
    inputs = [random_inputs(900 + 10 * d + r, (B, H, n, d), dtype, 1.0 / np.sqrt(d)) for r in range(5)]
    q, k, v = (to_dev(x, dtype) for x in inputs[0])
    out = torch.empty_like(q)
    need = ea.la_causal_workspace_bytes(B, H, n, d, chunk, q.dtype)
    assert need > 0  # few heads: the sequence is cut into segments, so both stages are captured
    ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_eager = torch.empty(need, dtype=torch.uint8, device=q.device)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ea.la_forward_causal(q, k, v, chunk=chunk, out=out, ws=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    say("graph capture causal", dtype, d, chunk, B, H, n)
    with torch.cuda.graph(graph):
        ea.la_forward_causal(q, k, v, chunk=chunk, out=out, ws=ws)
    for r in range(1, 5):
        for dst, src in zip((q, k, v), inputs[r]):
            dst.copy_(to_dev(src, dtype))
        torch.cuda.synchronize()
        out.fill_(float("nan"))
        say("graph replay causal", r)
        graph.replay()
        torch.cuda.synchronize()
        ref = ea.la_forward_causal(q, k, v, chunk=chunk, ws=ws_eager)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), (dtype, d, r)


def test_decode_graph_replays_are_consecutive_steps(ea):
    import torch
    B, H, d, steps = 4, 8, 128, 4
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    S0 = torch.rand(B, H, d, d, device="cuda", generator=g) * 0.1
    z0 = torch.rand(B, H, d, device="cuda", generator=g) + 1.0
    toks = [random_inputs(950 + r, (B, H, d), "bf16", 1.0 / np.sqrt(d)) for r in range(steps + 1)]
    q, k, v = (to_dev(x, "bf16") for x in toks[0])
    out = torch.empty_like(q)
    S, z = S0.clone(), z0.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # a warm-up step on scratch state
        ea.la_decode_step(q, k, v, S.clone(), z.clone(), out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    say("graph capture decode", B, H, d)
    with torch.cuda.graph(graph):
        ea.la_decode_step(q, k, v, S, z, out=out)
    S_ref, z_ref = S0.clone(), z0.clone()
    for r in range(1, steps + 1):
        for dst, src in zip((q, k, v), toks[r]):
            dst.copy_(to_dev(src, "bf16"))
        torch.cuda.synchronize()
        out.fill_(float("nan"))
        say("graph replay decode", r)
        graph.replay()
        torch.cuda.synchronize()
        ref = ea.la_decode_step(q, k, v, S_ref, z_ref)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), r
        assert torch.equal(S, S_ref) and torch.equal(z, z_ref), r
