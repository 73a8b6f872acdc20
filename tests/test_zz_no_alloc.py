"""The non-causal forward that allocates nothing (la_forward_noncausal_noalloc) against the one
that takes a workspace (la_forward_noncausal), through the C ABI: two calls in a row, the second
on a smaller input, each bit for bit equal to the workspace call and within the bf16 / fp32 bar
of the oracle.  The second call finds the first call's partials in the shared scratch and must
not be affected by them."""
import numpy as np
import pytest

import oracle
from gpu_util import f64, from_dev, need_gpu, say, to_dev
from metrics import TOL_BF16, TOL_F32, normwise_err
from seeded_inputs import random_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ea():
    need_gpu()
    import efficient_attention_amd
    return efficient_attention_amd


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("bf16", 128), ("f32", 64)])
def test_noalloc_equals_workspace_call(ea, dtype, d):
    import torch
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    # first a large call (many slices per head: the scratch fills with partials), then a smaller
    # one of another shape
    for i, (B, H, n) in enumerate([(2, 8, 9000), (1, 3, 1500)]):
        q, k, v = random_inputs(500 + 10 * d + i, (B, H, n, d), dtype, 1.0 / np.sqrt(d))
        tq, tk, tv = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
        assert ea.la_noncausal_workspace_bytes(B, H, n, d, tq.dtype) <= ea.LA_NOALLOC_SCRATCH_BYTES
        out = torch.full_like(tq, float("nan"))
        say("noalloc", dtype, d, B, H, n)
        ea.la_forward_noncausal_noalloc(tq, tk, tv, out=out)
        ref = ea.la_forward_noncausal(tq, tk, tv)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), (dtype, d, B, H, n)
        e = normwise_err(from_dev(out, dtype), oracle.noncausal_linear(f64(q, dtype), f64(k, dtype), f64(v, dtype)))
        assert e <= tol, e


def test_noalloc_refuses_shapes_beyond_its_scratch(ea):
    import torch
    B, H, n, d = 4096, 2, 64, 128  # one 66 KB partial state per head: more than the scratch
    assert ea.la_noncausal_workspace_bytes(B, H, n, d, torch.bfloat16) > ea.LA_NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, H, n, d), dtype=torch.bfloat16, device="cuda")
    out = torch.full_like(q, 3.0)
    say("noalloc too large")
    with pytest.raises(ea.LinAttnError) as e:
        ea.la_forward_noncausal_noalloc(q, q, q, out=out)
    assert e.value.status == -6
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())
