"""The memory-system measurement kernels (include/la_ceiling.h) compute what they claim, exactly:
the copy copies, the read-only stream's words XOR to the XOR of the buffer, and the causal-pattern
kernel writes (q + k + v) rounded to bf16 for every element, over ragged segments.  Their timings
are the ceilings bench.py reports; these tests make sure no work was left out."""
import numpy as np
import pytest

from gpu_util import need_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ea():
    need_gpu()
    import efficient_attention_amd
    return efficient_attention_amd


def test_ceiling_copy_and_read(ea):
    import torch
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    nbytes = (10 << 20) + 48  # not a multiple of the kernels' step
    src = torch.randint(-2 ** 31, 2 ** 31 - 1, (nbytes // 4,), dtype=torch.int32, device="cuda", generator=gen)
    dst = torch.zeros_like(src)
    say("ceiling copy / read")
    ea.la_ceiling_copy(src, dst)
    sink = ea.la_ceiling_read(src)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    words = src.cpu().numpy().view(np.uint32)
    assert np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32)) == np.bitwise_xor.reduce(words)


@pytest.mark.parametrize("B,H,n,seg_len", [(1, 3, 1000, 256), (2, 2, 128, 128), (1, 1, 4097, 4096)])
def test_ceiling_causal_pattern_is_q_plus_k_plus_v(ea, B, H, n, seg_len):
    import torch
    gen = torch.Generator(device="cuda")
    gen.manual_seed(n)
    q, k, v = (torch.randn(B, H, n, 128, device="cuda", generator=gen).to(torch.bfloat16) for _ in range(3))
    out = torch.full_like(q, float("nan"))
    say("ceiling causal pattern", B, H, n, seg_len)
    ea.la_ceiling_causal_pattern(q, k, v, seg_len, out=out)
    ref = ((q.float() + k.float()) + v.float()).to(torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
