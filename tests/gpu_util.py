"""Host <-> device plumbing for the GPU tests (no arithmetic of the method here)."""
import sys

import numpy as np
import pytest

from seeded_inputs import bf16_bits_to_f32


def need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import efficient_attention_amd as ea
    ea.load()  # raises if the HIP library is not built
    return torch


def say(*msg):
    """Name the case before a GPU step (flushed, so a crash still shows what was running)."""
    print("[gpu-case]", *msg, flush=True)
    sys.stdout.flush()


def to_dev(x, dtype):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def from_dev(t, dtype):
    """Device tensor -> float64 numpy (exact decode)."""
    import torch
    torch.cuda.synchronize()
    if dtype == "bf16":
        return bf16_bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    return t.float().cpu().numpy().astype(np.float64)


def f64(x, dtype):
    if dtype == "bf16":
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)
