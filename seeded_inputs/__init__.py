"""Seeded synthetic inputs shared by the tests, the smoke check and bench.py.

This module holds NO attention arithmetic: it draws seeded Gaussian numbers, encodes and
decodes bf16, and names the workload shapes.  It is the only code that both the fp64
oracle (``oracle/``) and the HIP path (``efficient_attention_amd/``) consume, and it imports
neither of them.

Generator.  Each (workload seed, tensor tag, batch index b, head index h) owns an
independent NumPy PCG64 stream seeded through ``SeedSequence([seed, tag, b, h])``.  So one
head's inputs can be regenerated alone (the oracle checks sampled heads of the large
workloads without generating the rest), and the full tensors can be generated in parallel
threads with the same bytes.  Values are ``standard_normal(dtype=float32)``, multiplied in
fp32 by ``scale`` (1/sqrt(d) where the workload says N(0,1)/sqrt(d)), then rounded to bf16
with round-to-nearest-even where the workload is bf16.

Workloads (the pages' shapes: d = 64 with n up to 16384 in the complexity and memory
tables, n = 65,536 with d_head = 128 and 32 heads in the long-context Q&A):
  C1 non-causal fp32  B=1 H=1  n=512   d=64            seed 1
  C2 causal     fp32  B=1 H=1  n=4096  d=64  chunk 64  seed 2
  C3 non-causal bf16  B=8 H=16 n=16384 d=64            seed 3
  C4 causal     bf16  B=4 H=32 n=65536 d=128 chunk 128 seed 4
  C5 decode     bf16  256 sequences x H=32, d=128, state from 1024 prior tokens, 512 steps,
                seed 5
FAVOR+ feature map (random features m; q, k, v N(0,1), feature scale d^(-1/4)):
  F3 non-causal bf16  B=8 H=16 n=16384 d=64  m=256            seed 6
  F4 causal     bf16  B=4 H=32 n=65536 d=128 m=128  chunk 64  seed 7
  F5 decode     bf16  256 x 32 heads, d=128, m=128, 1024 prior tokens, 512 steps, seed 8
The projection of a FAVOR+ workload is drawn by ``projection`` (i.i.d. N(0,1) rows) from
the workload seed.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

TAG_Q, TAG_K, TAG_V = 0, 1, 2
TAG_PRIOR_K, TAG_PRIOR_V = 3, 4
TAG_PROJ, TAG_PROJ_LEN = 5, 6


@dataclass(frozen=True)
class Workload:
    name: str
    form: str          # "noncausal" | "causal" | "decode"
    dtype: str         # "f32" | "bf16"
    B: int
    H: int
    n: int             # tokens per head (decode: steps)
    d: int
    chunk: int
    seed: int
    scaled: bool       # N(0,1)/sqrt(d) when True, N(0,1) otherwise
    prior: int = 0     # decode only: tokens folded into the initial state
    m: int = 0         # FAVOR+ workloads: random features (0: phi = elu + 1)


WORKLOADS = {
    "C1": Workload("C1", "noncausal", "f32", 1, 1, 512, 64, 0, 1, False),
    "C2": Workload("C2", "causal", "f32", 1, 1, 4096, 64, 64, 2, False),
    "C3": Workload("C3", "noncausal", "bf16", 8, 16, 16384, 64, 0, 3, True),
    "C4": Workload("C4", "causal", "bf16", 4, 32, 65536, 128, 128, 4, True),
    "C5": Workload("C5", "decode", "bf16", 256, 32, 512, 128, 0, 5, True, prior=1024),
    # the same shapes with FAVOR+ features: unit-variance q, k, feature scale d^(-1/4)
    "F3": Workload("F3", "noncausal", "bf16", 8, 16, 16384, 64, 0, 6, False, m=256),
    "F4": Workload("F4", "causal", "bf16", 4, 32, 65536, 128, 64, 7, False, m=128),
    "F5": Workload("F5", "decode", "bf16", 256, 32, 512, 128, 0, 8, False, prior=1024, m=128),
}


# ----------------------------------------------------------------------------- bf16 codec
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round-to-nearest-even), returned as uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    r = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = np.uint16(0x7FC0)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact decode of bf16 bit patterns (uint16) to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact decode of host data of the given storage type to float64."""
    if dtype == "bf16":
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def encode(x32: np.ndarray, dtype: str) -> np.ndarray:
    """float32 -> storage type (float32 unchanged, bf16 as uint16 bits)."""
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    return np.ascontiguousarray(x32, dtype=np.float32)


# ----------------------------------------------------------------------------- generation
def _stream(seed: int, tag: int, b: int, h: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tag, b, h])))


def head_tensor(seed: int, tag: int, b: int, h: int, rows: int, d: int, scaled: bool,
                dtype: str) -> np.ndarray:
    """One head's [rows, d] block of one tensor, in storage type."""
    x = _stream(seed, tag, b, h).standard_normal((rows, d), dtype=np.float32)
    if scaled:
        x *= np.float32(1.0 / np.sqrt(d))
    return encode(x, dtype)


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def full_tensor(seed: int, tag: int, B: int, H: int, rows: int, d: int, scaled: bool,
                dtype: str) -> np.ndarray:
    """[B, H, rows, d] tensor in storage type, heads generated in parallel threads."""
    st = np.uint16 if dtype == "bf16" else np.float32
    out = np.empty((B, H, rows, d), dtype=st)

    def fill(bh):
        b, h = divmod(bh, H)
        out[b, h] = head_tensor(seed, tag, b, h, rows, d, scaled, dtype)

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(fill, range(B * H)))
    return out


def forward_inputs(w: Workload, heads=None):
    """Q, K, V for a forward workload.  heads=None: full [B,H,n,d] tensors; otherwise a list
    of (b, h) pairs and the result is [len(heads), n, d] for those heads only."""
    if heads is None:
        return tuple(full_tensor(w.seed, t, w.B, w.H, w.n, w.d, w.scaled, w.dtype)
                     for t in (TAG_Q, TAG_K, TAG_V))
    res = []
    for t in (TAG_Q, TAG_K, TAG_V):
        res.append(np.stack([head_tensor(w.seed, t, b, h, w.n, w.d, w.scaled, w.dtype)
                             for (b, h) in heads]))
    return tuple(res)


def decode_inputs(w: Workload, heads=None, steps=None, prior=None):
    """Decode workload inputs: prior keys/values [.., prior, d] and per-step q, k, v
    [.., steps, d] (steps along axis -2, one token per step), all in storage type.
    heads=None gives [B, H, ...] tensors, otherwise [len(heads), ...]."""
    steps = w.n if steps is None else steps
    prior = w.prior if prior is None else prior

    def one(tag, rows, b, h):
        return head_tensor(w.seed, tag, b, h, rows, w.d, w.scaled, w.dtype)

    if heads is None:
        pk = full_tensor(w.seed, TAG_PRIOR_K, w.B, w.H, prior, w.d, w.scaled, w.dtype)
        pv = full_tensor(w.seed, TAG_PRIOR_V, w.B, w.H, prior, w.d, w.scaled, w.dtype)
        q = full_tensor(w.seed, TAG_Q, w.B, w.H, steps, w.d, w.scaled, w.dtype)
        k = full_tensor(w.seed, TAG_K, w.B, w.H, steps, w.d, w.scaled, w.dtype)
        v = full_tensor(w.seed, TAG_V, w.B, w.H, steps, w.d, w.scaled, w.dtype)
        return pk, pv, q, k, v
    pk = np.stack([one(TAG_PRIOR_K, prior, b, h) for (b, h) in heads])
    pv = np.stack([one(TAG_PRIOR_V, prior, b, h) for (b, h) in heads])
    q = np.stack([one(TAG_Q, steps, b, h) for (b, h) in heads])
    k = np.stack([one(TAG_K, steps, b, h) for (b, h) in heads])
    v = np.stack([one(TAG_V, steps, b, h) for (b, h) in heads])
    return pk, pv, q, k, v


def random_inputs(seed: int, shape, dtype: str = "f32", scale: float = 1.0):
    """Small ad-hoc Q, K, V of an arbitrary shape [..., n, d] for tests."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 99])))
    res = []
    for _ in range(3):
        x = g.standard_normal(shape, dtype=np.float32) * np.float32(scale)
        res.append(encode(x, dtype))
    return tuple(res)


def projection(seed: int, m: int, d: int, dtype: str) -> np.ndarray:
    """A FAVOR+ projection [m, d] with i.i.d. N(0, 1) entries, in storage type."""
    x = _stream(seed, TAG_PROJ, 0, 0).standard_normal((m, d), dtype=np.float32)
    return encode(x, dtype)


def orf_draws(seed: int, m: int, d: int):
    """The Gaussian numbers an orthogonal random projection is built from: ceil(m/d) blocks
    [d, d] and as many [d, d] blocks of length vectors, float64 N(0, 1)."""
    nb = -(-m // d)
    g = _stream(seed, TAG_PROJ, 1, 0).standard_normal((nb, d, d))
    ln = _stream(seed, TAG_PROJ_LEN, 1, 0).standard_normal((nb, d, d))
    return g, ln
