"""Analytic cost accounting that the pages print for linear vs standard attention.

TEST INFRASTRUCTURE ONLY (same rule as the rest of ``oracle/``).

Restated from:
  * "Linear Attention > Memory Efficiency" (mbrenndoerfer.com, Language AI Handbook ch. 123,
    section 7), code cell In[17] and its table Out[19]: the standard form stores the n x n
    weights (n^2 values); the linear form stores the D x d aggregate plus the D-vector key
    sum (D*d + D values), independent of n.
  * "Linear Attention > Computational Complexity Analysis" (same chapter, section 6), code
    cell In[14] and its table Out[15]: standard attention costs 2n^2 d (QK^T) + 5n^2
    (softmax) + 2n^2 d (weights times V); linear attention costs 2nd (feature map, a
    simplified count) + 2nDd (phi(K)^T V) + 2nDd (phi(Q) KV) + 2nD + n (normalisation).
  * Hoefler, "Let's Stop Calling Everything 'Linear Attention'", section 2 (memory-load
    traffic): a decode step's time is bounded below by the bytes it moves divided by the
    effective bandwidth.

Pinned by ``tests/test_accounting.py`` against every printed row of both tables.
"""
from __future__ import annotations


def memory_standard_attention(n: int, d: int, dtype_bytes: int = 4) -> int:
    """Bytes of the n x n attention weights (independent of d)."""
    return n * n * dtype_bytes


def memory_linear_attention(n: int, d: int, D: int | None = None, dtype_bytes: int = 4) -> int:
    """Bytes of the D x d key-value aggregate plus the D-vector key sum (independent of n)."""
    if D is None:
        D = d
    return D * d * dtype_bytes + D * dtype_bytes


def flops_standard_attention(n: int, d: int) -> int:
    return 2 * n * n * d + 5 * n * n + 2 * n * n * d


def flops_linear_attention(n: int, d: int, D: int | None = None) -> int:
    if D is None:
        D = d
    feature = 2 * n * d
    kv = 2 * n * D * d
    qkv = 2 * n * D * d
    norm = 2 * n * D + n
    return feature + kv + qkv + norm


def decode_time_floor_s(bytes_per_step: int, bandwidth_bytes_per_s: float) -> float:
    """Lower bound on one decode step's time: bytes moved / effective bandwidth."""
    return bytes_per_step / bandwidth_bytes_per_s


# Formatting used by the printed tables (reproduced so that a test can compare strings).
def fmt_flops(x: int) -> str:
    if x >= 1e9:
        return "%.2fG" % (x / 1e9)
    return "%.1fM" % (x / 1e6)


def fmt_mem_mb(x: int) -> str:
    """The memory table's MB is 10^6 bytes."""
    return "%.1f MB" % (x / 1e6)


def fmt_mem_kb(x: int) -> str:
    """The memory table's KB is 1024 bytes (16,640 B prints as 16.2 KB)."""
    return "%.1f KB" % (x / 1024)
