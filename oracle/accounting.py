"""Analytic cost figures the pages print for linear and softmax attention.

TEST INFRASTRUCTURE ONLY (same rule as the rest of ``oracle/``).

What the formulas are (restated, not transcribed):
  * "Linear Attention > Computational Complexity Analysis" (mbrenndoerfer.com, Language AI
    Handbook ch. 123, section 6) counts linear attention at 2nd + 4nDd + 2nD + n operations:
    every token pays 2d for the feature map (the page calls this count simplified), 2Dd for its
    share of phi(K)^T V, 2Dd for phi(q) times the aggregate, 2D for the normaliser's dot product
    and one division.  Softmax attention pays 4n^2 d + 5n^2: two n x n x d products and five
    operations per score for the softmax.  Its table Out[15] prints both at d = D = 64.
  * "Linear Attention > Memory Efficiency" (same chapter, section 7): the softmax form keeps n^2
    scores, the linear form a D x d aggregate and a D-vector key sum, whatever n is.  Its table
    Out[19] prints both in fp32 at d = 64, the first in MB of 10^6 bytes and the second in KB of
    1024 bytes.
  * Hoefler, "Let's Stop Calling Everything 'Linear Attention'", section 2 (memory-load
    traffic): a decode step cannot take less than the bytes it moves over the bandwidth.

D is the feature dimension; for an elementwise feature map such as elu + 1 it equals d.
Pinned by ``tests/test_accounting.py`` against every printed row of both tables.
"""
from __future__ import annotations


def linear_flops_per_token(d: int, features: int) -> int:
    """Operations one token costs in the linear form: 2d + 4Dd + 2D + 1."""
    return 2 * d + 4 * features * d + 2 * features + 1


def linear_attention_flops(n: int, d: int, features: int | None = None) -> int:
    """n tokens of the linear form (the cost is the same for every token)."""
    return n * linear_flops_per_token(d, d if features is None else features)


def softmax_attention_flops(n: int, d: int) -> int:
    """n^2 scores, each costing 4d for the two products and 5 for the softmax."""
    return n * n * (4 * d + 5)


def linear_state_bytes(d: int, features: int | None = None, word: int = 4) -> int:
    """The D x d aggregate and the D-vector key sum: what the linear form keeps, for any n."""
    D = d if features is None else features
    return D * (d + 1) * word  # D*d + D words


def score_matrix_bytes(n: int, word: int = 4) -> int:
    """The n x n scores of the softmax form."""
    return n * n * word


def decode_floor_seconds(step_bytes: int, bytes_per_second: float) -> float:
    """A decode step cannot beat its traffic over the bandwidth."""
    return step_bytes / bytes_per_second


# The tables' number formats, so that a test can compare the printed strings.
def as_ops(x: int) -> str:
    """Operation counts: mega (10^6) below a giga (10^9), one decimal; giga with two."""
    return "%.2fG" % (x / 1e9) if x >= 1e9 else "%.1fM" % (x / 1e6)


def as_megabytes(x: int) -> str:
    """The memory table's MB: 10^6 bytes, one decimal."""
    return "%.1f MB" % (x / 1e6)


def as_kibibytes(x: int) -> str:
    """The memory table's KB: 1024 bytes, one decimal (16,640 B prints as 16.2 KB)."""
    return "%.1f KB" % (x / 1024)
