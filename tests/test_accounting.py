"""Pin the cost formulas to every printed row of the pages' two tables (CPU only).

Sources: "Linear Attention > Computational Complexity Analysis" Out[15] and "Linear
Attention > Memory Efficiency" Out[19] (mbrenndoerfer.com, ch. 123); fixtures in
tests/golden/ quote the printed rows.
"""
import os

from oracle import accounting as A

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name, sep=None):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.strip().split(sep) for ln in f if ln.strip() and not ln.startswith("#")]


def test_flops_table_every_row():
    rows = _rows("flops_table.txt")
    assert len(rows) == 8
    d = 64
    for n, std, lin, speed in rows:
        n = int(n)
        s = A.softmax_attention_flops(n, d)
        li = A.linear_attention_flops(n, d)
        assert A.as_ops(s) == std, (n, s)
        assert A.as_ops(li) == lin, (n, li)
        assert "%.1fx" % (s / li) == speed, (n, s / li)


def test_flops_exact_values():
    # 2nd + 4nDd + 2nD + n at d = D = 64, n = 16384; the standard count 4n^2 d + 5n^2
    assert A.linear_attention_flops(16384, 64) == 272_646_144
    assert A.softmax_attention_flops(16384, 64) == 70_061_654_016
    # per head-token at d = 128: 2d + 4d^2 + 2d + 1
    assert A.linear_attention_flops(1, 128) == 66_049
    assert A.linear_attention_flops(1, 64) == 16_641


def test_memory_table_every_row():
    rows = _rows("memory_table.txt", "|")
    assert len(rows) == 6
    d = 64
    for n, std, lin, red in rows:
        n = int(n)
        s = A.score_matrix_bytes(n)
        li = A.linear_state_bytes(d)
        assert A.as_megabytes(s) == std, (n, s)
        assert A.as_kibibytes(li) == lin, (n, li)
        assert "%.0fx" % (s / li) == red, (n, s / li)


def test_feature_dimension_separate_from_d():
    # the printed formula with D != d (a feature map that changes the width): D*d + D words of
    # state and 2d + 4Dd + 2D + 1 operations per token
    assert A.linear_state_bytes(64, features=256) == (256 * 64 + 256) * 4
    assert A.linear_attention_flops(10, 64, features=256) == 10 * (2 * 64 + 4 * 256 * 64 + 2 * 256 + 1)


def test_state_is_16640_bytes_at_d64():
    assert A.linear_state_bytes(64) == 16640
    # "over 16 GB" for the standard matrix at 65,536 tokens
    assert A.score_matrix_bytes(65536) > 16e9


def test_decode_floor():
    # 8192 heads x (state read + write of 66,048 B each way + 4 x 256 B of q/k/v/out)
    per_step = 8192 * (2 * 66048 + 4 * 256)
    assert per_step == 1_090_519_040
    assert abs(A.decode_floor_seconds(per_step, 8.0e12) - 136.3e-6) < 0.1e-6
