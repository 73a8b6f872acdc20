"""CPU checks of the byte and floor arithmetic bench.py reports, against the per-workload figures
derived independently from the shapes (algorithmic bytes: q, k, v read and out written once per
head-token; decode: the fp32 state read and written plus q, k, v, out)."""
import bench
from seeded_inputs import WORKLOADS


def test_forward_bytes_of_the_workloads():
    C3, C4 = WORKLOADS["C3"], WORKLOADS["C4"]
    assert bench.algorithmic_bytes(C3.B, C3.H, C3.n, C3.d, 2) == 1_073_741_824
    assert bench.algorithmic_bytes(C4.B, C4.H, C4.n, C4.d, 2) == 8_589_934_592
    # 4 d eb bytes per head-token
    assert bench.algorithmic_bytes(1, 1, 1, 64, 4) == 1024


def test_decode_bytes_per_step():
    C5 = WORKLOADS["C5"]
    heads = C5.B * C5.H
    assert heads == 8192
    # per head: 2 (d^2 + d) fp32 for the state and z, 4 d bf16 for q, k, v, out = 133,120 B
    assert bench.decode_bytes(1, 128, 2) == 2 * (128 * 128 + 128) * 4 + 4 * 128 * 2 == 133_120
    assert bench.decode_bytes(heads, C5.d, 2) == 1_090_519_040


def test_favor_alu_floor():
    # 6 issue slots per feature value at 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz
    F3 = WORKLOADS["F3"]
    values = 2 * F3.m * F3.B * F3.H * F3.n
    assert values == 1_073_741_824
    assert abs(bench.favor_alu_floor_s(values) - values * 6 / (256 * 4 * 16 * 2.4e9)) < 1e-15
    assert 0.16 < bench.favor_alu_floor_s(values) * 1e3 < 0.17
