"""CPU check of the reduction the >2^31-element GPU tests rely on: with every key row outside an
"active" set made inactive (-1e4 in every feature for elu + 1, 300 for FAVOR+), the oracle
evaluated over the active keys alone gives the same rows as the oracle over all keys, causal
and not.  Small heads, so the full definition is cheap."""
import numpy as np
import pytest

import oracle
from oracle import favor
from test_gpu_maxsize import INACTIVE_ELU, INACTIVE_FAVOR, _elu_ref, _favor_ref


def _sparse_head(rng, n, d, inactive, kscale):
    q = rng.standard_normal((n, d)) * kscale
    v = rng.standard_normal((n, d))
    k = np.full((n, d), inactive)
    act = np.unique(np.concatenate([[0, n - 1], rng.integers(0, n, size=12)])).astype(np.int64)
    k[act] = rng.standard_normal((act.size, d)) * kscale
    qrows = np.unique(np.concatenate([[0, 1, n - 1], rng.integers(0, n, size=10)])).astype(np.int64)
    return q, k, v, act, qrows


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_elu_active_keys_reduction(causal, d):
    rng = np.random.default_rng(31 + d)
    q, k, v, act, qrows = _sparse_head(rng, 300, d, INACTIVE_ELU, d ** -0.5)
    full = oracle.rows(q, k, v, qrows, causal=causal)
    red = _elu_ref(q[qrows], k[act], v[act], act, qrows, causal)
    assert np.max(np.abs(full - red)) <= 1e-13 * np.max(np.abs(full))
    # an inactive row made active (features 1) does change the rows: the check has teeth
    k3 = k.copy()
    k3[np.setdiff1d(np.arange(300), act)[0]] = 0.0
    assert not np.allclose(oracle.rows(q, k3, v, qrows, causal=causal), full)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d,m", [(64, 256), (128, 128)])
def test_favor_active_keys_reduction(causal, d, m):
    rng = np.random.default_rng(41 + d + m)
    q, k, v, act, qrows = _sparse_head(rng, 300, d, INACTIVE_FAVOR, 1.0)
    W = rng.standard_normal((m, d))
    scale = d ** -0.25
    full = favor.rows(q, k, v, W, scale, qrows, causal=causal)
    red = _favor_ref(q[qrows], k[act], v[act], act, qrows, W, scale, causal)
    assert np.max(np.abs(full - red)) <= 1e-12 * np.max(np.abs(full))
    assert np.all(favor.features(k[np.setdiff1d(np.arange(300), act)], W, scale) == 0.0)
