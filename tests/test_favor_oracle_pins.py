"""Pins for the FAVOR+ oracle (oracle/favor.py), against what the mathematics fixes (CPU).

The pages name FAVOR+ as random features whose inner products approximate the softmax
kernel exp(x . y) ("Efficient Transformers: Linear Attention and Flash Attention", section
"Linear attention: reordering the matmuls, not shrinking them"); the feature formula is the
positive random feature map of Choromanski et al. (ICLR 2021).  A plausible slip and the pin
that catches it:
  * a wrong sign or factor on |x|^2/2, a missing 1/sqrt(m), scale applied once instead of to
    both projection and norm           -> unbiasedness within the closed-form standard error
  * W used transposed, or rows not orthogonal / not Gaussian-length -> ORF structure pins
  * the key norm term dropped or the wrong operand normalised -> zero- and one-feature closed
    forms (weights exp(-|k|^2/2) and exp(w.k - |k|^2/2))
  * features that do not reach the softmax kernel at all        -> convergence to softmax
  * a transposed aggregate                                      -> linear == quadratic
  * an off-by-one causal mask or update-after-read              -> recurrence == masked form
"""
import math

import numpy as np
import pytest

from oracle import favor
from seeded_inputs import orf_draws, projection


def _gauss(seed, shape):
    return np.random.default_rng(seed).standard_normal(shape)


def _unbiased_check(W, x, y, scale, sigmas=6.0):
    """phi(x).phi(y) against exp(scale^2 x.y), within `sigmas` standard errors of the mean of
    m i.i.d. samples f_i = exp(w_i.(x'+y') - (|x'|^2+|y'|^2)/2), whose variance has the closed
    form exp(2|x'+y'|^2 - |x'|^2 - |y'|^2) - exp(2 x'.y')."""
    m = W.shape[0]
    est = float(favor.features(x, W, scale) @ favor.features(y, W, scale))
    xs, ys = scale * x, scale * y
    a = xs + ys
    truth = math.exp(float(xs @ ys))
    var = math.exp(2 * float(a @ a) - float(xs @ xs) - float(ys @ ys)) - truth ** 2
    se = math.sqrt(var / m)
    assert abs(est - truth) <= sigmas * se, (est, truth, se)
    return est, truth, se


@pytest.mark.parametrize("scale", [1.0, 0.5])
def test_features_unbiased_for_softmax_kernel_iid(scale):
    d, m = 8, 400_000
    W = projection(11, m, d, "f32").astype(np.float64)
    rng = np.random.default_rng(5)
    for _ in range(4):
        x = 0.3 * rng.standard_normal(d)
        y = 0.3 * rng.standard_normal(d)
        est, truth, se = _unbiased_check(W, x, y, scale)
        # the check is sharp: six standard errors stay under 6% of the value
        assert se / truth < 1e-2


def _slip_no_norm(x, W, s):
    return np.exp((s * x) @ W.T) / math.sqrt(W.shape[0])


def _slip_full_norm(x, W, s):
    xs = s * x
    return np.exp(xs @ W.T - xs @ xs) / math.sqrt(W.shape[0])


def _slip_scale_on_projection_only(x, W, s):
    return np.exp((s * x) @ W.T - 0.5 * (x @ x)) / math.sqrt(W.shape[0])


def _slip_mean_not_root(x, W, s):
    xs = s * x
    return np.exp(xs @ W.T - 0.5 * (xs @ xs)) / W.shape[0]


@pytest.mark.parametrize("slip", [_slip_no_norm, _slip_full_norm, _slip_scale_on_projection_only,
                                  _slip_mean_not_root])
def test_unbiasedness_rejects_plausible_slips(slip):
    """The same bound fails for each slip (the slip is planted here, in a copy of the formula
    on the CPU), so the pin above would catch it in the oracle."""
    d, m, scale = 8, 400_000, 0.5
    W = projection(12, m, d, "f32").astype(np.float64)
    rng = np.random.default_rng(6)
    x = 0.6 * rng.standard_normal(d)
    y = 0.6 * rng.standard_normal(d)
    est = float(slip(x, W, scale) @ slip(y, W, scale))
    _, truth, se = _unbiased_check(W, x, y, scale)
    assert abs(est - truth) > 6.0 * se


def test_features_positive_and_shape():
    W = projection(13, 96, 16, "f32").astype(np.float64)
    x = 3.0 * _gauss(1, (5, 7, 16))
    f = favor.features(x, W, 0.5)
    assert f.shape == (5, 7, 96)
    assert np.all(f > 0)


def test_orf_blocks_orthogonal_with_gaussian_lengths():
    d, m = 16, 40
    g, ln = orf_draws(21, m, d)
    W = favor.orf_projection(g, ln)
    assert W.shape == (3 * d, d)
    for b in range(3):
        blk = W[b * d:(b + 1) * d]
        gram = blk @ blk.T
        off = gram - np.diag(np.diag(gram))
        assert np.abs(off).max() < 1e-10 * np.abs(np.diag(gram)).max()
        # row lengths are the norms of the independent length vectors
        np.testing.assert_allclose(np.linalg.norm(blk, axis=1), np.linalg.norm(ln[b], axis=1),
                                   rtol=1e-12)
    # the span of each block is the Gaussian block's row space (QR of G: G = Q R, rows of Q^T)
    q, _ = np.linalg.qr(g[0])
    np.testing.assert_allclose(np.abs(q.T @ (W[:d] / np.linalg.norm(W[:d], axis=1)[:, None]).T),
                               np.eye(d), atol=1e-10)


def test_features_unbiased_with_orf():
    d = 8
    m = 400_000
    g, ln = orf_draws(22, m, d)
    W = favor.orf_projection(g, ln)[:m]
    rng = np.random.default_rng(7)
    x = 0.5 * rng.standard_normal(d)
    y = 0.5 * rng.standard_normal(d)
    # orthogonal blocks only lower the variance, so the i.i.d. bound still holds
    _unbiased_check(W, x, y, 1.0)


def test_zero_projection_closed_form():
    """W = 0: every feature is exp(-|x'|^2/2)/sqrt(m), so the weights are exp(-|k'|^2/2) and
    the query drops out.  d = 1, keys 0 and 1, values 1 and 3, scale 1:
    out = (1 + 3 e^{-1/2}) / (1 + e^{-1/2}) for every query."""
    W = np.zeros((3, 1))
    k = np.array([[0.0], [1.0]])
    v = np.array([[1.0], [3.0]])
    q = np.array([[0.3], [-2.0]])
    e = math.exp(-0.5)
    want = (1 + 3 * e) / (1 + e)
    out = favor.noncausal(q, k, v, W, 1.0)
    np.testing.assert_allclose(out[:, 0], [want, want], rtol=1e-15)
    # causal: the first query sees only key 0 (value 1), the second both
    outc = favor.quadratic(q, k, v, W, 1.0, causal=True)
    np.testing.assert_allclose(outc[:, 0], [1.0, want], rtol=1e-15)


def test_one_feature_closed_form():
    """m = 1, w = (2): phi(x) = exp(2x' - x'^2/2), weights exp(2k - k^2/2) (q drops out).
    Keys 1 and -1, values 4 and 0: out = 4 e^{1.5} / (e^{1.5} + e^{-2.5})."""
    W = np.array([[2.0]])
    k = np.array([[1.0], [-1.0]])
    v = np.array([[4.0], [0.0]])
    q = np.array([[0.7], [0.1]])
    want = 4 * math.exp(1.5) / (math.exp(1.5) + math.exp(-2.5))
    out = favor.noncausal(q, k, v, W, 1.0)
    np.testing.assert_allclose(out[:, 0], [want, want], rtol=1e-14)
    # scale 1/2 on x: weights exp(2 (k/2) - (k/2)^2/2) = exp(k - k^2/8)
    want_half = 4 * math.exp(1 - 0.125) / (math.exp(1 - 0.125) + math.exp(-1 - 0.125))
    np.testing.assert_allclose(favor.noncausal(q, k, v, W, 0.5)[:, 0], [want_half] * 2,
                               rtol=1e-14)


def test_converges_to_softmax_attention():
    """With many features the estimator's attention approaches softmax attention with logits
    scale^2 q.k; its error shrinks as the feature count grows (roughly as 1/sqrt(m))."""
    # (the estimator's variance grows as exp(|q' + k'|^2): moderate norms keep m modest)
    n, d = 48, 16
    scale = d ** -0.25
    q, k = (0.5 * _gauss(s, (n, d)) for s in (31, 32))
    v = _gauss(33, (n, d))
    ref = favor.softmax_attention(q, k, v, scale)
    errs = {}
    for m in (256, 65536):
        g, ln = orf_draws(40, m, d)
        W = favor.orf_projection(g, ln)[:m]
        out = favor.noncausal(q, k, v, W, scale)
        errs[m] = np.abs(out - ref).max() / np.abs(ref).max()
    assert errs[65536] < 0.05
    assert errs[65536] < errs[256] / 4
    # causal too, row by row
    g, ln = orf_draws(47, 65536, d)
    W = favor.orf_projection(g, ln)
    outc = favor.quadratic(q, k, v, W, scale, causal=True)
    refc = favor.softmax_attention(q, k, v, scale, causal=True)
    assert np.abs(outc - refc).max() / np.abs(refc).max() < 0.05
    # the first query attends to key 0 only
    np.testing.assert_allclose(outc[0], v[0], rtol=1e-12)


def test_linear_form_equals_quadratic_form():
    W = projection(50, 64, 16, "f32").astype(np.float64)
    q, k, v = (_gauss(s, (2, 3, 37, 16)) for s in (51, 52, 53))
    a = favor.noncausal(q, k, v, W, 0.5)
    b = favor.quadratic(q, k, v, W, 0.5, causal=False)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)
    _, S, z = favor.noncausal(q, k, v, W, 0.5, return_state=True)
    S2, z2 = favor.state(k, v, W, 0.5)
    np.testing.assert_allclose(S, S2, rtol=1e-13)
    np.testing.assert_allclose(z, z2, rtol=1e-13)
    # the state is phi(K)^T V with the feature index first
    assert S.shape == (2, 3, 64, 16)


def test_recurrence_equals_masked_form_and_state_carry():
    W = projection(60, 32, 8, "f32").astype(np.float64)
    q, k, v = (_gauss(s, (3, 29, 8)) for s in (61, 62, 63))
    rec, S, z = favor.causal_recurrent(q, k, v, W, 0.7, return_state=True)
    quad = favor.quadratic(q, k, v, W, 0.7, causal=True)
    np.testing.assert_allclose(rec, quad, rtol=1e-12, atol=1e-13)
    # the final state is the state of all tokens; the last row equals the non-causal row
    S2, z2 = favor.state(k, v, W, 0.7)
    np.testing.assert_allclose(S, S2, rtol=1e-12)
    np.testing.assert_allclose(z, z2, rtol=1e-12)
    np.testing.assert_allclose(rec[:, -1], favor.noncausal(q, k, v, W, 0.7)[:, -1], rtol=1e-12)
    # split at token 11 with the state carried
    r1, S1, z1 = favor.causal_recurrent(q[:, :11], k[:, :11], v[:, :11], W, 0.7,
                                        return_state=True)
    r2 = favor.causal_recurrent(q[:, 11:], k[:, 11:], v[:, 11:], W, 0.7, s0=S1, z0=z1)
    np.testing.assert_allclose(np.concatenate([r1, r2], axis=1), rec, rtol=1e-12, atol=1e-13)
    # the first output is v_0: one key, weight cancels
    np.testing.assert_allclose(rec[:, 0], v[:, 0], rtol=1e-12)


def test_decode_step_updates_before_reading():
    W = projection(70, 16, 4, "f32").astype(np.float64)
    q, k, v = (_gauss(s, (4,)) for s in (71, 72, 73))
    out, S, z = favor.decode_step(q, k, v, np.zeros((16, 4)), np.zeros(16), W, 1.0)
    # from the empty state the step's own key is the only one: out = v
    np.testing.assert_allclose(out, v, rtol=1e-12)
    fk = favor.features(k, W, 1.0)
    np.testing.assert_allclose(S, np.outer(fk, v), rtol=1e-15)
    np.testing.assert_allclose(z, fk, rtol=1e-15)


def test_rows_equal_the_full_forms():
    W = projection(80, 32, 8, "f32").astype(np.float64)
    q, k, v = (_gauss(s, (57, 8)) for s in (81, 82, 83))
    idx = [0, 1, 17, 56]
    np.testing.assert_allclose(favor.rows(q, k, v, W, 0.6, idx, causal=True),
                               favor.quadratic(q, k, v, W, 0.6, causal=True)[idx], rtol=1e-12)
    np.testing.assert_allclose(favor.rows(q, k, v, W, 0.6, idx, causal=False),
                               favor.noncausal(q, k, v, W, 0.6)[idx], rtol=1e-12)
