"""Pins for the fp64 oracle, against what the pages and the mathematics fix (CPU only).

Each pin is chosen so that a plausible slip in the oracle fails at least one of them:
  * a wrong feature map (sign, branch, alpha)        -> phi values, torch ELU, positivity
  * a transposed aggregate or a swapped operand      -> linear vs quadratic on random data
  * a dropped or wrong normaliser                    -> worked example, ones vector, convexity
  * an off-by-one causal mask                        -> out_0 = v_0, recurrence vs masked form
  * update-after-read in the decode step             -> decode vs causal
  * a wrong chunk boundary or carry                  -> chunked vs recurrence at ragged sizes
Sources: "Efficient Transformers: Linear Attention and Flash Attention" (eq. Attention_i,
"Worked example", "The recurrent view", Active recall A4/A5).
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from seeded_inputs import random_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _frac_array(rows):
    return np.array([[float(Fraction(x)) for x in row] for row in rows])


def _worked():
    with open(os.path.join(GOLDEN, "worked_example.json")) as f:
        w = json.load(f)
    Q = np.array(w["Q"], dtype=np.float64)
    K = np.array(w["K"], dtype=np.float64)
    V = np.array(w["V"], dtype=np.float64)
    return w, Q, K, V


def _rand(seed, n, d, bh=1, scale=1.0):
    q, k, v = random_inputs(seed, (bh, n, d), "f32", scale)
    return q.astype(np.float64), k.astype(np.float64), v.astype(np.float64)


# --------------------------------------------------------------------- feature map
def test_phi_closed_form_values():
    # elu(x) + 1 with alpha = 1: x + 1 above zero, exp(x) at and below zero.
    assert oracle.phi(np.array([0.0]))[0] == 1.0
    assert oracle.phi(np.array([1.0]))[0] == 2.0
    assert oracle.phi(np.array([2.5]))[0] == 3.5
    assert oracle.phi(np.array([-1.0]))[0] == pytest.approx(0.36787944117144233, rel=1e-15)
    assert oracle.phi(np.array([-2.0]))[0] == pytest.approx(0.1353352832366127, rel=1e-15)
    # continuity at 0 from both sides
    eps = 1e-12
    assert abs(oracle.phi(np.array([eps]))[0] - oracle.phi(np.array([-eps]))[0]) < 3e-12


def test_phi_matches_library_elu():
    torch = pytest.importorskip("torch")
    x = np.linspace(-30, 30, 20001)
    ref = torch.nn.functional.elu(torch.from_numpy(x), alpha=1.0).numpy() + 1.0
    got = oracle.phi(x)
    # elu's own evaluation is expm1(x) + 1 below zero; agreement to a few ulps of 1
    assert np.max(np.abs(got - ref) / np.maximum(ref, 1e-300)) < 1e-12 or \
        np.max(np.abs(got - ref)) < 4e-16


def test_phi_positive_down_to_minus_80():
    # Active recall A4: phi must be non-negative; elu + 1 is strictly positive.
    x = np.linspace(-80, 80, 100001)
    assert np.all(oracle.phi(x) > 0)


# --------------------------------------------------------------------- worked example
def test_worked_example_both_orders():
    w, Q, K, V = _worked()
    p = w["printed"]
    out_lin, kv, z = oracle.noncausal_linear(Q, K, V, oracle.PHI_IDENTITY, return_state=True)
    out_quad, W = oracle.quadratic(Q, K, V, causal=False, feature_map=oracle.PHI_IDENTITY,
                                   return_weights=True)
    np.testing.assert_array_equal(W, np.array(p["scores_QKt"], dtype=np.float64))
    np.testing.assert_array_equal(W.sum(axis=1), np.array(p["row_sums"], dtype=np.float64))
    np.testing.assert_allclose(W / W.sum(axis=1, keepdims=True), _frac_array(p["weights"]),
                               rtol=0, atol=1e-15)
    np.testing.assert_array_equal(kv, np.array(p["KtV"], dtype=np.float64))
    np.testing.assert_array_equal(z, np.array(p["k_sum"], dtype=np.float64))
    expect = _frac_array(p["out"])
    np.testing.assert_allclose(out_lin, expect, rtol=0, atol=1e-15)
    np.testing.assert_allclose(out_quad, expect, rtol=0, atol=1e-15)
    # numerators and denominators printed for the linear path
    num = Q @ kv
    np.testing.assert_array_equal(num, np.array(p["numerators"], dtype=np.float64))
    np.testing.assert_array_equal(Q @ z, np.array(p["denominators"], dtype=np.float64))


def test_worked_example_causal_forms():
    w, Q, K, V = _worked()
    expect = _frac_array(w["derived_by_hand"]["causal_out"])
    for got in (oracle.quadratic(Q, K, V, causal=True, feature_map=oracle.PHI_IDENTITY),
                oracle.causal_recurrent(Q, K, V, feature_map=oracle.PHI_IDENTITY),
                oracle.causal_chunked(Q, K, V, 2, feature_map=oracle.PHI_IDENTITY)):
        np.testing.assert_allclose(got, expect, rtol=0, atol=1e-15)
    # the last causal row is the printed non-causal row
    np.testing.assert_allclose(expect[2], _frac_array(w["printed"]["out"])[2], atol=0)


def test_worked_example_decode_steps():
    w, Q, K, V = _worked()
    expect = _frac_array(w["derived_by_hand"]["causal_out"])
    S = np.zeros((2, 2))
    z = np.zeros(2)
    for t in range(3):
        out, S, z = oracle.decode_step(Q[t], K[t], V[t], S, z, oracle.PHI_IDENTITY)
        np.testing.assert_allclose(out, expect[t], atol=1e-15)
    np.testing.assert_array_equal(S, np.array(w["printed"]["KtV"], dtype=np.float64))
    np.testing.assert_array_equal(z, np.array(w["printed"]["k_sum"], dtype=np.float64))


# --------------------------------------------------------------------- brute force
def _brute_force_python(Q, K, V, causal):
    """Pure-Python triple loop of the definition (tiny sizes only)."""
    n, d = Q.shape

    def ph(x):
        return x + 1.0 if x > 0 else math.exp(x)

    out = np.zeros((n, d))
    for i in range(n):
        keys = range(i + 1) if causal else range(n)
        ws = []
        for j in keys:
            ws.append(sum(ph(Q[i, a]) * ph(K[j, a]) for a in range(d)))
        tot = sum(ws)
        for c in range(d):
            out[i, c] = sum(wj * V[j, c] for wj, j in zip(ws, keys)) / tot
    return out


@pytest.mark.parametrize("n,d", [(1, 1), (2, 3), (5, 4), (7, 2), (9, 8)])
def test_pure_python_brute_force(n, d):
    q, k, v = _rand(10 + n * 13 + d, n, d)
    for causal in (False, True):
        ref = _brute_force_python(q[0], k[0], v[0], causal)
        if causal:
            got = oracle.causal_recurrent(q, k, v)[0]
        else:
            got = oracle.noncausal_linear(q, k, v)[0]
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("n", [1, 2, 3, 17, 64])
@pytest.mark.parametrize("d", [1, 4, 16, 64])
def test_linear_equals_quadratic_tiny(n, d):
    q, k, v = _rand(n * 1000 + d, n, d, bh=2)
    a = oracle.noncausal_linear(q, k, v)
    b = oracle.quadratic(q, k, v, causal=False)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)


def test_linear_equals_quadratic_n512_d64():
    # the size of the small fp32 non-causal workload (n = 512, d = 64)
    q, k, v = _rand(1, 512, 64)
    a = oracle.noncausal_linear(q, k, v)
    b = oracle.quadratic(q, k, v, causal=False)
    assert np.max(np.abs(a - b)) / np.max(np.abs(b)) < 1e-12


# --------------------------------------------------------------------- causal forms
@pytest.mark.parametrize("n", [1, 2, 63, 64, 65, 130])
def test_recurrence_equals_masked_quadratic_and_chunked(n):
    d = 8
    q, k, v = _rand(500 + n, n, d, bh=2)
    rec = oracle.causal_recurrent(q, k, v)
    quad = oracle.quadratic(q, k, v, causal=True)
    np.testing.assert_allclose(rec, quad, rtol=1e-12, atol=1e-13)
    for C in (1, 16, 64, 128, max(n, 1)):
        ch = oracle.causal_chunked(q, k, v, C)
        np.testing.assert_allclose(ch, rec, rtol=1e-12, atol=1e-13)


def test_causal_special_rows():
    q, k, v = _rand(7, 50, 6)
    c = oracle.causal_recurrent(q, k, v)
    nc = oracle.noncausal_linear(q, k, v)
    np.testing.assert_allclose(c[0, 0], v[0, 0], rtol=1e-14)       # out_0 = v_0
    np.testing.assert_allclose(c[0, -1], nc[0, -1], rtol=1e-12)     # last row sees every key


def test_rows_helper_matches_full_forms():
    q, k, v = _rand(8, 40, 5)
    idx = np.array([0, 3, 39, 17])
    np.testing.assert_allclose(oracle.rows(q[0], k[0], v[0], idx, causal=False),
                               oracle.noncausal_linear(q, k, v)[0][idx], rtol=1e-12)
    np.testing.assert_allclose(oracle.rows(q[0], k[0], v[0], idx, causal=True),
                               oracle.causal_recurrent(q, k, v)[0][idx], rtol=1e-12)


# --------------------------------------------------------------------- invariants
def test_convex_combination_bound():
    # A4: with non-negative weights the output stays within the range of V's values
    q, k, v = _rand(9, 80, 6, scale=2.0)
    nc = oracle.noncausal_linear(q, k, v)[0]
    lo, hi = v[0].min(axis=0), v[0].max(axis=0)
    assert np.all(nc >= lo - 1e-12) and np.all(nc <= hi + 1e-12)
    c = oracle.causal_recurrent(q, k, v)[0]
    for i in range(80):
        lo, hi = v[0, :i + 1].min(axis=0), v[0, :i + 1].max(axis=0)
        assert np.all(c[i] >= lo - 1e-12) and np.all(c[i] <= hi + 1e-12)


def test_ones_vector_and_constant_rows():
    # Q(K^T 1) = (QK^T) 1: V = 1 gives out = 1; a constant value row v gives out = v
    q, k, _ = _rand(11, 33, 7)
    ones = np.ones_like(q)
    for f in (lambda V: oracle.noncausal_linear(q, k, V),
              lambda V: oracle.causal_recurrent(q, k, V),
              lambda V: oracle.causal_chunked(q, k, V, 8)):
        np.testing.assert_allclose(f(ones), 1.0, rtol=1e-13)
        row = np.linspace(-2, 3, 7)
        np.testing.assert_allclose(f(np.broadcast_to(row, q.shape).copy()),
                                   np.broadcast_to(row, q.shape), rtol=1e-12, atol=1e-13)


def test_denominator_positive():
    q, k, v = _rand(12, 64, 16, scale=20.0)      # large magnitudes, phi spans many decades
    _, kv, z = oracle.noncausal_linear(q, k, v, return_state=True)
    den = oracle.phi(q[0]) @ z[0]
    assert np.all(den > 0) and np.all(z > 0)


def test_permutation_invariance():
    q, k, v = _rand(13, 60, 6)
    perm = np.random.default_rng(0).permutation(60)
    a = oracle.noncausal_linear(q, k, v)
    b = oracle.noncausal_linear(q, k[:, perm], v[:, perm])
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)
    c = oracle.noncausal_linear(q[:, perm], k, v)
    np.testing.assert_allclose(c, a[:, perm], rtol=1e-12, atol=1e-14)


def test_linearity_in_v():
    q, k, v1 = _rand(14, 45, 5)
    _, _, v2 = _rand(15, 45, 5)
    al, be = 0.7, -1.9
    for f in (oracle.noncausal_linear, oracle.causal_recurrent):
        np.testing.assert_allclose(f(q, k, al * v1 + be * v2), al * f(q, k, v1) + be * f(q, k, v2),
                                   rtol=1e-11, atol=1e-12)


# --------------------------------------------------------------------- decode
def test_decode_from_zero_reproduces_causal():
    n, d = 37, 6
    q, k, v = _rand(16, n, d, bh=3)
    ref = oracle.causal_recurrent(q, k, v)
    S = np.zeros((3, d, d))
    z = np.zeros((3, d))
    for t in range(n):
        out, S, z = oracle.decode_step(q[:, t], k[:, t], v[:, t], S, z)
        np.testing.assert_allclose(out, ref[:, t], rtol=1e-12, atol=1e-14)


def test_decode_after_prior_equals_causal_on_concatenation():
    prior, steps, d = 40, 12, 5
    q, k, v = _rand(17, prior + steps, d, bh=2)
    S, z = oracle.state_accumulate(k[:, :prior], v[:, :prior])
    ref = oracle.causal_recurrent(q, k, v)
    for t in range(steps):
        out, S, z = oracle.decode_step(q[:, prior + t], k[:, prior + t], v[:, prior + t], S, z)
        np.testing.assert_allclose(out, ref[:, prior + t], rtol=1e-12, atol=1e-14)


def test_causal_from_state_splits():
    # forward(n) == forward(n1) then forward(n2) with the state carried
    n1, n2, d = 23, 31, 6
    q, k, v = _rand(18, n1 + n2, d, bh=2)
    full, Sf, zf = oracle.causal_recurrent(q, k, v, return_state=True)
    a, S1, z1 = oracle.causal_recurrent(q[:, :n1], k[:, :n1], v[:, :n1], return_state=True)
    b, S2, z2 = oracle.causal_recurrent(q[:, n1:], k[:, n1:], v[:, n1:], s0=S1, z0=z1,
                                        return_state=True)
    np.testing.assert_allclose(np.concatenate([a, b], axis=1), full, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(S2, Sf, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(z2, zf, rtol=1e-13)


def test_causal_from_state_equals_masked_pairwise_form_on_concatenation():
    # an initial state that sums prior tokens stands exactly for those tokens: the outputs are
    # the masked pairwise form's rows over [prior | tokens], and the final state is the plain
    # sum over all of them
    prior, n, d = 13, 21, 5
    q, k, v = _rand(22, prior + n, d, bh=2)
    S0, z0 = oracle.state_from_tokens_matmul(k[:, :prior], v[:, :prior])
    out, Sn, zn = oracle.causal_recurrent(q[:, prior:], k[:, prior:], v[:, prior:], s0=S0, z0=z0,
                                          return_state=True)
    ref = oracle.quadratic(q, k, v, causal=True)
    np.testing.assert_allclose(out, ref[:, prior:], rtol=1e-11, atol=1e-13)
    Sa, za = oracle.state_from_tokens_matmul(k, v)
    np.testing.assert_allclose(Sn, Sa, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(zn, za, rtol=1e-13)
    # no tokens: the final state is the initial one
    _, Se, ze = oracle.causal_recurrent(q[:, :0], k[:, :0], v[:, :0], s0=S0, z0=z0, return_state=True)
    assert np.array_equal(Se, S0) and np.array_equal(ze, z0)


def test_decode_resume_bitwise():
    # the state is the whole checkpoint: 6 + save/restore + 6 steps == 12 steps
    d = 4
    q, k, v = _rand(19, 12, d)
    S = np.zeros((1, d, d))
    z = np.zeros((1, d))
    outs = []
    for t in range(12):
        o, S, z = oracle.decode_step(q[:, t], k[:, t], v[:, t], S, z)
        outs.append(o)
    S2 = np.zeros((1, d, d))
    z2 = np.zeros((1, d))
    outs2 = []
    for t in range(6):
        o, S2, z2 = oracle.decode_step(q[:, t], k[:, t], v[:, t], S2, z2)
        outs2.append(o)
    saved = (S2.tobytes(), z2.tobytes())
    S3 = np.frombuffer(saved[0]).reshape(1, d, d).copy()
    z3 = np.frombuffer(saved[1]).reshape(1, d).copy()
    for t in range(6, 12):
        o, S3, z3 = oracle.decode_step(q[:, t], k[:, t], v[:, t], S3, z3)
        outs2.append(o)
    assert np.array_equal(np.array(outs), np.array(outs2))
    assert np.array_equal(S, S3) and np.array_equal(z, z3)


def test_state_size_matches_accounting():
    from oracle.accounting import linear_state_bytes
    # the state is D*d + D fp32 values whatever the sequence length
    assert linear_state_bytes(64) == 16640
    assert linear_state_bytes(128) == 66048
    _, kv, z = oracle.noncausal_linear(*_rand(20, 10, 64), return_state=True)
    assert (kv[0].size + z[0].size) * 4 == 16640


def test_state_matmul_equals_loop():
    _, k, v = _rand(21, 50, 8, bh=3)
    S1, z1 = oracle.state_accumulate(k, v)
    S2, z2 = oracle.state_from_tokens_matmul(k, v)
    np.testing.assert_allclose(S2, S1, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(z2, z1, rtol=1e-13)


def _classes(x):
    """0 finite, 1 +inf, 2 -inf, 3 NaN."""
    c = np.zeros(x.shape, dtype=np.int8)
    c[np.isposinf(x)] = 1
    c[np.isneginf(x)] = 2
    c[np.isnan(x)] = 3
    return c


def test_nonfinite_inputs_follow_the_formula():
    """IEEE behaviour of eq. Attention_i ("Linear attention: reordering the matmuls") on NaN and
    +-inf entries, derived by hand: phi(-inf) = e^-inf = 0 drops a feature; phi(+inf) = +inf and
    phi(NaN) = NaN; a query whose features are all -inf has phi(q) = 0, hence 0/0.  The three
    forms (non-causal, causal recurrence, decode) must give exactly these classes."""
    n, d = 6, 4
    rng = np.random.default_rng(77)
    q, k, v = (rng.standard_normal((1, 1, n, d)) * 0.5 for _ in range(3))
    q[0, 0, 1, :] = -np.inf      # query 1: phi(q) = 0 -> 0/0 in every column
    q[0, 0, 2, 0] = -np.inf      # query 2: one feature drops out, row stays finite
    k[0, 0, 3, 2] = np.nan       # key 3: NaN reaches every query that sees it
    v[0, 0, 4, 1] = np.inf       # value (4, 1): +inf in column 1 of every query that sees key 4
    with np.errstate(invalid="ignore", divide="ignore", over="ignore"):
        nc = oracle.noncausal_linear(q, k, v)
        ca = oracle.causal_recurrent(q, k, v)
        S, z = np.zeros((1, 1, d, d)), np.zeros((1, 1, d))
        dec = []
        for t in range(n):
            o, S, z = oracle.decode_step(q[:, :, t], k[:, :, t], v[:, :, t], S, z)
            dec.append(o)
        dec = np.stack(dec, axis=2)
    # non-causal: every query sees key 3 (NaN) -> every element NaN
    assert (_classes(nc) == 3).all()
    # causal: rows 0 and 2 see keys 0..i < 3 -> finite; row 1 is 0/0; rows 3.. see key 3 -> NaN
    exp = np.zeros((n, d), dtype=np.int8)
    exp[1, :] = 3
    exp[3:, :] = 3
    assert np.array_equal(_classes(ca)[0, 0], exp)
    assert np.array_equal(_classes(dec)[0, 0], exp)
    # the finite causal rows equal the same rows without the non-finite entries further on
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    k2[0, 0, 3, 2] = 0.0
    v2[0, 0, 4, 1] = 0.0
    with np.errstate(invalid="ignore", divide="ignore"):
        ca2 = oracle.causal_recurrent(q2, k2, v2)
    assert np.array_equal(ca[0, 0, [0, 2]], ca2[0, 0, [0, 2]])
    # +inf in a value without the NaN key: column 1 of rows >= 4 is +inf (positive weights), the
    # other columns stay finite
    with np.errstate(invalid="ignore", divide="ignore", over="ignore"):
        ca3 = oracle.causal_recurrent(q, k2, v)
    c3 = _classes(ca3)[0, 0]
    assert (c3[4:, 1] == 1).all() and (c3[4:, [0, 2, 3]] == 0).all() and (c3[[0, 2, 3], :] == 0).all()
    assert (c3[1, :] == 3).all()
