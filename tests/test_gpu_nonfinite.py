"""Non-finite inputs: NaN, +inf and -inf in q, k and v, for the non-causal, causal and decode
forms in fp32 and bf16, against the oracle's fp64 evaluation of eq. Attention_i ("Efficient
Transformers: Linear Attention and Flash Attention", section "Linear attention: reordering the
matmuls"; the recurrence of "The recurrent view").

What the formula gives, and the GPU must give too (every output element in the same class:
finite, +inf, -inf or NaN; finite rows within the usual bar):
  * phi(-inf) = exp(-inf) = 0: a -inf feature drops out; a query whose features are all -inf
    has 0/0 (NaN);
  * phi(NaN) = NaN and phi(+inf) = +inf: a query with one makes its row NaN (inf/inf or NaN);
    a key with one makes every query that sees it NaN (all rows for the non-causal form, rows
    j.. for the causal form, every later step for decode);
  * a value entry +-inf or NaN at key j reaches column c of every query that sees j.

One documented difference of the chunked causal kernels: a non-finite value at key j also
reaches column c of the queries in j's chunk that come before j, because the masked weights are
zeros that multiply it inside the chunk's value product (0 * inf = NaN).  The exact comparison
puts the value entries at chunk starts (no earlier query in the chunk); a separate test pins the
difference to that chunk and that column.
"""
import numpy as np
import pytest

import oracle
from gpu_util import f64, from_dev, need_gpu, say, to_dev
from metrics import TOL_BF16, TOL_F32, form_err
from seeded_inputs import encode, random_inputs

pytestmark = pytest.mark.gpu

TOL = {"f32": TOL_F32, "bf16": TOL_BF16}
N, D = 300, 64


@pytest.fixture(scope="module")
def ea():
    need_gpu()
    import efficient_attention_amd
    return efficient_attention_amd


def _classes(x):
    """0 finite, 1 +inf, 2 -inf, 3 NaN."""
    c = np.zeros(x.shape, dtype=np.int8)
    c[np.isposinf(x)] = 1
    c[np.isneginf(x)] = 2
    c[np.isnan(x)] = 3
    return c


def _inputs(dtype):
    """Five heads of N tokens, each with its own non-finite entries (value entries at rows 0, 128
    and 256: chunk starts for chunks of 64 and 128)."""
    q, k, v = random_inputs(321, (1, 5, N, D), dtype, 1.0 / np.sqrt(D))
    q, k, v = (f64(x, dtype).astype(np.float32) for x in (q, k, v))
    # head 0: queries -- NaN, +inf, one -inf feature, all features -inf
    q[0, 0, 10, 5] = np.nan
    q[0, 0, 20, 7] = np.inf
    q[0, 0, 40, 3] = -np.inf
    q[0, 0, 30, :] = -np.inf
    # head 1: a NaN key feature at row 150
    k[0, 1, 150, 4] = np.nan
    # head 2: value entries +inf (row 256, column 9), NaN (row 128, column 2), -inf (row 0, column 11)
    v[0, 2, 256, 9] = np.inf
    v[0, 2, 128, 2] = np.nan
    v[0, 2, 0, 11] = -np.inf
    # head 3: a +inf key feature at row 64; a -inf key feature at row 70 (drops out)
    k[0, 3, 64, 0] = np.inf
    k[0, 3, 70, 1] = -np.inf
    # head 4: untouched
    return encode(q, dtype), encode(k, dtype), encode(v, dtype)


def _compare(form, g, r, dtype):
    cg, cr = _classes(g), _classes(r)
    bad = np.argwhere(cg != cr)
    assert bad.size == 0, "class mismatch at %s: gpu %s oracle %s" % (
        bad[:5].tolist(), [g[tuple(i)] for i in bad[:5]], [r[tuple(i)] for i in bad[:5]])
    rows = np.all(cr == 0, axis=-1)  # rows the formula keeps finite
    assert form_err(form, g[rows][None], r[rows][None]) <= TOL[dtype]
    return cr


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("form,chunk", [("noncausal", 0), ("causal", 64), ("causal", 128)])
def test_nonfinite_forward(ea, form, chunk, dtype):
    if form == "causal" and dtype == "f32" and D * chunk > 8192:
        pytest.skip("fp32 needs d * chunk <= 8192")
    q, k, v = _inputs(dtype)
    say("non-finite inputs", form, chunk, dtype)
    tq, tk, tv = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
    out = ea.la_forward_noncausal(tq, tk, tv) if form == "noncausal" else ea.la_forward_causal(tq, tk, tv, chunk=chunk)
    g = from_dev(out, dtype)
    Q, K, V = f64(q, dtype), f64(k, dtype), f64(v, dtype)
    with np.errstate(invalid="ignore", divide="ignore", over="ignore"):
        r = oracle.noncausal_linear(Q, K, V) if form == "noncausal" else oracle.causal_recurrent(Q, K, V)
    cr = _compare(form, g, r, dtype)
    # the formula's pattern, spelled out
    nan_rows = np.all(cr[0, 0] == 3, axis=-1)
    assert nan_rows[[10, 20, 30]].all() and not nan_rows[40] and not nan_rows[0]
    head1 = np.all(cr[0, 1] == 3, axis=-1)
    head3 = np.all(cr[0, 3] == 3, axis=-1)
    if form == "noncausal":
        assert head1.all() and head3.all()
        assert (cr[0, 2][:, 9] == 1).all() and (cr[0, 2][:, 2] == 3).all() and (cr[0, 2][:, 11] == 2).all()
    else:
        assert head1[150:].all() and not head1[:150].any()
        assert head3[64:].all() and not head3[:64].any()
        assert (cr[0, 2][256:, 9] == 1).all() and (cr[0, 2][:256, 9] == 0).all()
        assert (cr[0, 2][128:, 2] == 3).all() and (cr[0, 2][:128, 2] == 0).all()
        assert (cr[0, 2][:, 11] == 2).all()
    assert (cr[0, 4] == 0).all()


@pytest.mark.parametrize("dtype,chunk", [("f32", 64), ("bf16", 64), ("bf16", 128)])
def test_nonfinite_value_stays_in_its_chunk(ea, dtype, chunk):
    """The chunked kernels' one difference from the formula, bounded: a +inf value at key j
    (not a chunk start) may turn column c of the queries chunk_start(j)..j-1 NaN; every other
    element is exactly as the formula has it."""
    q, k, v = random_inputs(322, (1, 2, N, D), dtype, 1.0 / np.sqrt(D))
    v = f64(v, dtype).astype(np.float32)
    j, c = 200, 9
    v[0, 0, j, c] = np.inf
    v = encode(v, dtype)
    say("non-finite value inside a chunk", dtype, chunk)
    g = from_dev(ea.la_forward_causal(to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), chunk=chunk), dtype)
    with np.errstate(invalid="ignore", over="ignore"):
        r = oracle.causal_recurrent(f64(q, dtype), f64(k, dtype), f64(v, dtype))
    start = (j // chunk) * chunk
    cg, cr = _classes(g), _classes(r)
    diff = np.argwhere(cg != cr)
    for (_, h, i, col) in diff:
        assert h == 0 and col == c and start <= i < j and cg[0, h, i, col] == 3, (h, i, col)
    rows = np.all((cr == 0) & (cg == 0), axis=-1)
    assert form_err("causal", g[rows][None], r[rows][None]) <= TOL[dtype]


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128)])
def test_nonfinite_decode(ea, dtype, d):
    import torch
    B, H, steps = 1, 4, 6
    q, k, v = random_inputs(323, (B, H, steps, d), dtype, 1.0 / np.sqrt(d))
    q, k, v = (f64(x, dtype).astype(np.float32) for x in (q, k, v))
    q[0, 0, 3, 1] = np.inf            # one step of head 0 reads with a +inf feature
    k[0, 1, 2, 4] = np.nan            # head 1 folds in a NaN key at step 2
    v[0, 2, 1, 9] = np.inf            # head 2: +inf value at step 1, column 9
    k[0, 3, 0, :] = -np.inf           # head 3: first key drops out entirely (0/0 at step 0)
    q, k, v = encode(q, dtype), encode(k, dtype), encode(v, dtype)
    S = torch.zeros((B, H, d, d), dtype=torch.float32, device="cuda")
    z = torch.zeros((B, H, d), dtype=torch.float32, device="cuda")
    Sr, zr = np.zeros((B, H, d, d)), np.zeros((B, H, d))
    say("non-finite decode", dtype, d)
    for t in range(steps):
        o = ea.la_decode_step(to_dev(q[:, :, t], dtype), to_dev(k[:, :, t], dtype), to_dev(v[:, :, t], dtype), S, z)
        with np.errstate(invalid="ignore", divide="ignore", over="ignore"):
            ro, Sr, zr = oracle.decode_step(f64(q[:, :, t], dtype), f64(k[:, :, t], dtype), f64(v[:, :, t], dtype), Sr, zr)
        g = from_dev(o, dtype)
        cg, cr = _classes(g), _classes(ro)
        assert np.array_equal(cg, cr), (t, cg, cr)
        fin = np.all(cr == 0, axis=-1)
        if fin.any():
            err = np.abs(g[fin] - ro[fin]).max(axis=-1) / np.abs(ro[fin]).max(axis=-1)
            assert err.max() <= TOL[dtype], (t, err)
    assert np.array_equal(_classes(S.cpu().numpy().astype(np.float64)), _classes(Sr))
    assert np.array_equal(_classes(z.cpu().numpy().astype(np.float64)), _classes(zr))


@pytest.mark.parametrize("form,chunk", [("noncausal", 0), ("causal", 64), ("causal", 128)])
def test_nonfinite_with_values_bf16_holds_exactly(ea, form, chunk):
    """fp32 inputs whose features and values bf16 holds exactly, so that the low half of every
    two-term split is the tiny stand-in, never zero: an infinite value must still give +-inf
    (inf * lo of an exact factor is inf, not NaN), as fp32 arithmetic and the formula do.
    q, k in {0, 0.5, 1, 1.5} (phi = x + 1 exact), v in {-2, -1, -0.5, 0.5, 1, 2}; +inf and -inf
    values at chunk starts of two heads."""
    rng = np.random.default_rng(324)
    shape = (1, 3, N, D)
    q = rng.choice(np.array([0.0, 0.5, 1.0, 1.5], np.float32), shape)
    k = rng.choice(np.array([0.0, 0.5, 1.0, 1.5], np.float32), shape)
    v = rng.choice(np.array([-2.0, -1.0, -0.5, 0.5, 1.0, 2.0], np.float32), shape)
    v[0, 0, 128, 5] = np.inf
    v[0, 1, 256, 7] = -np.inf
    say("non-finite with exact bf16 values", form, chunk)
    tq, tk, tv = to_dev(q, "f32"), to_dev(k, "f32"), to_dev(v, "f32")
    out = ea.la_forward_noncausal(tq, tk, tv) if form == "noncausal" else ea.la_forward_causal(tq, tk, tv, chunk=chunk)
    g = from_dev(out, "f32")
    Q, K, V = (x.astype(np.float64) for x in (q, k, v))
    with np.errstate(invalid="ignore", over="ignore"):
        r = oracle.noncausal_linear(Q, K, V) if form == "noncausal" else oracle.causal_recurrent(Q, K, V)
    cr = _compare(form, g, r, "f32")
    first = (0, 0) if form == "noncausal" else (128, 256)
    assert (cr[0, 0][first[0]:, 5] == 1).all() and (cr[0, 1][first[1]:, 7] == 2).all()
    assert (cr[0, 2] == 0).all()
