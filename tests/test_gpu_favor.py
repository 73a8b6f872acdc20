"""GPU parity of the FAVOR+ kernels (through the C ABI) against the fp64 oracle (oracle/favor.py).

Inputs: q, k, v ~ N(0, 1) in bf16 (the feature scale d^(-1/4) gives softmax-like logits), the
projection i.i.d. N(0, 1) rows in bf16 or an orthogonal projection from the oracle rounded to
bf16; the oracle computes with exactly those bf16 values in fp64.  Bar: bf16 normwise 2e-2 on
the outputs; the decode state (fp32 arithmetic) within 1e-4 of fp64 after its log-scale is
applied.
"""
import math

import numpy as np
import pytest

from gpu_util import f64, from_dev, need_gpu, say, to_dev
from metrics import TOL_BF16, normwise_err, rowwise_err
from oracle import favor
from seeded_inputs import encode, orf_draws, projection

pytestmark = pytest.mark.gpu

TOL_STATE = 1e-4


@pytest.fixture(scope="module")
def ea():
    need_gpu()
    import efficient_attention_amd
    return efficient_attention_amd


def _inputs(seed, shape, amp=1.0):
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 7])))
    return tuple(encode(amp * g.standard_normal(shape, dtype=np.float32), "bf16") for _ in range(3))


def _proj(seed, m, d, kind):
    if kind == "iid":
        return projection(seed, m, d, "bf16")
    g, ln = orf_draws(seed, m, d)
    return encode(favor.orf_projection(g, ln)[:m].astype(np.float32), "bf16")


NC_CASES = [
    # B, H, n, d, m, projection
    (1, 2, 1000, 64, 256, "iid"),     # several tiles and slices, ragged tail
    (2, 3, 333, 64, 128, "orf"),
    (1, 1, 31, 64, 64, "iid"),        # less than one tile
    (1, 1, 1, 64, 256, "orf"),        # one token
    (1, 2, 2500, 128, 64, "iid"),     # two query workgroups per head
    (2, 1, 777, 128, 128, "orf"),
    (2, 4, 4096, 64, 256, "iid"),     # 8 heads: the XCD mapping of the output kernel
]


@pytest.mark.parametrize("B,H,n,d,m,kind", NC_CASES)
def test_favor_noncausal_vs_oracle(ea, B, H, n, d, m, kind):
    q, k, v = _inputs(100 + n + d + m, (B, H, n, d))
    w = _proj(200 + m + d, m, d, kind)
    scale = d ** -0.25
    say("favor noncausal", B, H, n, d, m, kind)
    out = from_dev(ea.la_favor_forward_noncausal(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"),
                                                 to_dev(w, "bf16"), scale), "bf16")
    ref = favor.noncausal(f64(q, "bf16"), f64(k, "bf16"), f64(v, "bf16"), f64(w, "bf16"), scale)
    err = normwise_err(out, ref)
    say("  err", err)
    assert err <= TOL_BF16


@pytest.mark.parametrize("amp,scale", [(4.0, 64 ** -0.25), (3.0, 1.0)])
def test_favor_noncausal_exponents_beyond_fp32(ea, amp, scale):
    """Large inputs: the feature exponents reach -300 and below, where exp underflows in fp32 and
    the feature values differ by far more than fp32's range; the log-scale keeps the result."""
    B, H, n, d, m = 1, 2, 700, 64, 128
    q, k, v = _inputs(31, (B, H, n, d), amp)
    w = _proj(32, m, d, "iid")
    Q, K, V, Wd = f64(q, "bf16"), f64(k, "bf16"), f64(v, "bf16"), f64(w, "bf16")
    xs = scale * K
    u = xs @ Wd.T - 0.5 * np.sum(xs * xs, axis=-1, keepdims=True)
    assert u.min() < -100 and u.max() - u.min() > 88  # beyond fp32's exp: what the case claims
    say("favor noncausal large exponents", amp, scale)
    out = from_dev(ea.la_favor_forward_noncausal(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"),
                                                 to_dev(w, "bf16"), scale), "bf16")
    ref = favor.noncausal(Q, K, V, Wd, scale)
    assert np.all(np.isfinite(ref))
    err = normwise_err(out, ref)
    say("  err", err)
    assert err <= TOL_BF16


def _decode_run(ea, torch, q, k, v, w, scale, S, z, c):
    """Steps over axis -2 of q, k, v ([BH..., steps, d]); returns outputs [..., steps, d]."""
    steps = q.shape[-2]
    outs = []
    tw = to_dev(w, "bf16")
    for i in range(steps):
        o = ea.la_favor_decode_step(to_dev(np.ascontiguousarray(q[..., i, :]), "bf16"),
                                    to_dev(np.ascontiguousarray(k[..., i, :]), "bf16"),
                                    to_dev(np.ascontiguousarray(v[..., i, :]), "bf16"), tw, S, z, c, scale)
        outs.append(from_dev(o, "bf16"))
    return np.stack(outs, axis=-2)


def _true_state(torch, S, z, c):
    e = np.exp(c.cpu().numpy().astype(np.float64))
    return S.cpu().numpy().astype(np.float64) * e[..., None, None], z.cpu().numpy().astype(np.float64) * e[..., None]


@pytest.mark.parametrize("d,m", [(64, 256), (128, 128), (64, 64), (128, 64)])
def test_favor_decode_from_empty_state(ea, d, m):
    torch = pytest.importorskip("torch")
    B, H, steps = 3, 2, 40
    q, k, v = _inputs(300 + d + m, (B, H, steps, d))
    w = _proj(301 + m, m, d, "orf")
    scale = d ** -0.25
    S = torch.zeros((B, H, m, d), dtype=torch.float32, device="cuda")
    z = torch.zeros((B, H, m), dtype=torch.float32, device="cuda")
    c = torch.full((B, H), -math.inf, dtype=torch.float32, device="cuda")
    say("favor decode", d, m)
    outs = _decode_run(ea, torch, q, k, v, w, scale, S, z, c)
    Q, K, V, Wd = f64(q, "bf16"), f64(k, "bf16"), f64(v, "bf16"), f64(w, "bf16")
    ref, Sref, zref = favor.causal_recurrent(Q, K, V, Wd, scale, return_state=True)
    for i in range(steps):
        assert normwise_err(outs[..., i, :], ref[..., i, :], head_axes_last=1) <= TOL_BF16, i
    St, zt = _true_state(torch, S, z, c)
    assert normwise_err(St, Sref) <= TOL_STATE
    assert normwise_err(zt, zref, head_axes_last=1) <= TOL_STATE


def test_favor_decode_from_given_state_and_scale_jumps(ea):
    """Start from a prefix state handed over with an arbitrary log-scale, then keys whose
    exponents exceed everything before push the running maximum up (the rescale path)."""
    torch = pytest.importorskip("torch")
    B, H, d, m, prior, steps = 2, 2, 64, 128, 300, 12
    pq, pk, pv = _inputs(400, (B, H, prior, d))
    q, k, v = _inputs(401, (B, H, steps, d))
    w = _proj(402, m, d, "iid")
    scale = d ** -0.25
    Wd = f64(w, "bf16")
    # keys along rows of W at the norm that maximises their exponent (|w|^2 / 2, about d / 2):
    # far above the prefix's, so the log-scale must move
    k = f64(k, "bf16").astype(np.float32)
    for i in (4, 7, 10):
        k[:, :, i, :] = (Wd[i] / scale).astype(np.float32)
    k = encode(k, "bf16")
    S0, z0 = favor.state(f64(pk, "bf16"), f64(pv, "bf16"), Wd, scale)
    c0 = np.log(z0.max(axis=-1)) + 1.5  # any log-scale: stored values exp(-c0) times the true ones
    S = torch.from_numpy((S0 * np.exp(-c0)[..., None, None]).astype(np.float32)).cuda()
    z = torch.from_numpy((z0 * np.exp(-c0)[..., None]).astype(np.float32)).cuda()
    c = torch.from_numpy(c0.astype(np.float32)).cuda()
    c_start = c.clone()
    say("favor decode from state")
    outs = _decode_run(ea, torch, q, k, v, w, scale, S, z, c)
    ref, Sref, zref = favor.causal_recurrent(f64(q, "bf16"), f64(k, "bf16"), f64(v, "bf16"), Wd, scale,
                                             s0=S0, z0=z0, return_state=True)
    for i in range(steps):
        assert normwise_err(outs[..., i, :], ref[..., i, :], head_axes_last=1) <= TOL_BF16, i
    assert bool((c > c_start).all())  # the scale moved
    St, zt = _true_state(torch, S, z, c)
    assert normwise_err(St, Sref) <= TOL_STATE
    assert normwise_err(zt, zref, head_axes_last=1) <= TOL_STATE


def test_favor_decode_is_bitwise_reproducible(ea):
    torch = pytest.importorskip("torch")
    B, H, d, m = 4, 8, 128, 128
    q, k, v = _inputs(500, (B, H, 1, d))
    w = _proj(501, m, d, "iid")
    res = []
    for _ in range(2):
        S = torch.zeros((B, H, m, d), dtype=torch.float32, device="cuda")
        z = torch.zeros((B, H, m), dtype=torch.float32, device="cuda")
        c = torch.full((B, H), -math.inf, dtype=torch.float32, device="cuda")
        o = _decode_run(ea, torch, q, k, v, w, 0.3, S, z, c)
        res.append((o, S.cpu().numpy(), z.cpu().numpy(), c.cpu().numpy()))
    for a, b in zip(res[0], res[1]):
        assert np.array_equal(a, b)


# ----------------------------------------------------------------------------- causal
CA_CASES = [
    # B, H, n, d, m, projection
    (1, 2, 1000, 64, 256, "iid"),     # 16 segments per head: leading-segment sums on every cut
    (2, 3, 333, 64, 128, "orf"),
    (1, 1, 31, 64, 64, "iid"),        # less than one chunk
    (1, 1, 1, 128, 128, "orf"),       # one token
    (1, 2, 2500, 128, 64, "iid"),
    (2, 1, 777, 128, 128, "orf"),
    (2, 4, 4096, 64, 256, "iid"),
    (64, 4, 200, 128, 128, "iid"),    # one segment per head
]


def _causal_ref(Q, K, V, Wd, scale):
    if Q.shape[-2] <= 2048:
        return favor.quadratic(Q, K, V, Wd, scale, causal=True)
    return favor.causal_recurrent(Q, K, V, Wd, scale)


@pytest.mark.parametrize("B,H,n,d,m,kind", CA_CASES)
def test_favor_causal_vs_oracle(ea, B, H, n, d, m, kind):
    q, k, v = _inputs(600 + n + d + m, (B, H, n, d))
    w = _proj(700 + m + d, m, d, kind)
    scale = d ** -0.25
    say("favor causal", B, H, n, d, m, kind)
    out = from_dev(ea.la_favor_forward_causal(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"),
                                              to_dev(w, "bf16"), scale), "bf16")
    ref = _causal_ref(f64(q, "bf16"), f64(k, "bf16"), f64(v, "bf16"), f64(w, "bf16"), scale)
    err = rowwise_err(out, ref)
    say("  err", err)
    assert err <= TOL_BF16


@pytest.mark.parametrize("amp,scale", [(4.0, 64 ** -0.25), (3.0, 1.0)])
def test_favor_causal_exponents_beyond_fp32(ea, amp, scale):
    B, H, n, d, m = 1, 2, 700, 64, 128
    q, k, v = _inputs(41, (B, H, n, d), amp)
    w = _proj(42, m, d, "iid")
    say("favor causal large exponents", amp, scale)
    out = from_dev(ea.la_favor_forward_causal(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"),
                                              to_dev(w, "bf16"), scale), "bf16")
    ref = favor.quadratic(f64(q, "bf16"), f64(k, "bf16"), f64(v, "bf16"), f64(w, "bf16"), scale, causal=True)
    assert np.all(np.isfinite(ref))
    err = rowwise_err(out, ref)
    say("  err", err)
    assert err <= TOL_BF16


@pytest.mark.parametrize("n,d,m", [(1000, 64, 256), (777, 128, 128), (64, 64, 64)])
def test_favor_causal_final_state_then_decode(ea, n, d, m):
    """Prefill with the final state, hand it to the decode step: outputs and the state after the
    decode steps follow the recurrence over all n + steps tokens."""
    torch = pytest.importorskip("torch")
    B, H, steps = 2, 2, 8
    q, k, v = _inputs(800 + n, (B, H, n + steps, d))
    w = _proj(801 + m, m, d, "orf")
    scale = d ** -0.25
    tw = to_dev(w, "bf16")
    pre = lambda x: to_dev(np.ascontiguousarray(x[:, :, :n]), "bf16")
    say("favor causal final state", n, d, m)
    out, S, z, c = ea.la_favor_forward_causal(pre(q), pre(k), pre(v), tw, scale, final_state=True)
    Q, K, V, Wd = f64(q, "bf16"), f64(k, "bf16"), f64(v, "bf16"), f64(w, "bf16")
    ref, Sref, zref = favor.causal_recurrent(Q, K, V, Wd, scale, return_state=True)
    _, Spre, zpre = favor.causal_recurrent(Q[:, :, :n], K[:, :, :n], V[:, :, :n], Wd, scale, return_state=True)
    assert rowwise_err(from_dev(out, "bf16"), ref[:, :, :n]) <= TOL_BF16
    St, zt = _true_state(torch, S, z, c)
    assert normwise_err(St, Spre) <= TOL_BF16
    assert normwise_err(zt, zpre, head_axes_last=1) <= TOL_BF16
    outs = _decode_run(ea, torch, q[:, :, n:], k[:, :, n:], v[:, :, n:], w, scale, S, z, c)
    for i in range(steps):
        assert normwise_err(outs[..., i, :], ref[:, :, n + i], head_axes_last=1) <= TOL_BF16, i
    St, zt = _true_state(torch, S, z, c)
    assert normwise_err(St, Sref) <= TOL_BF16


def test_favor_causal_empty_sequence_state(ea):
    torch = pytest.importorskip("torch")
    B, H, d, m = 2, 3, 64, 128
    q = torch.empty((B, H, 0, d), dtype=torch.bfloat16, device="cuda")
    w = to_dev(_proj(900, m, d, "iid"), "bf16")
    Sn = torch.full((B, H, m, d), 7.0, dtype=torch.float32, device="cuda")
    zn = torch.full((B, H, m), 7.0, dtype=torch.float32, device="cuda")
    cn = torch.zeros((B, H), dtype=torch.float32, device="cuda")
    say("favor causal empty")
    ea.la_favor_forward_causal(q, q, q, w, 0.3, final_state=True, Sn=Sn, zn=zn, cn=cn)
    torch.cuda.synchronize()
    assert float(Sn.abs().max()) == 0.0 and float(zn.abs().max()) == 0.0
    assert bool(torch.isinf(cn).all()) and float(cn.max()) < 0


def test_favor_causal_last_row_equals_noncausal(ea):
    B, H, n, d, m = 2, 2, 1500, 64, 256
    q, k, v = _inputs(910, (B, H, n, d))
    w = _proj(911, m, d, "iid")
    tq, tk, tv, tw = (to_dev(x, "bf16") for x in (q, k, v, w))
    say("favor causal vs noncausal last row")
    oc = from_dev(ea.la_favor_forward_causal(tq, tk, tv, tw, 0.35), "bf16")
    on = from_dev(ea.la_favor_forward_noncausal(tq, tk, tv, tw, 0.35), "bf16")
    assert normwise_err(oc[:, :, -1:], on[:, :, -1:]) <= TOL_BF16


@pytest.mark.parametrize("B,H,n,d,m", [(1, 2, 1000, 128, 128), (2, 3, 333, 64, 128), (1, 1, 129, 128, 64),
                                       (2, 4, 4096, 128, 128), (3, 2, 77, 64, 64)])
def test_favor_causal_chunk128_vs_oracle(ea, B, H, n, d, m):
    q, k, v = _inputs(1000 + n + d + m, (B, H, n, d))
    w = _proj(1001 + m + d, m, d, "orf")
    scale = d ** -0.25
    tq, tk, tv, tw = (to_dev(x, "bf16") for x in (q, k, v, w))
    say("favor causal chunk 128", B, H, n, d, m)
    out = from_dev(ea.la_favor_forward_causal(tq, tk, tv, tw, scale, chunk=128), "bf16")
    ref = _causal_ref(f64(q, "bf16"), f64(k, "bf16"), f64(v, "bf16"), f64(w, "bf16"), scale)
    err = rowwise_err(out, ref)
    say("  err", err)
    assert err <= TOL_BF16
    # chunk 64 and chunk 128 agree to rounding
    o64 = from_dev(ea.la_favor_forward_causal(tq, tk, tv, tw, scale, chunk=64), "bf16")
    assert rowwise_err(out, o64) <= TOL_BF16


def test_favor_causal_chunk128_final_state_and_large_exponents(ea):
    torch = pytest.importorskip("torch")
    B, H, n, d, m = 1, 2, 700, 128, 128
    q, k, v = _inputs(1100, (B, H, n, d), 2.0)  # exponents -425..-104 (fp64 still holds the products)
    w = _proj(1101, m, d, "iid")
    say("favor causal chunk 128 large exponents + state")
    out, S, z, c = ea.la_favor_forward_causal(*(to_dev(x, "bf16") for x in (q, k, v, w)), 1.0, chunk=128,
                                              final_state=True)
    Q, K, V, Wd = f64(q, "bf16"), f64(k, "bf16"), f64(v, "bf16"), f64(w, "bf16")
    ref = favor.quadratic(Q, K, V, Wd, 1.0, causal=True)
    assert rowwise_err(from_dev(out, "bf16"), ref) <= TOL_BF16
    _, Sref, zref = favor.noncausal(Q, K, V, Wd, 1.0, return_state=True)
    St, zt = _true_state(torch, S, z, c)
    assert normwise_err(St, Sref) <= TOL_BF16
    assert normwise_err(zt, zref, head_axes_last=1) <= TOL_BF16


# ----------------------------------------------------------------------------- invariants
@pytest.mark.parametrize("form", ["noncausal", "causal"])
def test_favor_forward_invariants_and_determinism(ea, form):
    """Properties every positive feature map gives eq. Attention_i, checked on the FAVOR+ forwards:
    outputs are convex combinations of value rows (within each column's range of the keys seen),
    a constant value row comes back unchanged, and two runs are bitwise equal."""
    B, H, n, d, m = 2, 3, 700, 64, 256
    q, k, v = _inputs(900 + (form == "causal"), (B, H, n, d))
    w = _proj(901, m, d, "orf")
    scale = d ** -0.25
    tq, tk, tv, tw = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), to_dev(w, "bf16")
    fwd = ea.la_favor_forward_noncausal if form == "noncausal" else ea.la_favor_forward_causal
    say("favor invariants", form)
    a = from_dev(fwd(tq, tk, tv, tw, scale), "bf16")
    b = from_dev(fwd(tq, tk, tv, tw, scale), "bf16")
    assert np.array_equal(a, b)
    V = f64(v, "bf16")
    if form == "noncausal":
        lo = V.min(axis=2, keepdims=True)
        hi = V.max(axis=2, keepdims=True)
    else:
        lo = np.minimum.accumulate(V, axis=2)
        hi = np.maximum.accumulate(V, axis=2)
    span = np.abs(V).max()
    slack = 2e-2 * span  # bf16 features and outputs
    assert np.all(a >= lo - slack) and np.all(a <= hi + slack)
    # a constant value row c: every output row is c
    row = np.linspace(-1.5, 2.0, d, dtype=np.float32)
    vc = encode(np.broadcast_to(row, (B, H, n, d)).copy(), "bf16")
    c = from_dev(fwd(tq, tk, to_dev(vc, "bf16"), tw, scale), "bf16")
    np.testing.assert_allclose(c, np.broadcast_to(f64(vc, "bf16")[0, 0, 0], c.shape), rtol=1e-2, atol=1e-2)
