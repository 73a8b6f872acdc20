"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle, on seeded inputs.

Sizes here span several tiles and ragged tails while the oracle still finishes in seconds.
Error measure (tests/metrics.py): per row for causal outputs, per head otherwise; bars: fp32 <= 1e-4,
bf16 <= 2e-2.
"""
import zlib

import numpy as np
import pytest

import oracle
from metrics import TOL_BF16, TOL_F32, floored_elementwise_err, form_err, normwise_err, rowwise_err
from gpu_util import f64, from_dev, need_gpu, say, to_dev
from seeded_inputs import WORKLOADS, encode, forward_inputs, random_inputs

pytestmark = pytest.mark.gpu

TOL = {"f32": TOL_F32, "bf16": TOL_BF16}


@pytest.fixture(scope="module")
def ea():
    need_gpu()
    import efficient_attention_amd
    return efficient_attention_amd


def run_forward(ea, form, q, k, v, dtype, chunk=64):
    tq, tk, tv = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
    if form == "noncausal":
        out = ea.la_forward_noncausal(tq, tk, tv)
    else:
        out = ea.la_forward_causal(tq, tk, tv, chunk=chunk)
    return from_dev(out, dtype)


def oracle_forward(form, q, k, v, dtype):
    Q, K, V = f64(q, dtype), f64(k, dtype), f64(v, dtype)
    if form == "noncausal":
        return oracle.noncausal_linear(Q, K, V)
    return oracle.causal_recurrent(Q, K, V)


# ----------------------------------------------------------------------------- worked example
def _embedded_worked_example(d):
    """The pages' hand-worked 3-token example, fed through elu + 1 preimages: phi(0) = 1,
    phi(1) = 2, phi(2) = 3, phi(-1e4) = 0, and padded to width d with phi = 0 features and
    zero values."""
    Qp = np.full((3, d), -1e4, dtype=np.float32)
    Kp = np.full((3, d), -1e4, dtype=np.float32)
    V = np.zeros((3, d), dtype=np.float32)
    Qp[:, :2] = [[0, -1e4], [-1e4, 0], [0, 0]]
    Kp[:, :2] = [[1, 0], [0, 2], [0, 0]]
    V[:, :2] = [[1, 0], [0, 1], [1, 1]]
    return Qp[None, None], Kp[None, None], V[None, None]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
def test_worked_example_through_gpu(ea, dtype, d):
    q, k, v = (encode(x, dtype) for x in _embedded_worked_example(d))
    printed = np.array([[0.75, 0.5], [0.4, 0.8], [5 / 9, 2 / 3]])
    causal_rows = np.array([[1.0, 0.0], [0.25, 0.75], [5 / 9, 2 / 3]])
    tol = 1e-6 if dtype == "f32" else 4e-3
    say("worked example noncausal", dtype, d)
    g = run_forward(ea, "noncausal", q, k, v, dtype)
    np.testing.assert_allclose(g[0, 0, :, :2], printed, atol=tol)
    assert np.all(g[0, 0, :, 2:] == 0)
    for chunk in (64, 128):
        if dtype == "f32" and d * chunk > 8192:
            continue
        say("worked example causal", dtype, d, chunk)
        g = run_forward(ea, "causal", q, k, v, dtype, chunk)
        np.testing.assert_allclose(g[0, 0, :, :2], causal_rows, atol=tol)
    say("worked example decode", dtype, d)
    import torch
    S = torch.zeros((1, 1, d, d), dtype=torch.float32, device="cuda")
    z = torch.zeros((1, 1, d), dtype=torch.float32, device="cuda")
    for t in range(3):
        o = ea.la_decode_step(to_dev(q[:, :, t], dtype), to_dev(k[:, :, t], dtype),
                              to_dev(v[:, :, t], dtype), S, z)
        np.testing.assert_allclose(from_dev(o, dtype)[0, 0, :2], causal_rows[t], atol=tol)
    Sh = S.cpu().numpy()[0, 0]
    np.testing.assert_array_equal(Sh[:2, :2], [[3, 2], [2, 4]])   # the printed K^T V
    np.testing.assert_array_equal(z.cpu().numpy()[0, 0, :2], [4, 5])  # the printed key sum


# ----------------------------------------------------------------------------- small configs
def test_c1_noncausal_fp32_vs_linear_and_quadratic(ea):
    w = WORKLOADS["C1"]
    q, k, v = forward_inputs(w)
    say("C1", w)
    g = run_forward(ea, "noncausal", q, k, v, "f32")
    Q, K, V = f64(q, "f32"), f64(k, "f32"), f64(v, "f32")
    ref_lin = oracle.noncausal_linear(Q, K, V)
    ref_quad = oracle.quadratic(Q, K, V, causal=False)
    e1, e2 = normwise_err(g, ref_lin), normwise_err(g, ref_quad)
    print("C1 normwise err vs linear %.3e vs quadratic %.3e, floored elementwise %.3e"
          % (e1, e2, floored_elementwise_err(g, ref_lin)))
    assert e1 <= TOL_F32 and e2 <= TOL_F32


def test_c2_causal_fp32_chunk64(ea):
    w = WORKLOADS["C2"]
    q, k, v = forward_inputs(w)
    say("C2", w)
    g = run_forward(ea, "causal", q, k, v, "f32", chunk=64)
    ref = oracle_forward("causal", q, k, v, "f32")
    e = rowwise_err(g, ref)
    print("C2 rowwise err %.3e floored elementwise %.3e" % (e, floored_elementwise_err(g, ref)))
    assert e <= TOL_F32


# ----------------------------------------------------------------------------- shape sweep
CASES = []
for form in ("noncausal", "causal"):
    for dtype in ("f32", "bf16"):
        for d in (64, 128):
            for n in (1, 2, 3, 63, 64, 65, 127, 128, 129, 300, 1000):
                for chunk in ((64, 128) if form == "causal" else (0,)):
                    if form == "causal" and dtype == "f32" and d * chunk > 8192:
                        continue
                    CASES.append((form, dtype, d, n, chunk))


@pytest.mark.parametrize("form,dtype,d,n,chunk", CASES)
def test_shape_sweep(ea, form, dtype, d, n, chunk):
    B, H = 2, 3
    scale = 1.0 if dtype == "f32" else 1.0 / np.sqrt(d)
    q, k, v = random_inputs(zlib.crc32(repr((form, dtype, d, n, chunk)).encode()) % 100000, (B, H, n, d), dtype, scale)
    say(form, dtype, "d=%d n=%d chunk=%d" % (d, n, chunk))
    g = run_forward(ea, form, q, k, v, dtype, chunk or 64)
    ref = oracle_forward(form, q, k, v, dtype)
    e = form_err(form, g, ref)
    assert e <= TOL[dtype], e


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("B,H,n", [(2, 8, 5000), (1, 8, 4113), (3, 8, 2048)])
def test_noncausal_heads_in_multiples_of_8(ea, d, B, H, n):
    # B*H a multiple of 8 takes the output kernel's head-per-XCD workgroup order; several query
    # tiles per head, the last one ragged
    q, k, v = random_inputs(zlib.crc32(repr(("nc8", d, B, H, n)).encode()) % 100000, (B, H, n, d), "bf16",
                            1.0 / np.sqrt(d))
    say("noncausal bf16 B=%d H=%d n=%d d=%d" % (B, H, n, d))
    g = run_forward(ea, "noncausal", q, k, v, "bf16", 64)
    ref = oracle_forward("noncausal", q, k, v, "bf16")
    e = normwise_err(g, ref)
    assert e <= TOL["bf16"], e


@pytest.mark.parametrize("dtype,d,chunk", [("bf16", 64, 64), ("bf16", 128, 128), ("f32", 64, 64),
                                           ("bf16", 64, 128), ("bf16", 128, 64), ("f32", 128, 64)])
def test_causal_many_segments_ragged(ea, dtype, d, chunk):
    # one head: the sequence is cut into many segments whose state sums seed each other
    B, H, n = 1, 1, 16 * chunk + 37
    q, k, v = random_inputs(77 + d + chunk, (B, H, n, d), dtype, 1.0 / np.sqrt(d))
    assert ea.la_causal_workspace_bytes(B, H, n, d, chunk, 1 if dtype == "bf16" else 0) > 0
    say("causal segments", dtype, d, chunk, n)
    g = run_forward(ea, "causal", q, k, v, dtype, chunk)
    ref = oracle_forward("causal", q, k, v, dtype)
    assert rowwise_err(g, ref) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chunk_invariance(ea, dtype):
    d, n = 64, 777
    q, k, v = random_inputs(5, (2, 2, n, d), dtype, 1.0 / np.sqrt(d))
    ref = oracle_forward("causal", q, k, v, dtype)
    outs = []
    for chunk in (64, 128):
        say("chunk invariance", dtype, chunk)
        g = run_forward(ea, "causal", q, k, v, dtype, chunk)
        assert rowwise_err(g, ref) <= TOL[dtype]
        outs.append(g)
    assert rowwise_err(outs[0], outs[1]) <= TOL[dtype]


@pytest.mark.parametrize("form", ["noncausal", "causal"])
def test_invariants_on_gpu(ea, form):
    # V = 1 gives out = 1; a constant value row gives that row; out_0 = v_0 for causal
    d, n = 64, 200
    q, k, _ = random_inputs(9, (1, 2, n, d), "f32", 1.0)
    row = np.linspace(-2, 3, d, dtype=np.float32)
    v = np.broadcast_to(row, q.shape).copy()
    say("invariants", form)
    g = run_forward(ea, form, q, k, v, "f32")
    np.testing.assert_allclose(g, np.broadcast_to(row, g.shape), rtol=1e-5, atol=1e-5)
    if form == "causal":
        _, _, v2 = random_inputs(10, (1, 2, n, d), "f32", 1.0)
        g2 = run_forward(ea, form, q, k, v2, "f32")
        # out_0 = A_00 v_0 / A_00: every other factor cancels, so what remains is how v_0 itself
        # enters the products.  The fp32 kernels take it as a two-term bf16 split, hi + lo,
        # which holds v_0 to 2^-16 of its size (plain fp32 arithmetic would give 1e-7)
        np.testing.assert_allclose(g2[:, :, 0], v2[:, :, 0], rtol=2.0 ** -16 + 1e-6, atol=1e-6)


@pytest.mark.parametrize("form", ["noncausal", "causal"])
def test_extreme_inputs(ea, form):
    # large magnitudes: phi spans exp(-60) .. 61, weights vary over many decades
    d, n = 64, 300
    q, k, v = random_inputs(11, (1, 2, n, d), "f32", 20.0)
    q = np.clip(q, -60, 60)
    k = np.clip(k, -60, 60)
    say("extreme inputs", form)
    g = run_forward(ea, form, q, k, v, "f32")
    ref = oracle_forward(form, q, k, v, "f32")
    assert form_err(form, g, ref) <= TOL_F32


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("form", ["noncausal", "causal"])
def test_zero_denominator_rows(ea, form, dtype):
    """The degenerate case of eq. Attention_i: a query whose features all underflow to 0 (every
    entry -1e4, elu + 1 = exp(-1e4) = 0), or, causally, a query that sees only such keys, has
    numerator and denominator 0; the result is the IEEE 0/0 (NaN), as the oracle's fp64
    evaluation of the formula gives, and every other row is unaffected."""
    d, n = 64, 300
    q, k, v = random_inputs(13, (1, 2, n, d), dtype, 1.0 / np.sqrt(d))
    q, k = f64(q, dtype).astype(np.float32), f64(k, dtype).astype(np.float32)
    q[0, 0, [3, 17, 299]] = -1e4
    q[0, 1, 150] = -1e4
    k[0, 1, :5] = -1e4  # causal rows 0..4 of head 1 see only zero keys
    q, k = encode(q, dtype), encode(k, dtype)
    say("zero denominators", form, dtype)
    g = run_forward(ea, form, q, k, v, dtype)
    with np.errstate(invalid="ignore"):
        ref = oracle_forward(form, q, k, v, dtype)
    bad = np.isnan(ref).any(axis=-1)
    assert bad[0, 0, [3, 17, 299]].all() and bad[0, 1, 150]
    assert bad[0, 1, :5].all() == (form == "causal")
    assert np.array_equal(np.isnan(g), np.isnan(ref))
    assert np.isfinite(g[~bad]).all()
    for h in range(2):
        ok = ~bad[0, h]
        assert form_err(form, g[0, h][ok][None], ref[0, h][ok][None]) <= TOL[dtype]


def test_decode_zero_feature_key_leaves_state(ea):
    """Decode with a key whose features are all 0 (entries -1e4): the state does not move, and
    from the empty state the output is 0/0 (NaN); the next ordinary token then gives v."""
    import torch
    B, H, d = 2, 3, 128
    q, k, v = random_inputs(14, (B, H, 2, d), "bf16", 1.0 / np.sqrt(d))
    k0 = encode(np.full((B, H, d), -1e4, dtype=np.float32), "bf16")
    S = torch.zeros((B, H, d, d), dtype=torch.float32, device="cuda")
    z = torch.zeros((B, H, d), dtype=torch.float32, device="cuda")
    say("decode zero-feature key")
    o1 = from_dev(ea.la_decode_step(to_dev(q[:, :, 0], "bf16"), to_dev(k0, "bf16"), to_dev(v[:, :, 0], "bf16"), S, z), "bf16")
    assert np.isnan(o1).all()
    assert not bool(S.any()) and not bool(z.any())
    o2 = from_dev(ea.la_decode_step(to_dev(q[:, :, 1], "bf16"), to_dev(k[:, :, 1], "bf16"), to_dev(v[:, :, 1], "bf16"), S, z), "bf16")
    np.testing.assert_allclose(o2, f64(v[:, :, 1], "bf16"), rtol=2.0 ** -7, atol=0)  # v to a bf16 ulp


@pytest.mark.parametrize("form", ["noncausal", "causal"])
def test_linear_in_values(ea, form):
    """The output is linear in V for fixed Q, K (eq. Attention_i: fixed weights times values):
    out(a V1 + b V2) = a out(V1) + b out(V2), fp32 within its bar."""
    d, n = 128, 900
    q, k, v1 = random_inputs(17, (1, 2, n, d), "f32", 1.0 / np.sqrt(d))
    _, _, v2 = random_inputs(18, (1, 2, n, d), "f32", 1.0)
    a, b = np.float32(0.75), np.float32(-1.25)
    v3 = (a * v1 + b * v2).astype(np.float32)
    say("linearity", form)
    g1 = run_forward(ea, form, q, k, v1, "f32")
    g2 = run_forward(ea, form, q, k, v2, "f32")
    g3 = run_forward(ea, form, q, k, v3, "f32")
    assert form_err(form, g3, float(a) * g1 + float(b) * g2) <= TOL_F32


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_noncausal_permutations(ea, dtype):
    """Eq. Attention_i sums over the keys: permuting the rows of (K, V) together leaves the
    non-causal outputs unchanged (to rounding: the sums are taken in another order), and
    permuting the rows of Q permutes the outputs (bitwise: each query row is computed alone)."""
    d, n = 64, 1500
    q, k, v = random_inputs(16, (1, 2, n, d), dtype, 1.0 / np.sqrt(d))
    rng = np.random.default_rng(16)
    pk = rng.permutation(n)
    pq = rng.permutation(n)
    say("permutations", dtype)
    g = run_forward(ea, "noncausal", q, k, v, dtype)
    gk = run_forward(ea, "noncausal", q, k[:, :, pk].copy(), v[:, :, pk].copy(), dtype)
    gq = run_forward(ea, "noncausal", q[:, :, pq].copy(), k, v, dtype)
    assert normwise_err(gk, g) <= TOL[dtype]
    assert np.array_equal(gq, g[:, :, pq])


def test_calls_on_a_side_stream(ea):
    """Entry points given another stream (a torch stream or its raw handle) run there, with
    their outputs and workspaces allocated on it, while the default stream is busy; results
    equal the default-stream calls bitwise."""
    import torch
    d = 128
    q, k, v = random_inputs(15, (2, 4, 3000, d), "bf16", 1.0 / np.sqrt(d))
    tq, tk, tv = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    say("side stream")
    ref = [ea.la_forward_noncausal(tq, tk, tv), ea.la_forward_causal(tq, tk, tv, chunk=128),
           ea.la_forward_causal(tq, tk, tv, chunk=64)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    busy = torch.randn(4096, 4096, device="cuda")
    for _ in range(4):
        busy = busy @ busy.T * 1e-3  # default-stream work running meanwhile
    got = [ea.la_forward_noncausal(tq, tk, tv, stream=side),
           ea.la_forward_causal(tq, tk, tv, chunk=128, stream=side),
           ea.la_forward_causal(tq, tk, tv, chunk=64, stream=side.cuda_stream)]
    side.synchronize()
    torch.cuda.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a, b)


@pytest.mark.parametrize("form", ["noncausal", "causal"])
def test_deterministic(ea, form):
    d, n = 128, 1500
    q, k, v = random_inputs(12, (1, 3, n, d), "bf16", 1.0 / np.sqrt(d))
    say("determinism", form)
    a = run_forward(ea, form, q, k, v, "bf16", 128)
    b = run_forward(ea, form, q, k, v, "bf16", 128)
    assert np.array_equal(a, b)


def test_errors_write_nothing(ea):
    import torch
    q = torch.ones((1, 1, 64, 64), dtype=torch.bfloat16, device="cuda")
    out = torch.full_like(q, 7.0)
    say("error path")
    with pytest.raises(ea.LinAttnError):
        ea.la_forward_causal(q, q, q, chunk=96, out=out)
    with pytest.raises(ea.LinAttnError):
        ea.la_forward_noncausal(q, q, q, out=out, ws=torch.zeros(16, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())


# ----------------------------------------------------------------------------- decode
def _state_from_prior(pk, pv, dtype):
    S, z = oracle.state_from_tokens_matmul(f64(pk, dtype), f64(pv, dtype))
    return S.astype(np.float32), z.astype(np.float32)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 64), ("f32", 128)])
def test_decode_steps_vs_oracle(ea, dtype, d):
    import torch
    B, H, prior, steps = 3, 5, 100, 40
    scale = 1.0 / np.sqrt(d)
    pk, pv, _ = random_inputs(20 + d, (B, H, prior, d), dtype, scale)
    q, k, v = random_inputs(21 + d, (B, H, steps, d), dtype, scale)
    S0, z0 = _state_from_prior(pk, pv, dtype)
    S = torch.from_numpy(S0).cuda()
    z = torch.from_numpy(z0).cuda()
    Sr, zr = S0.astype(np.float64), z0.astype(np.float64)
    say("decode", dtype, d)
    for t in range(steps):
        o = ea.la_decode_step(to_dev(q[:, :, t], dtype), to_dev(k[:, :, t], dtype), to_dev(v[:, :, t], dtype), S, z)
        ro, Sr, zr = oracle.decode_step(f64(q[:, :, t], dtype), f64(k[:, :, t], dtype), f64(v[:, :, t], dtype), Sr, zr)
        e = normwise_err(from_dev(o, dtype), ro, head_axes_last=1)
        assert e <= TOL[dtype], (t, e)
    assert normwise_err(S.cpu().numpy(), Sr) <= 1e-5
    assert normwise_err(z.cpu().numpy(), zr, head_axes_last=1) <= 1e-5


def test_decode_from_zero_equals_causal(ea):
    import torch
    B, H, n, d = 2, 2, 70, 64
    q, k, v = random_inputs(30, (B, H, n, d), "bf16", 1.0 / np.sqrt(d))
    S = torch.zeros((B, H, d, d), dtype=torch.float32, device="cuda")
    z = torch.zeros((B, H, d), dtype=torch.float32, device="cuda")
    say("decode from zero vs causal")
    outs = []
    for t in range(n):
        o = ea.la_decode_step(to_dev(q[:, :, t], "bf16"), to_dev(k[:, :, t], "bf16"), to_dev(v[:, :, t], "bf16"), S, z)
        outs.append(from_dev(o, "bf16"))
    g = np.stack(outs, axis=2)
    ref = oracle_forward("causal", q, k, v, "bf16")
    assert rowwise_err(g, ref) <= TOL_BF16
    gc = run_forward(ea, "causal", q, k, v, "bf16", 64)
    assert rowwise_err(g, gc) <= TOL_BF16


def test_decode_resume_bitwise(ea):
    import torch
    B, H, n, d = 4, 8, 24, 128
    q, k, v = random_inputs(31, (B, H, n, d), "bf16", 1.0 / np.sqrt(d))
    dq, dk, dv = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")

    def steps(S, z, t0, t1):
        res = []
        for t in range(t0, t1):
            res.append(ea.la_decode_step(dq[:, :, t].contiguous(), dk[:, :, t].contiguous(),
                                         dv[:, :, t].contiguous(), S, z).clone())
        return res

    say("decode resume")
    S1 = torch.zeros((B, H, d, d), dtype=torch.float32, device="cuda")
    z1 = torch.zeros((B, H, d), dtype=torch.float32, device="cuda")
    full = steps(S1, z1, 0, n)
    S2 = torch.zeros_like(S1)
    z2 = torch.zeros_like(z1)
    first = steps(S2, z2, 0, n // 2)
    saved = (S2.cpu().numpy().tobytes(), z2.cpu().numpy().tobytes())
    S3 = torch.from_numpy(np.frombuffer(saved[0], dtype=np.float32).reshape(B, H, d, d).copy()).cuda()
    z3 = torch.from_numpy(np.frombuffer(saved[1], dtype=np.float32).reshape(B, H, d).copy()).cuda()
    second = steps(S3, z3, n // 2, n)
    for a, b in zip(full, first + second):
        assert torch.equal(a, b)
    assert torch.equal(S1, S3) and torch.equal(z1, z3)


# ----------------------------------------------------------------------------- causal stages
# ----------------------------------------------------------------------------- causal with state in/out
def _state_err(g, r):
    """Normwise error per head of [B, H, d, d] (or [B, H, d]) states."""
    return normwise_err(g, r, head_axes_last=2 if np.ndim(r) == 4 else 1)


@pytest.mark.parametrize("dtype,d,chunk", [("bf16", 128, 128), ("bf16", 64, 64), ("bf16", 64, 128),
                                           ("bf16", 128, 64), ("f32", 64, 64), ("f32", 128, 64)])
def test_causal_state_vs_oracle(ea, dtype, d, chunk):
    # out and final state from an initial state built from prior tokens; few heads, so the
    # sequence is cut into segments (the state enters every segment)
    import torch
    B, H, prior, n = 2, 3, 90, 700
    scale = 1.0 if dtype == "f32" else 1.0 / np.sqrt(d)
    pk, pv, _ = random_inputs(40 + d + chunk, (B, H, prior, d), dtype, scale)
    q, k, v = random_inputs(41 + d + chunk, (B, H, n, d), dtype, scale)
    S0, z0 = _state_from_prior(pk, pv, dtype)
    say("causal state in/out", dtype, d, chunk)
    out, Sn, zn = ea.la_forward_causal_state(to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), chunk,
                                             torch.from_numpy(S0).cuda(), torch.from_numpy(z0).cuda())
    ref, Sr, zr = oracle.causal_recurrent(f64(q, dtype), f64(k, dtype), f64(v, dtype),
                                          s0=S0.astype(np.float64), z0=z0.astype(np.float64), return_state=True)
    assert rowwise_err(from_dev(out, dtype), ref) <= TOL[dtype]
    assert _state_err(Sn.cpu().numpy(), Sr) <= TOL[dtype]
    assert _state_err(zn.cpu().numpy(), zr) <= TOL[dtype]


@pytest.mark.parametrize("dtype,d,chunk", [("bf16", 128, 128), ("f32", 64, 64)])
def test_causal_state_from_zero_matches_forward(ea, dtype, d, chunk):
    # no initial state: the outputs are those of la_forward_causal, bit for bit, and the final
    # state is the plain sum over all tokens
    B, H, n = 2, 4, 1000
    scale = 1.0 if dtype == "f32" else 1.0 / np.sqrt(d)
    q, k, v = random_inputs(50 + d, (B, H, n, d), dtype, scale)
    tq, tk, tv = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
    say("causal state from zero", dtype, d, chunk)
    out, Sn, zn = ea.la_forward_causal_state(tq, tk, tv, chunk)
    plain = ea.la_forward_causal(tq, tk, tv, chunk=chunk)
    assert np.array_equal(from_dev(out, dtype), from_dev(plain, dtype))
    Sr, zr = oracle.state_from_tokens_matmul(f64(k, dtype), f64(v, dtype))
    assert _state_err(Sn.cpu().numpy(), Sr) <= TOL[dtype]
    assert _state_err(zn.cpu().numpy(), zr) <= TOL[dtype]


@pytest.mark.parametrize("dtype,d,chunk", [("bf16", 64, 64), ("bf16", 128, 128), ("f32", 64, 128)])
def test_causal_state_pieces_bitwise(ea, dtype, d, chunk):
    # 256 heads give one segment per head; cut at a chunk boundary, two calls with the state
    # carried do the same arithmetic as one call: outputs and final state agree bit for bit
    import torch
    B, H, n1, n2 = 16, 16, 2 * chunk, 150
    scale = 1.0 if dtype == "f32" else 1.0 / np.sqrt(d)
    q, k, v = random_inputs(60 + d + chunk, (B, H, n1 + n2, d), dtype, scale)
    tq, tk, tv = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
    assert ea.la_causal_plan(B, H, n1 + n2, d, chunk, tq.dtype) >= n1 + n2  # one segment
    say("causal state pieces", dtype, d, chunk)
    full, Sf, zf = ea.la_forward_causal_state(tq, tk, tv, chunk)
    a, S1, z1 = ea.la_forward_causal_state(tq[:, :, :n1].contiguous(), tk[:, :, :n1].contiguous(),
                                           tv[:, :, :n1].contiguous(), chunk)
    b, S2, z2 = ea.la_forward_causal_state(tq[:, :, n1:].contiguous(), tk[:, :, n1:].contiguous(),
                                           tv[:, :, n1:].contiguous(), chunk, S1, z1)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([a, b], dim=2), full)
    assert torch.equal(S2, Sf) and torch.equal(z2, zf)


@pytest.mark.parametrize("dtype,d,chunk", [("bf16", 128, 128), ("bf16", 64, 64), ("f32", 128, 64)])
def test_causal_state_pieces_segmented(ea, dtype, d, chunk):
    # few heads (several segments per head) and a cut inside a chunk: agreement to rounding
    B, H, n1, n2 = 1, 2, 1000, 1333
    scale = 1.0 if dtype == "f32" else 1.0 / np.sqrt(d)
    q, k, v = random_inputs(70 + d + chunk, (B, H, n1 + n2, d), dtype, scale)
    tq, tk, tv = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
    say("causal state pieces, segmented", dtype, d, chunk)
    a, S1, z1 = ea.la_forward_causal_state(tq[:, :, :n1].contiguous(), tk[:, :, :n1].contiguous(),
                                           tv[:, :, :n1].contiguous(), chunk)
    b, S2, z2 = ea.la_forward_causal_state(tq[:, :, n1:].contiguous(), tk[:, :, n1:].contiguous(),
                                           tv[:, :, n1:].contiguous(), chunk, S1, z1)
    ref, Sr, zr = oracle.causal_recurrent(f64(q, dtype), f64(k, dtype), f64(v, dtype), return_state=True)
    g = np.concatenate([from_dev(a, dtype), from_dev(b, dtype)], axis=2)
    assert rowwise_err(g, ref) <= TOL[dtype]
    assert _state_err(S2.cpu().numpy(), Sr) <= TOL[dtype]
    assert _state_err(z2.cpu().numpy(), zr) <= TOL[dtype]


def test_prefill_then_decode(ea):
    # the final state of a causal prefill is the decode step's state: decoding the next tokens
    # continues the causal outputs of the whole sequence
    B, H, n, steps, d = 2, 4, 517, 20, 128
    q, k, v = random_inputs(80, (B, H, n + steps, d), "bf16", 1.0 / np.sqrt(d))
    tq, tk, tv = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    say("prefill then decode")
    _, S, z = ea.la_forward_causal_state(tq[:, :, :n].contiguous(), tk[:, :, :n].contiguous(),
                                         tv[:, :, :n].contiguous(), 128)
    outs = []
    for t in range(n, n + steps):
        o = ea.la_decode_step(tq[:, :, t].contiguous(), tk[:, :, t].contiguous(), tv[:, :, t].contiguous(), S, z)
        outs.append(from_dev(o, "bf16"))
    ref = oracle.causal_recurrent(f64(q, "bf16"), f64(k, "bf16"), f64(v, "bf16"))
    assert rowwise_err(np.stack(outs, axis=2), ref[:, :, n:]) <= TOL_BF16


def test_causal_state_empty_sequence(ea):
    # n = 0: the final state is the initial one (zeros without one), nothing else is touched
    import torch
    B, H, d = 3, 2, 64
    e = torch.empty((B, H, 0, d), dtype=torch.bfloat16, device="cuda")
    S0 = torch.randn(B, H, d, d, device="cuda")
    z0 = torch.rand(B, H, d, device="cuda")
    say("causal state, empty sequence")
    out, Sn, zn = ea.la_forward_causal_state(e, e, e, 64, S0, z0)
    torch.cuda.synchronize()
    assert out.shape == e.shape and torch.equal(Sn, S0) and torch.equal(zn, z0)
    Sn.fill_(7.0)
    zn.fill_(7.0)
    _, Sn, zn = ea.la_forward_causal_state(e, e, e, 64, Sn=Sn, zn=zn)
    torch.cuda.synchronize()
    assert torch.count_nonzero(Sn) == 0 and torch.count_nonzero(zn) == 0


# ----------------------------------------------------------------------------- variable-length batches
def _packed(seed, lengths, H, d, dtype, scale):
    """Per-sequence inputs [H, n_s, d] and their packed form [sum_s H n_s, d] (sequence blocks
    back to back)."""
    seqs = [random_inputs(seed + 17 * i, (H, n, d), dtype, scale) for i, n in enumerate(lengths)]
    packed = [np.concatenate([s[j].reshape(-1, d) for s in seqs]) for j in range(3)]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    return seqs, packed, cu


VARLEN = [("noncausal", "bf16", 64, 0), ("noncausal", "bf16", 128, 0), ("noncausal", "f32", 64, 0),
          ("causal", "bf16", 128, 128), ("causal", "bf16", 64, 64), ("causal", "bf16", 64, 128),
          ("causal", "f32", 64, 64), ("causal", "f32", 128, 64)]


@pytest.mark.parametrize("form,dtype,d,chunk", VARLEN)
def test_varlen_equals_each_sequence_alone(ea, form, dtype, d, chunk):
    # a ragged batch (empty, one-token, chunk-edge and several-segment sequences) gives each
    # sequence the result of the fixed-length call on it alone, and the oracle's
    import torch
    H = 3
    lengths = [300, 0, 1, chunk + 1 if chunk else 65, 2500, 64, 1000]
    scale = 1.0 if dtype == "f32" else 1.0 / np.sqrt(d)
    seqs, (pq, pk, pv), cu = _packed(90 + d + chunk, lengths, H, d, dtype, scale)
    tq, tk, tv = to_dev(pq, dtype), to_dev(pk, dtype), to_dev(pv, dtype)
    say("varlen", form, dtype, d, chunk)
    if form == "noncausal":
        out = ea.la_forward_noncausal_varlen(tq, tk, tv, cu, H)
    else:
        out = ea.la_forward_causal_varlen(tq, tk, tv, cu, H, chunk=chunk)
    g = from_dev(out, dtype)
    for i, (n, (q, k, v)) in enumerate(zip(lengths, seqs)):
        if n == 0:
            continue
        gs = g[H * cu[i]:H * cu[i + 1]].reshape(H, n, d)
        ref = oracle_forward(form, q[None], k[None], v[None], dtype)[0]
        assert form_err(form, gs, ref) <= TOL[dtype], (i, n)
        alone = run_forward(ea, form, q[None], k[None], v[None], dtype, chunk or 64)[0]
        assert form_err(form, gs, alone) <= TOL[dtype], (i, n)


def test_varlen_many_sequences_long(ea):
    # many sequences of mixed lengths, several segments for the longest, 128-token chunks
    H, d = 4, 128
    rng = np.random.default_rng(3)
    lengths = [int(x) for x in rng.integers(0, 6000, size=24)]
    seqs, (pq, pk, pv), cu = _packed(95, lengths, H, d, "bf16", 1.0 / np.sqrt(d))
    tq, tk, tv = to_dev(pq, "bf16"), to_dev(pk, "bf16"), to_dev(pv, "bf16")
    say("varlen many sequences")
    for form in ("noncausal", "causal"):
        out = (ea.la_forward_noncausal_varlen(tq, tk, tv, cu, H) if form == "noncausal"
               else ea.la_forward_causal_varlen(tq, tk, tv, cu, H, chunk=128))
        g = from_dev(out, "bf16")
        for i in (0, 7, 23, int(np.argmax(lengths))):
            n = lengths[i]
            if n == 0:
                continue
            q, k, v = seqs[i]
            gs = g[H * cu[i]:H * cu[i + 1]].reshape(H, n, d)
            assert form_err(form, gs, oracle_forward(form, q[None], k[None], v[None], "bf16")[0]) <= TOL_BF16


def test_decode_masked_skips_inactive_sequences(ea):
    # active sequences step exactly as la_decode_step and as the oracle's decode step ("The
    # recurrent view": fold in (k, v), then read with q); inactive ones keep state and out
    import torch
    B, H, d = 5, 3, 128
    q, k, v = random_inputs(96, (B, H, d), "bf16", 1.0 / np.sqrt(d))
    S0 = torch.randn(B, H, d, d, device="cuda") * 0.01
    z0 = torch.rand(B, H, d, device="cuda") + 1.0
    active = torch.tensor([1, 0, 1, 1, 0], dtype=torch.uint8, device="cuda")
    tq, tk, tv = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    say("decode masked")
    S1, z1 = S0.clone(), z0.clone()
    full = ea.la_decode_step(tq, tk, tv, S1, z1)
    S2, z2 = S0.clone(), z0.clone()
    out = torch.full_like(full, 7.0)
    ea.la_decode_step_masked(tq, tk, tv, S2, z2, active, out=out)
    torch.cuda.synchronize()
    on = active.bool()
    assert torch.equal(out[on], full[on]) and torch.equal(S2[on], S1[on]) and torch.equal(z2[on], z1[on])
    off = ~on
    assert torch.all(out[off] == 7.0) and torch.equal(S2[off], S0[off]) and torch.equal(z2[off], z0[off])
    idx = on.cpu().numpy().astype(bool)
    ro, Sr, zr = oracle.decode_step(f64(q, "bf16")[idx], f64(k, "bf16")[idx], f64(v, "bf16")[idx],
                                    S0.cpu().numpy().astype(np.float64)[idx], z0.cpu().numpy().astype(np.float64)[idx])
    assert normwise_err(from_dev(out, "bf16")[idx], ro, head_axes_last=1) <= TOL_BF16
    assert _state_err(S2.cpu().numpy()[idx], Sr) <= TOL_F32
    assert _state_err(z2.cpu().numpy()[idx], zr) <= TOL_F32


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("bf16", 128), ("f32", 64)])
def test_state_sums_vs_oracle(ea, dtype, d):
    import torch
    B, H, n, seg_len, nseg = 2, 3, 1000, 300, 4          # last segment ragged (100 tokens)
    q, k, v = random_inputs(40 + d, (B, H, n, d), dtype, 1.0 / np.sqrt(d))
    say("state sums", dtype, d)
    sums = ea.la_state_sums(to_dev(k, dtype), to_dev(v, dtype), seg_len, nseg)
    torch.cuda.synchronize()
    g = sums.cpu().numpy().astype(np.float64)
    K, V = f64(k, dtype), f64(v, dtype)
    for s in range(nseg):
        S, z = oracle.state_accumulate(K[:, :, s * seg_len:(s + 1) * seg_len], V[:, :, s * seg_len:(s + 1) * seg_len])
        ref = np.concatenate([S.reshape(B, H, d * d), z], axis=-1)
        # bf16 rounds phi(K) once before the MFMA; fp32 holds every factor to 2^-16 (a two-term
        # bf16 split, with errors of either sign) and sums z from the fp32 features
        assert normwise_err(g[:, :, s], ref, head_axes_last=1) <= (4e-3 if dtype == "bf16" else 1e-6)


@pytest.mark.parametrize("dtype,d,chunk", [("bf16", 128, 128), ("bf16", 64, 64), ("f32", 64, 128)])
def test_causal_segments_from_oracle_sums(ea, dtype, d, chunk):
    import torch
    B, H, n = 1, 2, 5 * chunk + 11
    seg_len = 2 * chunk                                    # 3 segments, last one ragged
    q, k, v = random_inputs(50 + d, (B, H, n, d), dtype, 1.0 / np.sqrt(d))
    Q, K, V = f64(q, dtype), f64(k, dtype), f64(v, dtype)
    sums = []
    for s in range(2):
        S, z = oracle.state_accumulate(K[:, :, s * seg_len:(s + 1) * seg_len], V[:, :, s * seg_len:(s + 1) * seg_len])
        sums.append(np.concatenate([S.reshape(B, H, d * d), z], axis=-1))
    sums = torch.from_numpy(np.stack(sums, axis=2).astype(np.float32)).cuda()
    say("causal segments from oracle sums", dtype, d, chunk)
    out = ea.la_causal_segments(to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), sums, seg_len, chunk)
    assert rowwise_err(from_dev(out, dtype), oracle.causal_recurrent(Q, K, V)) <= TOL[dtype]


@pytest.mark.parametrize("dtype,d,chunk,B,H,n", [("bf16", 128, 128, 2, 4, 3000), ("bf16", 64, 64, 1, 1, 5000),
                                                 ("f32", 64, 64, 1, 3, 2000)])
def test_stages_compose_to_forward_causal(ea, dtype, d, chunk, B, H, n):
    q, k, v = random_inputs(60 + d, (B, H, n, d), dtype, 1.0 / np.sqrt(d))
    tq, tk, tv = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
    seg_len = ea.la_causal_plan(B, H, n, d, chunk, tq.dtype)
    nseg = -(-n // seg_len)
    assert nseg > 1
    say("stages compose", dtype, d, chunk, B, H, n, seg_len)
    sums = ea.la_state_sums(tk, tv, seg_len, nseg - 1)
    a = ea.la_causal_segments(tq, tk, tv, sums, seg_len, chunk)
    b = ea.la_forward_causal(tq, tk, tv, chunk=chunk)
    assert np.array_equal(from_dev(a, dtype), from_dev(b, dtype))


@pytest.mark.parametrize("fill", [0x00, 0x3F, 0xFF])
def test_workspace_contents_do_not_matter(ea, fill):
    # regression: a workspace reused across shapes may hold an earlier call's partial sums
    # where this call keeps its arrival counters; every call must initialise them itself
    import torch
    dtype = "bf16"
    shapes = [(1, 1, 5000, 64, 64), (2, 4, 3000, 128, 128), (4, 8, 1500, 64, 64)]
    ref = {}
    for (B, H, n, d, chunk) in shapes:
        q, k, v = random_inputs(70 + n, (B, H, n, d), dtype, 1.0 / np.sqrt(d))
        ref[(B, H, n, d, chunk)] = (q, k, v, oracle_forward("causal", q, k, v, dtype),
                                    oracle_forward("noncausal", q, k, v, dtype))
    big = 64 << 20
    ws = torch.full((big,), fill, dtype=torch.uint8, device="cuda")
    say("workspace fill", fill)
    for (B, H, n, d, chunk), (q, k, v, rc, rn) in ref.items():
        tq, tk, tv = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
        gc = from_dev(ea.la_forward_causal(tq, tk, tv, chunk=chunk, ws=ws), dtype)
        gn = from_dev(ea.la_forward_noncausal(tq, tk, tv, ws=ws), dtype)
        assert rowwise_err(gc, rc) <= TOL_BF16
        assert normwise_err(gn, rn) <= TOL_BF16
        # and bitwise equal to a run on a fresh workspace
        gc2 = from_dev(ea.la_forward_causal(tq, tk, tv, chunk=chunk,
                                            ws=torch.zeros(big, dtype=torch.uint8, device="cuda")), dtype)
        assert np.array_equal(gc, gc2)


def test_release_workspaces_drops_the_cached_buffers(ea):
    # calls given no workspace share one per (device, stream); release_workspaces hands them back
    import torch
    from efficient_attention_amd import _binding
    dtype = "bf16"
    q, k, v = (to_dev(x, dtype) for x in random_inputs(81, (2, 4, 3000, 64), dtype, 0.125))
    _binding.release_workspaces()
    say("workspace cache")
    a = ea.la_forward_noncausal(q, k, v)
    torch.cuda.synchronize()
    need = ea.la_noncausal_workspace_bytes(2, 4, 3000, 64, torch.bfloat16)
    assert need > 0
    assert _binding.release_workspaces(device=q.device) >= need
    assert _binding.release_workspaces() == 0
    assert _binding.release_workspaces(device=q.device) == 0
    b = ea.la_forward_noncausal(q, k, v)  # a new cached workspace, the same result
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert _binding.release_workspaces() >= need
