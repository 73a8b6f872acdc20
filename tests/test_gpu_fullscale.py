"""GPU parity at the workloads' full sizes, in the launch configuration bench.py times.

The oracle cannot redo every full-size workload in seconds on one core, so the tests check:
  * for C3, C4, the 16 grid points and F3, every head against the oracle's full computation
    (non-causal form, causal recurrence), one head per host thread (about 13 s for C4's 128
    heads on 16 cores); for F4, whose oracle is a token loop in numpy, one whole head,
  * single rows (sampled, incl. segment and chunk boundaries and the last row) against the
    quadratic definition at O(n d) per row,
  * for decode, every step's output of sampled heads, and the final state of EVERY head
    against the fp64 sum of all tokens it has seen.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import oracle
from gpu_util import f64, from_dev, need_gpu, say, to_dev
from metrics import TOL_BF16, form_err, normwise_err, rowwise_err
from seeded_inputs import WORKLOADS, decode_inputs, forward_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ea():
    need_gpu()
    import efficient_attention_amd
    return efficient_attention_amd


def _sample_rows(n, extra, rng, count=12):
    rows = set(int(x) for x in rng.integers(0, n, size=count))
    rows.update(r for r in extra if 0 <= r < n)
    return np.array(sorted(rows), dtype=np.int64)


def _check_forward(ea, name, form):
    w = WORKLOADS[name]
    say(name, "generating inputs", w)
    q, k, v = forward_inputs(w)
    tq, tk, tv = to_dev(q, w.dtype), to_dev(k, w.dtype), to_dev(v, w.dtype)
    say(name, "GPU run")
    if form == "noncausal":
        out = ea.la_forward_noncausal(tq, tk, tv)
    else:
        out = ea.la_forward_causal(tq, tk, tv, chunk=w.chunk)
    g = from_dev(out, w.dtype)
    assert np.all(np.isfinite(g))
    # every head against the oracle's full computation; the heads are independent, and the C
    # oracle (called through ctypes, which releases the interpreter lock) runs one per thread

    def head_err(bh):
        b, h = divmod(bh, w.H)
        Q, K, V = (f64(x[b, h], w.dtype) for x in (q, k, v))
        ref = oracle.noncausal_linear(Q, K, V) if form == "noncausal" else oracle.causal_recurrent(Q, K, V)
        return form_err(form, g[b, h], ref)

    say(name, "oracle on all", w.B * w.H, "heads")
    with ThreadPoolExecutor(max(1, min(16, os.cpu_count() or 1))) as ex:
        errs = np.array(list(ex.map(head_err, range(w.B * w.H))))
    worst = int(np.argmax(errs))
    print("%s all %d heads: worst err %.3e (head %d), median %.3e" % (name, errs.size, errs[worst], worst,
                                                                    float(np.median(errs))))
    assert errs.max() <= TOL_BF16, (worst, errs[worst])
    # sampled rows of other heads, by the quadratic definition
    rng = np.random.default_rng(7)
    seg_len = ea.la_causal_plan(w.B, w.H, w.n, w.d, w.chunk or 128, tq.dtype) if form == "causal" else w.n
    extra = [0, 1, w.n - 1, seg_len - 1, seg_len, seg_len + 1, (w.chunk or 64) - 1, w.chunk or 64]
    for _ in range(6):
        b, h = int(rng.integers(0, w.B)), int(rng.integers(0, w.H))
        rows = _sample_rows(w.n, extra, rng)
        say(name, "oracle rows", b, h, len(rows))
        Q, K, V = (f64(x[b, h], w.dtype) for x in (q, k, v))
        ref = oracle.rows(Q, K, V, rows, causal=(form == "causal"))
        e = form_err(form, g[b, h][rows][None], ref[None])
        assert e <= TOL_BF16, (b, h, e)


def test_c3_noncausal_bf16_full(ea):
    _check_forward(ea, "C3", "noncausal")


def test_c4_causal_bf16_full(ea):
    _check_forward(ea, "C4", "causal")


def test_c5_decode_full(ea):
    import torch
    w = WORKLOADS["C5"]
    say("C5 generating inputs")
    pk, pv, q, k, v = decode_inputs(w)
    B, H, d, steps = w.B, w.H, w.d, w.n
    # initial state: the 1024 prior tokens summed by the oracle in fp64, rounded to fp32; the
    # same fp32 bytes start the GPU and the oracle
    say("C5 initial state (oracle, fp64 matmul)")
    S0 = np.empty((B, H, d, d), dtype=np.float32)
    z0 = np.empty((B, H, d), dtype=np.float32)
    for b in range(B):
        S, z = oracle.state_from_tokens_matmul(f64(pk[b], w.dtype), f64(pv[b], w.dtype))
        S0[b], z0[b] = S, z
    S = torch.from_numpy(S0).cuda()
    z = torch.from_numpy(z0).cuda()
    dq = to_dev(q, w.dtype).permute(2, 0, 1, 3).contiguous()   # [steps, B, H, d]
    dk = to_dev(k, w.dtype).permute(2, 0, 1, 3).contiguous()
    dv = to_dev(v, w.dtype).permute(2, 0, 1, 3).contiguous()
    rng = np.random.default_rng(5)
    sample = [(0, 0), (B - 1, H - 1)] + [(int(rng.integers(0, B)), int(rng.integers(0, H))) for _ in range(14)]
    sb = torch.tensor([s[0] for s in sample], device="cuda")
    sh = torch.tensor([s[1] for s in sample], device="cuda")
    outs = []
    say("C5 GPU 512 steps")
    for t in range(steps):
        o = ea.la_decode_step(dq[t], dk[t], dv[t], S, z)
        outs.append(o[sb, sh].clone())
    g = np.stack([from_dev(x, w.dtype) for x in outs], axis=1)     # [sample, steps, d]
    say("C5 oracle on sampled heads")
    worst = 0.0
    for i, (b, h) in enumerate(sample):
        Sr, zr = S0[b, h].astype(np.float64), z0[b, h].astype(np.float64)
        Q, K, V = (f64(x[b, h], w.dtype) for x in (q, k, v))
        for t in range(steps):
            ro, Sr, zr = oracle.decode_step(Q[t], K[t], V[t], Sr, zr)
            e = normwise_err(g[i, t][None], ro[None], head_axes_last=1)
            worst = max(worst, e)
            assert e <= TOL_BF16, (b, h, t, e)
        assert normwise_err(S[b, h].cpu().numpy(), Sr) <= 1e-4
    print("C5 worst per-step normwise err on sampled heads %.3e" % worst)
    # final state of every head vs the fp64 sum over all 1024 + 512 tokens
    say("C5 final state of every head")
    Sg, zg = S.cpu().numpy(), z.cpu().numpy()
    for b in range(B):
        Sa, za = oracle.state_from_tokens_matmul(f64(k[b], w.dtype), f64(v[b], w.dtype))
        Sref = S0[b].astype(np.float64) + Sa
        zref = z0[b].astype(np.float64) + za
        assert normwise_err(Sg[b], Sref) <= 1e-4
        assert normwise_err(zg[b], zref, head_axes_last=1) <= 1e-5


def test_c4_causal_in_two_pieces_with_state(ea):
    # C4 run as two calls, the second continuing from the first one's final state (cut inside
    # a chunk): sampled rows against the quadratic definition over the whole sequence, the
    # outputs against the one-call forward, and the final state of every head against the
    # fp64 sum over all tokens
    import torch
    w = WORKLOADS["C4"]
    say("C4 pieces generating inputs")
    q, k, v = forward_inputs(w)
    tq, tk, tv = to_dev(q, w.dtype), to_dev(k, w.dtype), to_dev(v, w.dtype)
    cut = 40000
    say("C4 pieces GPU runs")
    a, S1, z1 = ea.la_forward_causal_state(tq[:, :, :cut].contiguous(), tk[:, :, :cut].contiguous(),
                                           tv[:, :, :cut].contiguous(), w.chunk)
    b_, S2, z2 = ea.la_forward_causal_state(tq[:, :, cut:].contiguous(), tk[:, :, cut:].contiguous(),
                                            tv[:, :, cut:].contiguous(), w.chunk, S1, z1)
    g = np.concatenate([from_dev(a, w.dtype), from_dev(b_, w.dtype)], axis=2)
    del a, b_
    assert np.all(np.isfinite(g))
    say("C4 pieces vs one call")
    whole = from_dev(ea.la_forward_causal(tq, tk, tv, chunk=w.chunk), w.dtype)
    e = rowwise_err(g, whole)
    print("C4 two pieces vs one call rowwise err %.3e" % e)
    assert e <= TOL_BF16
    rng = np.random.default_rng(11)
    extra = [0, cut - 1, cut, cut + 1, w.n - 1]
    for _ in range(6):
        b, h = int(rng.integers(0, w.B)), int(rng.integers(0, w.H))
        rows = _sample_rows(w.n, extra, rng)
        say("C4 pieces oracle rows", b, h, len(rows))
        Q, K, V = (f64(x[b, h], w.dtype) for x in (q, k, v))
        ref = oracle.rows(Q, K, V, rows, causal=True)
        assert rowwise_err(g[b, h][rows][None], ref[None]) <= TOL_BF16
    say("C4 pieces final state of every head")
    Sg, zg = S2.cpu().numpy(), z2.cpu().numpy()
    worst = 0.0
    for b in range(w.B):
        Sa, za = oracle.state_from_tokens_matmul(f64(k[b], w.dtype), f64(v[b], w.dtype))
        worst = max(worst, normwise_err(Sg[b], Sa), normwise_err(zg[b], za, head_axes_last=1))
    print("C4 final state normwise err %.3e" % worst)
    assert worst <= TOL_BF16


# ----------------------------------------------------------------------------- the metric's grid
GRID = [(form, dtype, n, d) for dtype in ("bf16", "f32") for form in ("noncausal", "causal")
        for n in (16384, 65536) for d in (64, 128)]


@pytest.mark.parametrize("form,dtype,n,d", GRID)
def test_grid_point_full_size(ea, form, dtype, n, d):
    # every shape of the metric's grid, in the launch configuration `bench.py --grid` times
    # (128 heads, inputs drawn on the device from a seeded generator): every head against the
    # oracle's full computation (one head per host thread, heads fetched in batches), and
    # sampled rows of two heads against the quadratic definition
    import zlib

    import torch
    B, H = 8, 16
    chunk = 64 if (dtype == "f32" and d == 128) else 128  # as bench.py --grid
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    gen = torch.Generator(device="cuda")
    gen.manual_seed(zlib.crc32(repr((form, dtype, n, d)).encode()))
    say("grid", form, dtype, n, d, "GPU run")
    q, k, v = [(torch.randn(B, H, n, d, device="cuda", generator=gen) * d ** -0.5).to(tdt) for _ in range(3)]
    out = ea.la_forward_noncausal(q, k, v) if form == "noncausal" else ea.la_forward_causal(q, k, v, chunk=chunk)
    torch.cuda.synchronize()
    tol = TOL_BF16 if dtype == "bf16" else 1e-4

    def host(t):
        return t.float().cpu().numpy().astype(np.float64)

    seg_len = ea.la_causal_plan(B, H, n, d, chunk, tdt) if form == "causal" else n
    rng = np.random.default_rng(zlib.crc32(repr(("rows", form, dtype, n, d)).encode()))
    extra = [0, 1, chunk - 1, chunk, seg_len - 1, seg_len, n - 1]
    for (b, h) in [(0, 0), (B - 1, H - 1)]:
        Q, K, V, G = host(q[b, h]), host(k[b, h]), host(v[b, h]), host(out[b, h])
        assert np.all(np.isfinite(G))
        rows = _sample_rows(n, extra, rng, count=10)
        say("grid", form, dtype, n, d, "oracle rows", b, h)
        ref = oracle.rows(Q, K, V, rows, causal=(form == "causal"))
        assert form_err(form, G[rows][None], ref[None]) <= tol, (b, h)

    def head_err(Q, K, V, G):
        whole = oracle.noncausal_linear(Q, K, V) if form == "noncausal" else oracle.causal_recurrent(Q, K, V)
        return form_err(form, G, whole)

    say("grid", form, dtype, n, d, "oracle on all", B * H, "heads")
    nthreads = max(1, min(16, os.cpu_count() or 1))
    errs = []
    with ThreadPoolExecutor(nthreads) as ex:
        for h0 in range(0, B * H, nthreads):
            batch = [divmod(bh, H) for bh in range(h0, min(B * H, h0 + nthreads))]
            data = [(host(q[b, h]), host(k[b, h]), host(v[b, h]), host(out[b, h])) for (b, h) in batch]
            errs += list(ex.map(lambda a: head_err(*a), data))
    errs = np.array(errs)
    print("grid %s %s n=%d d=%d all %d heads: worst err %.3e" % (form, dtype, n, d, errs.size, errs.max()))
    assert errs.max() <= tol, (int(np.argmax(errs)), errs.max())



# ----------------------------------------------------------------------------- FAVOR+
def _favor_forward(ea, name):
    from oracle import favor
    from seeded_inputs import projection
    w = WORKLOADS[name]
    say(name, "generating inputs", w)
    q, k, v = forward_inputs(w)
    wp = projection(w.seed, w.m, w.d, "bf16")
    scale = w.d ** -0.25
    tq, tk, tv, tw = (to_dev(x, "bf16") for x in (q, k, v, wp))
    say(name, "GPU run")
    if w.form == "noncausal":
        out = ea.la_favor_forward_noncausal(tq, tk, tv, tw, scale)
    else:
        out = ea.la_favor_forward_causal(tq, tk, tv, tw, scale, chunk=w.chunk)
    del tq, tk, tv
    g = from_dev(out, "bf16")
    assert np.all(np.isfinite(g))
    Wd = f64(wp, "bf16")
    causal = w.form == "causal"
    # whole heads: every head for the non-causal form (numpy's products release the interpreter
    # lock, one head per thread), the last head for the causal form (its oracle is a token loop)

    def head_err(bh):
        b, h = divmod(bh, w.H)
        Q, K, V = (f64(x[b, h], "bf16") for x in (q, k, v))
        ref = favor.causal_recurrent(Q, K, V, Wd, scale) if causal else favor.noncausal(Q, K, V, Wd, scale)
        return form_err(w.form, g[b, h], ref)

    heads = [w.B * w.H - 1] if causal else list(range(w.B * w.H))
    say(name, "oracle on", len(heads), "heads")
    with ThreadPoolExecutor(max(1, min(16, os.cpu_count() or 1))) as ex:
        errs = np.array(list(ex.map(head_err, heads)))
    print("%s %d whole heads: worst err %.3e" % (name, len(heads), errs.max()))
    assert errs.max() <= TOL_BF16, (heads[int(np.argmax(errs))], errs.max())
    # sampled rows of other heads, by the definition
    rng = np.random.default_rng(8)
    seg_len = ea.la_causal_plan(w.B, w.H, w.n, w.d, 64, 1) if causal else w.n
    extra = [0, 1, w.n - 1, seg_len - 1, seg_len, seg_len + 1, 63, 64]
    for _ in range(4):
        b, h = int(rng.integers(0, w.B)), int(rng.integers(0, w.H))
        rows = _sample_rows(w.n, extra, rng)
        say(name, "oracle rows", b, h, len(rows))
        Q, K, V = (f64(x[b, h], "bf16") for x in (q, k, v))
        ref = favor.rows(Q, K, V, Wd, scale, rows, causal)
        e = form_err(w.form, g[b, h][rows][None], ref[None])
        assert e <= TOL_BF16, (b, h, e)


def test_f3_favor_noncausal_full(ea):
    _favor_forward(ea, "F3")


def test_f4_favor_causal_full(ea):
    _favor_forward(ea, "F4")


def test_f5_favor_decode_full(ea):
    """Prefill 1024 tokens per head with the causal forward (final state), then 6 decode steps
    for all 8192 heads; sampled heads' outputs and states against the fp64 recurrence."""
    import torch
    from oracle import favor
    from seeded_inputs import projection
    w = WORKLOADS["F5"]
    steps = 6
    say("F5 generating inputs")
    pk, pv, dq, dk, dv = decode_inputs(w, steps=steps)
    rng = np.random.default_rng(9)
    wp = projection(w.seed, w.m, w.d, "bf16")
    scale = w.d ** -0.25
    tw = to_dev(wp, "bf16")
    tpk, tpv = to_dev(pk, "bf16"), to_dev(pv, "bf16")
    say("F5 prefill")  # (the prefill's outputs are not used: its keys stand in for its queries)
    _, S, z, c = ea.la_favor_forward_causal(tpk, tpk, tpv, tw, scale, final_state=True)
    del tpk, tpv
    outs = []
    for i in range(steps):
        o = ea.la_favor_decode_step(to_dev(np.ascontiguousarray(dq[:, :, i]), "bf16"),
                                    to_dev(np.ascontiguousarray(dk[:, :, i]), "bf16"),
                                    to_dev(np.ascontiguousarray(dv[:, :, i]), "bf16"), tw, S, z, c, scale)
        outs.append(from_dev(o, "bf16"))
    g = np.stack(outs, axis=2)
    assert np.all(np.isfinite(g))
    Wd = f64(wp, "bf16")
    cs = c.cpu().numpy().astype(np.float64)
    Ss = S.cpu().numpy()
    zs = z.cpu().numpy()
    heads = [(0, 0), (w.B - 1, w.H - 1)] + [(int(rng.integers(0, w.B)), int(rng.integers(0, w.H))) for _ in range(14)]
    for (b, h) in heads:
        K = np.concatenate([f64(pk[b, h], "bf16"), f64(dk[b, h], "bf16")])
        V = np.concatenate([f64(pv[b, h], "bf16"), f64(dv[b, h], "bf16")])
        Qd = f64(dq[b, h], "bf16")
        S0, z0 = favor.state(K[: w.prior], V[: w.prior], Wd, scale)
        ref, Sref, zref = favor.causal_recurrent(Qd, K[w.prior:], V[w.prior:], Wd, scale, s0=S0, z0=z0,
                                                 return_state=True)
        assert normwise_err(g[b, h], ref) <= TOL_BF16, (b, h)
        St = Ss[b, h].astype(np.float64) * np.exp(cs[b, h])
        zt = zs[b, h].astype(np.float64) * np.exp(cs[b, h])
        assert normwise_err(St, Sref) <= TOL_BF16, (b, h)
        assert normwise_err(zt[None], zref[None]) <= TOL_BF16, (b, h)
