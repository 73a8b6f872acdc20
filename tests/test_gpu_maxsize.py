"""GPU parity past 32-bit indexing (through the C ABI): tensors of more than 2^31 elements.

Every [B, H, n, d] tensor here holds 2.2-2.3e9 elements (4.4-4.6 GB in bf16, 8.9-9.1 GB in
fp32), in two layouts:
  * "long": one head of n = 2^31/d + 2^27/d + 77 tokens, so row offsets inside a head leave the
    int32 range (17.8M tokens at d = 128, 35.7M at d = 64);
  * "wide": 128 heads of n = 2^31/(128 d) + 4173 tokens, so the head bases leave it.
The decode steps run 139,264 heads (a 9.1 GB state) and a variable-length batch puts its second
sequence's heads past element 2^31.

Keys.  Only a few rows per head take part ("active" keys: row 0 of every head, and in the
checked heads rows on both sides of the element offsets 2^29, 2^30 and 2^31 (byte offsets
2^31 and 2^32 in either dtype), random rows and the last rows).  Every other key row is
-1e4 in every feature, whose elu + 1 is exp(-1e4): exactly 0 in fp32 and in fp64.  For FAVOR+
the other rows are 300 in every feature, whose exponent w.x' - |x'|^2/2 is about -5e5, again
exactly 0 once exponentiated.  By the definition of attention ("Efficient Transformers:
Linear Attention and Flash Attention", eq. Attention_i) a key of zero feature vector adds
nothing to any numerator or denominator, so an output row is the same definition over the
active keys alone, which the oracle evaluates at O(active x d) per row.  The kernels still
stream, index and accumulate all n rows, so a 32-bit offset anywhere would drop, repeat or
misplace active keys or output rows; outputs start as NaN, so a row never written fails the
finiteness check over the whole output.
"""
import numpy as np
import pytest

import oracle
from gpu_util import from_dev, need_gpu, say
from metrics import TOL_BF16, TOL_F32, normwise_err, rowwise_err
from oracle import favor
from seeded_inputs import projection

pytestmark = pytest.mark.gpu

CRIT = (1 << 29, 1 << 30, 1 << 31)   # element offsets whose neighbours every test touches
INACTIVE_ELU = -1.0e4
INACTIVE_FAVOR = 300.0


@pytest.fixture(scope="module")
def ea():
    need_gpu()
    import efficient_attention_amd
    return efficient_attention_amd


def _layout(name, d):
    if name == "long":
        return 1, 1, (1 << 31) // d + (1 << 27) // d + 77
    return 2, 64, (1 << 31) // (128 * d) + 4173


def _tdtype(torch, dtype):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


class Case:
    """Inputs on the device plus, for each checked head, its active key rows and query rows."""

    def __init__(self, torch, dtype, d, layout, seed, inactive, qscale, kscale):
        self.dtype, self.d = dtype, d
        self.B, self.H, self.n = _layout(layout, d)
        B, H, n = self.B, self.H, self.n
        bh = B * H
        assert bh * n * d > (1 << 31)
        td = _tdtype(torch, dtype)
        gen = torch.Generator(device="cuda")
        gen.manual_seed(seed)
        rng = np.random.default_rng(seed)
        shape = (B, H, n, d)
        say("maxsize inputs", dtype, d, layout, shape)
        self.q = torch.randn(shape, dtype=td, device="cuda", generator=gen).mul_(qscale)
        self.v = torch.randn(shape, dtype=td, device="cuda", generator=gen)
        self.k = torch.full(shape, inactive, dtype=td, device="cuda")
        # checked heads: the first, the last, and those holding the critical offsets
        heads = {0, bh - 1}
        crit_rows = {}
        for e in CRIT:
            for x in (e // d - 1, e // d, e // d + 1):
                if x < bh * n:
                    heads.add(x // n)
                    crit_rows.setdefault(x // n, set()).add(x % n)
        self.heads = sorted(heads)
        self.active, self.queries = {}, {}
        flat = [np.arange(bh, dtype=np.int64) * n]          # row 0 of every head
        for h in self.heads:
            extra = crit_rows.get(h, set())
            act = {0, n - 2, n - 1} | extra | set(int(x) for x in rng.integers(0, n, size=48))
            qs = {0, 1, n - 1} | extra | set(int(x) for x in rng.integers(0, n, size=24))
            self.active[h] = np.array(sorted(x for x in act if 0 <= x < n), dtype=np.int64)
            self.queries[h] = np.array(sorted(x for x in qs if 0 <= x < n), dtype=np.int64)
            flat.append(h * n + self.active[h])
        rows = torch.from_numpy(np.unique(np.concatenate(flat))).cuda()
        vals = torch.randn((rows.numel(), d), dtype=td, device="cuda", generator=gen).mul_(kscale)
        self.k.view(-1, d)[rows] = vals
        torch.cuda.synchronize()

    def rows(self, t, h, idx):
        """Rows idx of head h of device tensor t, decoded exactly to float64."""
        import torch
        flat = torch.from_numpy(h * self.n + idx).cuda()
        return from_dev(t.view(-1, self.d)[flat].contiguous(), self.dtype)

    def free(self, torch):
        del self.q, self.k, self.v
        torch.cuda.empty_cache()


def _elu_ref(Q, Kc, Vc, act, qrows, causal):
    """Rows of eq. Attention_i over the active keys (Kc, Vc at rows act, sorted) for the query
    rows qrows (values Q): j over all active keys, or the active keys j <= i when causal."""
    d = Q.shape[1]
    out = np.empty_like(Q)
    if not causal:
        a = len(act)
        Qp = np.zeros((max(a, len(qrows)), d))
        Qp[:len(qrows)] = Q
        Kp = np.full((Qp.shape[0], d), INACTIVE_ELU)   # padding keys: features exactly 0
        Vp = np.zeros((Qp.shape[0], d))
        Kp[:a], Vp[:a] = Kc, Vc
        return oracle.rows(Qp, Kp, Vp, np.arange(len(qrows)), causal=False)
    for r, i in enumerate(qrows):
        cnt = int(np.searchsorted(act, i, side="right"))   # active keys j <= i (row 0 is one)
        Qp = np.zeros((cnt, d))
        Qp[0] = Q[r]
        out[r] = oracle.rows(Qp, Kc[:cnt], Vc[:cnt], [0], causal=False)[0]
    return out


def _favor_ref(Q, Kc, Vc, act, qrows, W, scale, causal):
    if not causal:
        return favor.rows(Q, Kc, Vc, W, scale, np.arange(len(qrows)), causal=False)
    out = np.empty_like(Q)
    for r, i in enumerate(qrows):
        cnt = int(np.searchsorted(act, i, side="right"))
        out[r] = favor.rows(Q[r:r + 1], Kc[:cnt], Vc[:cnt], W, scale, [0], causal=False)[0]
    return out


def _check(case, out, ref_fn, tol, label, causal=False):
    import torch
    assert bool(torch.isfinite(out).all()), "%s: an output row was not written" % label
    worst = 0.0
    for h in case.heads:
        act, qrows = case.active[h], case.queries[h]
        Q = case.rows(case.q, h, qrows)
        Kc = case.rows(case.k, h, act)
        Vc = case.rows(case.v, h, act)
        g = case.rows(out, h, qrows)
        ref = ref_fn(Q, Kc, Vc, act, qrows)
        e = rowwise_err(g[None], ref[None]) if causal else normwise_err(g[None], ref[None])
        worst = max(worst, e)
        assert e <= tol, (label, h, e)
    print("%s: worst err %.3e over heads %s" % (label, worst, case.heads))


# ----------------------------------------------------------------------------- elu + 1
ELU_CASES = [(dt, d, lay) for dt in ("bf16", "f32") for d in (64, 128) for lay in ("long", "wide")]


@pytest.fixture(scope="module", params=ELU_CASES, ids=lambda c: "%s-d%d-%s" % c)
def elu_case(request, ea):
    import torch
    dtype, d, layout = request.param
    case = Case(torch, dtype, d, layout, seed=1000 + d + (7 if layout == "long" else 0),
                inactive=INACTIVE_ELU, qscale=d ** -0.5, kscale=d ** -0.5)
    yield case
    case.free(torch)


def test_maxsize_noncausal(ea, elu_case):
    import torch
    c = elu_case
    out = torch.full_like(c.q, float("nan"))
    say("maxsize noncausal GPU", c.dtype, c.d, c.B, c.H, c.n)
    ea.la_forward_noncausal(c.q, c.k, c.v, out=out)
    tol = TOL_BF16 if c.dtype == "bf16" else TOL_F32
    _check(c, out, lambda Q, K, V, a, r: _elu_ref(Q, K, V, a, r, False), tol, "noncausal %s d=%d" % (c.dtype, c.d))
    del out


def test_maxsize_causal(ea, elu_case):
    import torch
    c = elu_case
    chunk = 64 if (c.dtype == "f32" and c.d == 128) else 128
    seg_len = ea.la_causal_plan(c.B, c.H, c.n, c.d, chunk, c.q.dtype)
    for h in c.heads:  # query rows on both sides of every segment boundary
        extra = [x for s in range(1, 17) for x in (s * seg_len - 1, s * seg_len) if x < c.n]
        c.queries[h] = np.unique(np.concatenate([c.queries[h], np.array(extra, dtype=np.int64)]))
    out = torch.full_like(c.q, float("nan"))
    say("maxsize causal GPU", c.dtype, c.d, c.B, c.H, c.n, "chunk", chunk, "seg_len", seg_len)
    ea.la_forward_causal(c.q, c.k, c.v, chunk=chunk, out=out)
    tol = TOL_BF16 if c.dtype == "bf16" else TOL_F32
    _check(c, out, lambda Q, K, V, a, r: _elu_ref(Q, K, V, a, r, True), tol, "causal %s d=%d" % (c.dtype, c.d),
           causal=True)
    del out


def test_maxsize_causal_varlen(ea):
    """Two sequences of 4 heads (4.1M and 4.4M tokens, d = 128): the first sequence ends just
    below element 2^31, so the second sequence's heads run past it."""
    import torch
    d, H = 128, 4
    lens = [4_100_000 + 77, 4_400_000 + 5]
    cu = np.array([0, lens[0], lens[0] + lens[1]], dtype=np.int64)
    rows_total = H * int(cu[-1])
    assert rows_total * d > (1 << 31) and H * lens[0] * d < (1 << 31)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(77)
    rng = np.random.default_rng(77)
    say("maxsize varlen inputs", lens, H, d)
    q = torch.randn((rows_total, d), dtype=torch.bfloat16, device="cuda", generator=gen).mul_(d ** -0.5)
    v = torch.randn((rows_total, d), dtype=torch.bfloat16, device="cuda", generator=gen)
    k = torch.full((rows_total, d), INACTIVE_ELU, dtype=torch.bfloat16, device="cuda")
    checks = []  # (first row of the head, its length, active rows, query rows)
    firsts = []
    for s in range(2):
        for h in range(H):
            first, ns = H * int(cu[s]) + h * lens[s], lens[s]
            firsts.append(first)
            if (s, h) in ((0, 0), (1, 0), (1, H - 1)):
                act = np.unique(np.concatenate([[0, ns - 1], rng.integers(0, ns, size=40)])).astype(np.int64)
                qs = np.unique(np.concatenate([[0, 1, ns - 1], rng.integers(0, ns, size=20)])).astype(np.int64)
                checks.append((first, act, qs))
    flat = np.unique(np.concatenate([np.array(firsts, dtype=np.int64)] + [f + a for f, a, _ in checks]))
    idx = torch.from_numpy(flat).cuda()
    k[idx] = torch.randn((idx.numel(), d), dtype=torch.bfloat16, device="cuda", generator=gen).mul_(d ** -0.5)
    out = torch.full_like(q, float("nan"))
    say("maxsize varlen causal GPU")
    ea.la_forward_causal_varlen(q, k, v, cu, H, chunk=128, out=out)
    assert bool(torch.isfinite(out).all())
    rowsof = lambda t, r: from_dev(t[torch.from_numpy(r).cuda()].contiguous(), "bf16")
    for first, act, qs in checks:
        ref = _elu_ref(rowsof(q, first + qs), rowsof(k, first + act), rowsof(v, first + act), act, qs, True)
        e = rowwise_err(rowsof(out, first + qs)[None], ref[None])
        assert e <= TOL_BF16, (first, e)
    del q, k, v, out
    torch.cuda.empty_cache()


def test_maxsize_decode(ea):
    """One decode step of 139,264 heads at d = 128: the fp32 state is 9.1 GB, past 2^31
    elements; sampled heads on both sides of the critical offsets against the oracle's step."""
    import torch
    B, H, d = 4352, 32, 128
    bh = B * H
    assert bh * d * d > (1 << 31)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(99)
    say("maxsize decode inputs", B, H, d)
    S = torch.randn((B, H, d, d), dtype=torch.float32, device="cuda", generator=gen).mul_(0.1)
    z = torch.rand((B, H, d), dtype=torch.float32, device="cuda", generator=gen).add_(1.0)
    q, k, v = (torch.randn((B, H, d), dtype=torch.bfloat16, device="cuda", generator=gen).mul_(d ** -0.5)
               for _ in range(3))
    heads = sorted({0, bh - 1} | {x for e in CRIT for x in (e // (d * d) - 1, e // (d * d)) if 0 <= x < bh}
                   | set(int(x) for x in np.random.default_rng(99).integers(0, bh, size=8)))
    hs = torch.tensor(heads, device="cuda")
    S0 = S.view(bh, d, d)[hs].double().cpu().numpy()
    z0 = z.view(bh, d)[hs].double().cpu().numpy()
    out = torch.full_like(q, float("nan"))
    say("maxsize decode GPU")
    ea.la_decode_step(q, k, v, S, z, out=out)
    assert bool(torch.isfinite(out).all())
    Qh = from_dev(q.view(bh, d)[hs].contiguous(), "bf16")
    Kh = from_dev(k.view(bh, d)[hs].contiguous(), "bf16")
    Vh = from_dev(v.view(bh, d)[hs].contiguous(), "bf16")
    ro, Sr, zr = oracle.decode_step(Qh, Kh, Vh, S0, z0)
    assert normwise_err(from_dev(out.view(bh, d)[hs].contiguous(), "bf16"), ro, head_axes_last=1) <= TOL_BF16
    assert normwise_err(S.view(bh, d, d)[hs].double().cpu().numpy(), Sr) <= TOL_F32
    assert normwise_err(z.view(bh, d)[hs].double().cpu().numpy(), zr, head_axes_last=1) <= TOL_F32
    del S, z, q, k, v, out
    torch.cuda.empty_cache()


# ----------------------------------------------------------------------------- FAVOR+
FAVOR_CASES = [(128, 128, "long"), (64, 256, "wide")]


@pytest.fixture(scope="module", params=FAVOR_CASES, ids=lambda c: "d%d-m%d-%s" % c)
def favor_case(request, ea):
    import torch
    d, m, layout = request.param
    case = Case(torch, "bf16", d, layout, seed=2000 + d + m, inactive=INACTIVE_FAVOR, qscale=1.0, kscale=1.0)
    case.m = m
    case.w = torch.from_numpy(projection(2100 + m, m, d, "bf16").view(np.int16)).view(torch.bfloat16).cuda()
    case.W = from_dev(case.w, "bf16")
    yield case
    case.free(torch)


def test_maxsize_favor_noncausal(ea, favor_case):
    import torch
    c = favor_case
    scale = c.d ** -0.25
    out = torch.full_like(c.q, float("nan"))
    say("maxsize favor noncausal GPU", c.d, c.m, c.B, c.H, c.n)
    ea.la_favor_forward_noncausal(c.q, c.k, c.v, c.w, scale, out=out)
    _check(c, out, lambda Q, K, V, a, r: _favor_ref(Q, K, V, a, r, c.W, scale, False), TOL_BF16,
           "favor noncausal d=%d m=%d" % (c.d, c.m))
    del out


def test_maxsize_favor_causal(ea, favor_case):
    import torch
    c = favor_case
    scale = c.d ** -0.25
    out = torch.full_like(c.q, float("nan"))
    say("maxsize favor causal GPU", c.d, c.m, c.B, c.H, c.n)
    ea.la_favor_forward_causal(c.q, c.k, c.v, c.w, scale, chunk=64, out=out)
    _check(c, out, lambda Q, K, V, a, r: _favor_ref(Q, K, V, a, r, c.W, scale, True), TOL_BF16,
           "favor causal d=%d m=%d" % (c.d, c.m), causal=True)
    del out


def test_maxsize_favor_decode(ea):
    """One FAVOR+ decode step of 139,264 heads (d = m = 128, a 9.1 GB state) from a given state
    with log-scale 0; sampled heads against the oracle's step."""
    import torch
    B, H, d, m = 4352, 32, 128, 128
    bh = B * H
    gen = torch.Generator(device="cuda")
    gen.manual_seed(98)
    say("maxsize favor decode inputs", B, H, d, m)
    S = torch.randn((B, H, m, d), dtype=torch.float32, device="cuda", generator=gen).mul_(0.1)
    z = torch.rand((B, H, m), dtype=torch.float32, device="cuda", generator=gen).add_(1.0)
    c = torch.zeros((B, H), dtype=torch.float32, device="cuda")
    q, k, v = (torch.randn((B, H, d), dtype=torch.bfloat16, device="cuda", generator=gen) for _ in range(3))
    w = torch.from_numpy(projection(2200, m, d, "bf16").view(np.int16)).view(torch.bfloat16).cuda()
    W = from_dev(w, "bf16")
    scale = d ** -0.25
    heads = sorted({0, bh - 1} | {x for e in CRIT for x in (e // (m * d) - 1, e // (m * d)) if 0 <= x < bh}
                   | set(int(x) for x in np.random.default_rng(98).integers(0, bh, size=8)))
    hs = torch.tensor(heads, device="cuda")
    S0 = S.view(bh, m, d)[hs].double().cpu().numpy()
    z0 = z.view(bh, m)[hs].double().cpu().numpy()
    out = torch.full_like(q, float("nan"))
    say("maxsize favor decode GPU")
    ea.la_favor_decode_step(q, k, v, w, S, z, c, scale, out=out)
    assert bool(torch.isfinite(out).all())
    Qh = from_dev(q.view(bh, d)[hs].contiguous(), "bf16")
    Kh = from_dev(k.view(bh, d)[hs].contiguous(), "bf16")
    Vh = from_dev(v.view(bh, d)[hs].contiguous(), "bf16")
    ro, Sr, zr = favor.decode_step(Qh, Kh, Vh, S0, z0, W, scale)
    assert normwise_err(from_dev(out.view(bh, d)[hs].contiguous(), "bf16"), ro, head_axes_last=1) <= TOL_BF16
    cs = np.exp(c.view(bh)[hs].double().cpu().numpy())
    St = S.view(bh, m, d)[hs].double().cpu().numpy() * cs[:, None, None]
    zt = z.view(bh, m)[hs].double().cpu().numpy() * cs[:, None]
    assert normwise_err(St, Sr) <= 1e-4
    assert normwise_err(zt, zr, head_axes_last=1) <= 1e-4
    del S, z, c, q, k, v, out
    torch.cuda.empty_cache()
