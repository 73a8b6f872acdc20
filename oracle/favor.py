"""fp64 oracle for linear attention with the FAVOR+ feature map (positive random features).

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may import it.

What the pages fix.  "Efficient Transformers: Linear Attention and Flash Attention"
(section "Linear attention: reordering the matmuls, not shrinking them") names FAVOR+ from
Choromanski et al., "Rethinking Attention with Performers" (ICLR 2021), as the alternative
to elu + 1: non-negative random features whose inner products approximate the softmax
kernel exp(x . y), used in the same reassociated attention (Active recall A4 asks for a
non-negative feature map so that the normaliser stays positive).  The pages give no formula.
The reading taken here is the published positive random feature map of that paper:

    phi(x) = exp(W x' - |x'|^2 / 2) / sqrt(m),   x' = scale * x,

with W [m, d] the projection whose rows are Gaussian directions (drawn i.i.d. N(0, I_d), or
in orthogonal blocks with chi-distributed lengths: ``orf_projection``).  For every x, y:
E_w[exp(w.x - |x|^2/2) exp(w.y - |y|^2/2)] = exp(x . y), so phi(x) . phi(y) estimates
exp(scale^2 x . y); scale = d^(-1/4) gives the kernel of softmax attention.

Attention with it is the definition of eq. Attention_i with this phi: out_i =
sum_j (phi(q_i).phi(k_j)) v_j / sum_j phi(q_i).phi(k_j) over all j (non-causal) or j <= i
(causal), and the recurrence of "The recurrent view" for the decode step (S += phi(k) v^T,
z += phi(k), then out = phi(q)^T S / phi(q)^T z).

Everything here is plain numpy in float64; a library matrix product is the only compound
step.  Pinned in ``tests/test_favor_oracle_pins.py`` (unbiasedness against the closed form
and its variance, orthogonality of the blocks, the zero- and one-feature closed forms,
convergence to softmax attention, associativity, the causal mask and the recurrence).
"""
from __future__ import annotations

import math

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def features(x, W, scale):
    """phi(x) for x [..., d] and projection W [m, d]: exp(W x' - |x'|^2/2) / sqrt(m), x' =
    scale * x.  Returns [..., m]."""
    x = _f64(x) * float(scale)
    W = _f64(W)
    m = W.shape[0]
    proj = x @ W.T                                   # w_i . x'
    half_norm = 0.5 * np.sum(x * x, axis=-1, keepdims=True)
    return np.exp(proj - half_norm) / math.sqrt(m)


def orf_projection(gauss_blocks, gauss_lengths):
    """Orthogonal random projection from pre-drawn Gaussians.

    gauss_blocks [nb, d, d]: i.i.d. N(0, 1) blocks; gauss_lengths [nb, d, d]: i.i.d. N(0, 1)
    vectors whose norms give the row lengths.  Each block's rows are the orthonormal basis of
    its Gaussian block (QR), each row then stretched to the length of an independent Gaussian
    vector in R^d, so that every row is marginally N(0, I_d) and the rows of a block are
    orthogonal.  Returns [nb * d, d]; the caller keeps the first m rows."""
    G = _f64(gauss_blocks)
    L = _f64(gauss_lengths)
    rows = []
    for b in range(G.shape[0]):
        q, r = np.linalg.qr(G[b])
        # fix the sign ambiguity of QR so that the basis is a function of the draw
        q = q * np.sign(np.diag(r))[None, :]
        lengths = np.linalg.norm(L[b], axis=1)
        rows.append(q.T * lengths[:, None])
    return np.concatenate(rows, axis=0)


def noncausal(q, k, v, W, scale, return_state=False):
    """Non-causal attention with phi = FAVOR+ features, in the reassociated order:
    S = phi(K)^T V, z = phi(K)^T 1, out = phi(Q) S / phi(Q) z.  q, k, v [..., n, d]."""
    fq = features(q, W, scale)
    fk = features(k, W, scale)
    S = np.swapaxes(fk, -1, -2) @ _f64(v)
    z = fk.sum(axis=-2)
    num = fq @ S
    den = np.einsum("...nm,...m->...n", fq, z)
    out = num / den[..., None]
    if return_state:
        return out, S, z
    return out


def quadratic(q, k, v, W, scale, causal):
    """The explicit n x n form: A = phi(Q) phi(K)^T (lower triangle with the diagonal when
    causal), out = A V / A 1."""
    fq = features(q, W, scale)
    fk = features(k, W, scale)
    A = fq @ np.swapaxes(fk, -1, -2)
    if causal:
        n = A.shape[-1]
        A = A * np.tril(np.ones((n, n)))
    return (A @ _f64(v)) / A.sum(axis=-1, keepdims=True)


def rows(q, k, v, W, scale, row_idx, causal):
    """Selected output rows of ONE head ([n, d] inputs) by the definition: out_i = sum_j w_ij v_j /
    sum_j w_ij, w_ij = phi(q_i) . phi(k_j), over all j (or j <= i when causal)."""
    fk = features(k, W, scale)
    v = _f64(v)
    idx = np.asarray(row_idx, dtype=np.int64)
    fq = features(_f64(q)[idx], W, scale)
    out = np.empty((idx.size, v.shape[-1]))
    for r, i in enumerate(idx):
        end = int(i) + 1 if causal else fk.shape[0]
        wts = fk[:end] @ fq[r]
        out[r] = (wts @ v[:end]) / wts.sum()
    return out


def decode_step(q, k, v, S, z, W, scale):
    """One step of the recurrence per head, update first: S + phi(k) v^T, z + phi(k), then
    out = phi(q)^T S / phi(q)^T z.  q, k, v [..., d]; S [..., m, d]; z [..., m].  Returns
    (out, S_new, z_new); the inputs are not modified."""
    fk = features(k, W, scale)
    fq = features(q, W, scale)
    S2 = _f64(S) + fk[..., :, None] * _f64(v)[..., None, :]
    z2 = _f64(z) + fk
    num = np.einsum("...m,...mc->...c", fq, S2)
    den = np.einsum("...m,...m->...", fq, z2)
    return num / den[..., None], S2, z2


def causal_recurrent(q, k, v, W, scale, s0=None, z0=None, return_state=False):
    """Causal attention by the token-by-token recurrence (decode_step over the tokens), from
    the state (s0, z0) (zero when absent).  q, k, v [..., n, d]."""
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    m = _f64(W).shape[0]
    lead = q.shape[:-2]
    n, d = q.shape[-2], q.shape[-1]
    S = np.zeros(lead + (m, d)) if s0 is None else _f64(s0).copy()
    z = np.zeros(lead + (m,)) if z0 is None else _f64(z0).copy()
    out = np.empty(lead + (n, d))
    for i in range(n):
        out[..., i, :], S, z = decode_step(q[..., i, :], k[..., i, :], v[..., i, :], S, z, W, scale)
    if return_state:
        return out, S, z
    return out


def state(k, v, W, scale):
    """(S, z) = (phi(K)^T V, phi(K)^T 1) over the tokens of k, v [..., n, d]."""
    fk = features(k, W, scale)
    return np.swapaxes(fk, -1, -2) @ _f64(v), fk.sum(axis=-2)


def softmax_attention(q, k, v, scale, causal=False):
    """Softmax attention with logits scale^2 q . k (the kernel FAVOR+ estimates); textbook
    form, used only to pin the estimator's limit."""
    q = _f64(q)
    k = _f64(k)
    logits = (scale * scale) * (q @ np.swapaxes(k, -1, -2))
    if causal:
        n = logits.shape[-1]
        logits = np.where(np.tril(np.ones((n, n))) > 0, logits, -np.inf)
    logits = logits - logits.max(axis=-1, keepdims=True)
    p = np.exp(logits)
    return (p @ _f64(v)) / p.sum(axis=-1, keepdims=True)
