"""fp64 CPU oracle for kernelized linear attention (phi = elu + 1).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path (the HIP
library and its Python binding) never imports, links or runs anything here, and this
package imports nothing from the product path.

The arithmetic lives in ``linattn_oracle.c`` (plain single-threaded C, fp64, no BLAS, no
OpenMP, built ``-O2`` without fast-math).  This module only marshals numpy arrays into it.
Every function takes and returns float64 arrays; inputs that were generated in fp32 or
bf16 are decoded to float64 exactly by the caller before they get here.

Definitions followed: "Efficient Transformers: Linear Attention and Flash Attention"
(aicomputerinstitute.com, grade 12) -- eq. Attention_i in "Linear attention: reordering the
matmuls, not shrinking them", the two evaluation orders of "Worked example: the
reassociation trick, by hand", and the recurrence of "The recurrent view: attention as an
RNN".  Every oracle function is pinned by tests in ``tests/test_oracle_pins.py``; none is
parity-unpinned.

The FAVOR+ feature map (positive random features) lives in ``oracle/favor.py`` (numpy,
fp64), pinned by ``tests/test_favor_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "linattn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

PHI_ELU1 = 0
PHI_IDENTITY = 1

_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle into oracle/liboracle.so with gcc (-O2, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
               "-fno-fast-math", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=True)
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I = ctypes.c_int64
    C = ctypes.c_int
    lib.orc_phi.argtypes = [ctypes.c_double, C]
    lib.orc_phi.restype = ctypes.c_double
    lib.orc_noncausal_linear.argtypes = [P, P, P, P, I, I, I, C, P, P]
    lib.orc_quadratic.argtypes = [P, P, P, P, I, I, I, C, C, P]
    lib.orc_causal_recurrent.argtypes = [P, P, P, P, I, I, I, C, P, P, P, P]
    lib.orc_causal_chunked.argtypes = [P, P, P, P, I, I, I, I, C]
    lib.orc_decode_step.argtypes = [P, P, P, P, P, P, I, I, C]
    lib.orc_rows.argtypes = [P, P, P, P, I, I, P, I, C, C]
    lib.orc_phi_rows.argtypes = [P, P, I, C]
    lib.orc_state_accumulate.argtypes = [P, P, P, P, I, I, I, C]
    for name in ("orc_noncausal_linear", "orc_quadratic", "orc_causal_recurrent",
                 "orc_causal_chunked", "orc_decode_step", "orc_rows", "orc_phi_rows",
                 "orc_state_accumulate"):
        getattr(lib, name).restype = None
    _lib = lib
    return lib


def _f64(x):
    a = np.ascontiguousarray(x, dtype=np.float64)
    return a


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _heads(x):
    """View [..., n, d] as [BH, n, d]."""
    x = _f64(x)
    n, d = x.shape[-2], x.shape[-1]
    bh = int(np.prod(x.shape[:-2], dtype=np.int64))  # explicit, so that n = 0 works too
    return x.reshape(bh, n, d), x.shape


def phi(x, feature_map: int = PHI_ELU1):
    """phi applied elementwise (elu + 1, or the identity of the worked example)."""
    lib = _load()
    x = _f64(x)
    y = np.empty_like(x)
    lib.orc_phi_rows(_ptr(x), _ptr(y), x.size, feature_map)
    return y


def noncausal_linear(q, k, v, feature_map: int = PHI_ELU1, return_state: bool = False):
    """out_i = phi(q_i) KV / phi(q_i) z with KV = phi(K)^T V, z = sum_j phi(k_j), per head.

    q, k, v: [..., n, d].  Returns out ([..., n, d]) and, with return_state, (KV, z) of
    shapes [..., d, d] and [..., d]."""
    lib = _load()
    Q, shape = _heads(q)
    K, _ = _heads(k)
    V, _ = _heads(v)
    BH, n, d = Q.shape
    out = np.empty_like(Q)
    kv = np.empty((BH, d, d)) if return_state else None
    z = np.empty((BH, d)) if return_state else None
    lib.orc_noncausal_linear(_ptr(Q), _ptr(K), _ptr(V), _ptr(out), BH, n, d, feature_map,
                             _ptr(kv), _ptr(z))
    out = out.reshape(shape)
    if return_state:
        return out, kv.reshape(shape[:-2] + (d, d)), z.reshape(shape[:-2] + (d,))
    return out


def quadratic(q, k, v, causal: bool, feature_map: int = PHI_ELU1, return_weights: bool = False):
    """Explicit n x n form: W = phi(Q) phi(K)^T (masked to j <= i when causal), rows
    normalised by their sums, times V.  With return_weights also returns unnormalised W."""
    lib = _load()
    Q, shape = _heads(q)
    K, _ = _heads(k)
    V, _ = _heads(v)
    BH, n, d = Q.shape
    out = np.empty_like(Q)
    w = np.empty((BH, n, n)) if return_weights else None
    lib.orc_quadratic(_ptr(Q), _ptr(K), _ptr(V), _ptr(out), BH, n, d, int(bool(causal)),
                      feature_map, _ptr(w))
    out = out.reshape(shape)
    if return_weights:
        return out, w.reshape(shape[:-2] + (n, n))
    return out


def causal_recurrent(q, k, v, feature_map: int = PHI_ELU1, s0=None, z0=None,
                     return_state: bool = False):
    """Causal form by the token-by-token recurrence, optionally from an initial state
    (s0 [..., d, d], z0 [..., d]); with return_state also returns the final (S, z)."""
    lib = _load()
    Q, shape = _heads(q)
    K, _ = _heads(k)
    V, _ = _heads(v)
    BH, n, d = Q.shape
    out = np.empty_like(Q)
    S0 = _f64(s0).reshape(BH, d, d) if s0 is not None else None
    Z0 = _f64(z0).reshape(BH, d) if z0 is not None else None
    sf = np.empty((BH, d, d)) if return_state else None
    zf = np.empty((BH, d)) if return_state else None
    lib.orc_causal_recurrent(_ptr(Q), _ptr(K), _ptr(V), _ptr(out), BH, n, d, feature_map,
                             _ptr(S0), _ptr(Z0), _ptr(sf), _ptr(zf))
    out = out.reshape(shape)
    if return_state:
        return out, sf.reshape(shape[:-2] + (d, d)), zf.reshape(shape[:-2] + (d,))
    return out


def causal_chunked(q, k, v, chunk: int, feature_map: int = PHI_ELU1):
    """Causal form regrouped into chunks of `chunk` tokens (intra-chunk pairwise part plus
    the state carried from earlier chunks)."""
    lib = _load()
    if chunk < 1:
        raise ValueError("chunk must be >= 1")
    Q, shape = _heads(q)
    K, _ = _heads(k)
    V, _ = _heads(v)
    BH, n, d = Q.shape
    out = np.empty_like(Q)
    lib.orc_causal_chunked(_ptr(Q), _ptr(K), _ptr(V), _ptr(out), BH, n, d, chunk, feature_map)
    return out.reshape(shape)


def decode_step(q, k, v, S, z, feature_map: int = PHI_ELU1):
    """One recurrent step per head: S += phi(k) v^T, z += phi(k), out = phi(q)S / phi(q)z.

    q, k, v: [..., d]; S: [..., d, d]; z: [..., d].  Returns (out, S_new, z_new); the
    inputs are not modified."""
    lib = _load()
    qq = _f64(q)
    shape = qq.shape
    d = shape[-1]
    qq = qq.reshape(-1, d)
    kk = _f64(k).reshape(-1, d)
    vv = _f64(v).reshape(-1, d)
    BH = qq.shape[0]
    S2 = np.array(_f64(S).reshape(BH, d, d), copy=True)
    z2 = np.array(_f64(z).reshape(BH, d), copy=True)
    out = np.empty((BH, d))
    lib.orc_decode_step(_ptr(qq), _ptr(kk), _ptr(vv), _ptr(S2), _ptr(z2), _ptr(out), BH, d,
                        feature_map)
    return out.reshape(shape), S2.reshape(shape[:-1] + (d, d)), z2.reshape(shape)


def rows(q, k, v, row_idx, causal: bool, feature_map: int = PHI_ELU1):
    """Selected output rows of ONE head ([n, d] inputs) by the quadratic definition."""
    lib = _load()
    Q = _f64(q)
    K = _f64(k)
    V = _f64(v)
    n, d = Q.shape
    idx = np.ascontiguousarray(row_idx, dtype=np.int64)
    if idx.size and (idx.min() < 0 or idx.max() >= n):
        raise IndexError("row index out of range")
    phik = np.empty_like(K)
    lib.orc_phi_rows(_ptr(K), _ptr(phik), K.size, feature_map)
    out = np.empty((idx.size, d))
    lib.orc_rows(_ptr(Q), _ptr(phik), _ptr(V), _ptr(out), n, d,
                 idx.ctypes.data_as(ctypes.c_void_p), idx.size, int(bool(causal)), feature_map)
    return out


def state_accumulate(k, v, S=None, z=None, feature_map: int = PHI_ELU1):
    """(S, z) += (sum_j phi(k_j) v_j^T, sum_j phi(k_j)) over the tokens of k, v [..., n, d]."""
    lib = _load()
    K, shape = _heads(k)
    V, _ = _heads(v)
    BH, n, d = K.shape
    S2 = np.zeros((BH, d, d)) if S is None else np.array(_f64(S).reshape(BH, d, d), copy=True)
    z2 = np.zeros((BH, d)) if z is None else np.array(_f64(z).reshape(BH, d), copy=True)
    lib.orc_state_accumulate(_ptr(K), _ptr(V), _ptr(S2), _ptr(z2), BH, n, d, feature_map)
    return S2.reshape(shape[:-2] + (d, d)), z2.reshape(shape[:-2] + (d,))


def state_from_tokens_matmul(k, v, feature_map: int = PHI_ELU1):
    """(S, z) = (phi(K)^T V, sum_j phi(k_j)) per head for k, v [..., n, d], with the library
    fp64 matrix product as the one step (used to build large decode states quickly; pinned
    against state_accumulate)."""
    K = _f64(k)
    V = _f64(v)
    fk = phi(K, feature_map)
    S = np.matmul(np.swapaxes(fk, -1, -2), V)
    z = fk.sum(axis=-2)
    return S, z
