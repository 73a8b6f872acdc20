"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every symbol that
include/*.h declares, and rejects bad arguments before launching anything.

The validation calls pass fake (never dereferenced) addresses: every case here fails or
returns before the library touches HIP.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "linattn.h")
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include")) if f.endswith(".h"))

ea = pytest.importorskip("efficient_attention_amd")


def _lib():
    if not os.path.exists(ea.LIB_PATH):
        pytest.fail("liblinattn.so is not built; run `python -m efficient_attention_amd.build`")
    return ea.load()


def _declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names.update(re.findall(r"\b(la_[a-z_]+)\s*\(", text))
    return sorted(names)


def _header_constant(name):
    m = re.search(r"\b%s\s*=\s*(-?\d+)" % name, open(HEADER).read())
    if m is None:
        m = re.search(r"#define\s+%s\s+(\d+)" % name, open(HEADER).read())
    return int(m.group(1))


def test_exports_every_declared_symbol():
    lib = _lib()
    declared = _declared_functions()
    assert set(declared) == set(ea.EXPORTS), declared
    for name in declared:
        assert hasattr(lib, name), name


def test_abi_version_and_status_strings():
    assert ea.la_abi_version() == _header_constant("LA_ABI_VERSION")
    for code in range(-9, 1):
        s = ea.la_status_string(code)
        assert isinstance(s, str) and s
    assert ea.la_status_string(-1000) == "unknown status"


def test_workspace_sizes():
    assert ea.la_noncausal_workspace_bytes(0, 4, 100, 64, 1) == 0
    assert ea.la_noncausal_workspace_bytes(2, 4, 0, 64, 1) == 0
    assert ea.la_noncausal_workspace_bytes(2, 4, 100, 96, 1) == 0       # unsupported d
    w = ea.la_noncausal_workspace_bytes(8, 16, 16384, 64, 1)
    # at least one fp32 [KV | z] state per head
    assert w >= 8 * 16 * (64 * 64 + 64) * 4
    assert ea.la_causal_workspace_bytes(1, 1, 10, 64, 96, 1) == 0       # unsupported chunk
    # many heads: one segment per head, no workspace
    assert ea.la_causal_workspace_bytes(64, 8, 4096, 64, 64, 1) == 0
    # one head: the sequence is cut into segments, whose state sums need a workspace
    assert ea.la_causal_workspace_bytes(1, 1, 4096, 64, 64, 0) > 0


def test_noncausal_plans_of_the_workload_shapes():
    # The stage-1 plan aims at the stage-1 kernel's workgroup slots on 256 compute units: 512
    # workgroups, 1024 for the fp32 kernel at d = 64.  128 heads therefore take 4 (or 8) slices
    # each, and each slice writes one fp32 [KV | z] partial; for bf16 at d = 64 each head's
    # partials are then added into one more state.
    E64, E128 = (64 * 64 + 64) * 4, (128 * 128 + 128) * 4
    assert ea.la_noncausal_workspace_bytes(8, 16, 16384, 64, 1) == 128 * 4 * E64 + 128 * E64
    assert ea.la_noncausal_workspace_bytes(8, 16, 16384, 64, 0) == 128 * 8 * E64
    assert ea.la_noncausal_workspace_bytes(8, 16, 16384, 128, 1) == 128 * 4 * E128
    assert ea.la_noncausal_workspace_bytes(8, 16, 16384, 128, 0) == 128 * 4 * E128
    # enough heads for one slice each: the states themselves, nothing added afterwards
    assert ea.la_noncausal_workspace_bytes(64, 16, 4096, 64, 1) == 1024 * E64
    assert ea.la_noncausal_workspace_bytes(64, 32, 4096, 64, 0) == 2048 * E64


P = ctypes.c_void_p


def _nc(lib, q=0x1000, k=0x2000, v=0x3000, out=0x4000, B=1, H=1, n=8, d=64, dtype=1,
        ws=0x100000, wsb=1 << 30):
    return lib.la_forward_noncausal(P(q), P(k), P(v), P(out), B, H, n, d, dtype, P(ws), wsb, None)


def _ca(lib, q=0x1000, k=0x2000, v=0x3000, out=0x4000, B=1, H=1, n=8, d=64, chunk=64, dtype=1,
        ws=0x100000, wsb=1 << 30):
    return lib.la_forward_causal(P(q), P(k), P(v), P(out), B, H, n, d, chunk, dtype, P(ws), wsb, None)


def _dec(lib, q=0x1000, k=0x2000, v=0x3000, S=0x10000, z=0x20000, out=0x4000, B=1, H=1, d=64, dtype=1):
    return lib.la_decode_step(P(q), P(k), P(v), P(S), P(z), P(out), B, H, d, dtype, None)


def test_validation_noncausal():
    lib = _lib()
    assert _nc(lib, dtype=7) == -3
    assert _nc(lib, n=-1) == -2
    assert _nc(lib, B=1 << 40, H=1 << 40) == -2
    assert _nc(lib, d=96) == -4
    assert _nc(lib, n=0, q=0, k=0, v=0, out=0) == 0          # empty: no-op, no pointers needed
    assert _nc(lib, B=0) == 0
    assert _nc(lib, q=0) == -1
    assert _nc(lib, out=0) == -1
    assert _nc(lib, k=0x2008) == -5                          # misaligned
    assert _nc(lib, ws=0) == -6
    assert _nc(lib, wsb=16) == -6
    assert _nc(lib, out=0x1000) == -7                        # out aliases q
    assert _nc(lib, out=0x100000 + 64) == -7                  # out inside the workspace


def test_validation_noncausal_noalloc():
    # every check happens before the library looks up its scratch (no HIP call on these paths)
    lib = _lib()
    na = lambda q=0x1000, k=0x2000, v=0x3000, out=0x4000, B=1, H=1, n=8, d=64, dtype=1: \
        lib.la_forward_noncausal_noalloc(P(q), P(k), P(v), P(out), B, H, n, d, dtype, None)
    assert na(dtype=7) == -3
    assert na(n=-1) == -2
    assert na(d=96) == -4
    assert na(n=0, q=0, out=0) == 0
    assert na(q=0) == -1
    assert na(out=0x4008) == -5
    assert na(out=0x1000) == -7
    limit = ea.LA_NOALLOC_SCRATCH_BYTES
    assert limit == _header_shift_constant("LA_NOALLOC_SCRATCH_BYTES")
    # a shape whose partials exceed the scratch is refused with the workspace error
    big = (4096, 2, 64)  # B*H = 8192 heads at d = 128: one 66 KB state each
    assert ea.la_noncausal_workspace_bytes(big[0], big[1], big[2], 128, 1) > limit
    far = 1 << 36  # inputs and output far apart (no overlap)
    assert na(q=far, k=2 * far, v=3 * far, out=4 * far, B=big[0], H=big[1], n=big[2], d=128) == -6
    # the bench's non-causal workload fits
    assert ea.la_noncausal_workspace_bytes(8, 16, 16384, 64, 1) <= limit
    assert ea.la_noncausal_workspace_bytes(4, 32, 16384, 128, 1) <= limit


def _header_shift_constant(name):
    m = re.search(r"#define\s+%s\s+\(\(size_t\)(\d+)\s*<<\s*(\d+)\)" % name, open(HEADER).read())
    return int(m.group(1)) << int(m.group(2))


def test_validation_causal():
    lib = _lib()
    assert _ca(lib, chunk=96) == -4
    assert _ca(lib, chunk=128, d=128, dtype=0) == -4          # fp32 (d, chunk) = (128, 128)
    assert _ca(lib, d=32) == -4
    assert _ca(lib, n=0, q=0) == 0
    assert _ca(lib, v=0) == -1
    assert _ca(lib, out=0x4004) == -5
    assert _ca(lib, n=4096, ws=0) == -6                      # one head -> needs a workspace
    assert _ca(lib, out=0x2000) == -7


def _cs(lib, q=0x1000, k=0x2000, v=0x3000, out=0x4000, S0=0, z0=0, Sn=0, zn=0, B=1, H=1, n=8, d=64,
        chunk=64, dtype=1, ws=0x100000, wsb=1 << 30):
    return lib.la_forward_causal_state(P(q), P(k), P(v), P(out), P(S0 or None), P(z0 or None), P(Sn or None),
                                       P(zn or None), B, H, n, d, chunk, dtype, P(ws), wsb, None)


def test_validation_causal_state():
    lib = _lib()
    S, Z = 0x200000, 0x300000
    assert _cs(lib, S0=S) == -1                                # z0 missing
    assert _cs(lib, Sn=S) == -1                                # zn missing
    assert _cs(lib, S0=S, z0=Z, Sn=S, zn=Z + 0x40000) == -7    # final state over the initial one
    assert _cs(lib, Sn=S, zn=S + 0x100) == -7                  # Sn and zn overlap
    assert _cs(lib, Sn=S + 4, zn=Z) == -5                      # misaligned
    assert _cs(lib, Sn=S, zn=Z, out=S) == -7                   # out over the final state
    assert _cs(lib, Sn=S, zn=Z, k=Z) == -7                     # final state over an input
    assert _cs(lib, S0=S, z0=Z, out=Z) == -7                   # out over the initial state
    assert _cs(lib, B=0, S0=S) == -1                           # pairs are checked first
    assert _cs(lib, B=0, Sn=S, zn=Z) == 0                      # no heads: nothing to write
    assert _cs(lib, chunk=96, Sn=S, zn=Z) == -4


def _cu(vals):
    return (ctypes.c_int64 * len(vals))(*vals)


def test_validation_varlen():
    lib = _lib()
    nc = lambda cu, nseq, H=2, d=64, dtype=1, ws=0x100000, wsb=1 << 30, q=0x1000: lib.la_forward_noncausal_varlen(
        P(q), P(0x2000), P(0x3000), P(0x4000), cu, nseq, H, d, dtype, P(ws), wsb, None)
    ca = lambda cu, nseq, chunk=64, H=2, d=64, dtype=1: lib.la_forward_causal_varlen(
        P(0x1000), P(0x2000), P(0x3000), P(0x4000), cu, nseq, H, d, chunk, dtype, P(0x100000), 1 << 30, None)
    assert nc(None, 2) == -1                                   # no offsets
    assert nc(_cu([1, 5, 9]), 2) == -2                         # not starting at 0
    assert nc(_cu([0, 5, 3]), 2) == -2                         # decreasing
    assert nc(_cu(list(range(258))), 257) == -4                # more than 256 sequences
    assert nc(_cu([0, 5, 9]), 2, d=96) == -4
    assert nc(_cu([0, 0, 0]), 2, q=0) == 0                     # no tokens: nothing to do
    assert nc(_cu([0, 5, 9]), 2, q=0) == -1
    assert nc(_cu([0, 5, 9]), 2, ws=0) == -6
    assert ca(_cu([0, 5, 9]), 2, chunk=96) == -4
    assert ca(_cu([0, 5, 3]), 2) == -2
    # workspace: planned for the longest sequence
    cu = [0, 100, 100, 5000]
    assert ea.la_noncausal_varlen_workspace_bytes(cu, 4, 64, 1) == ea.la_noncausal_workspace_bytes(3, 4, 4900, 64, 1)
    assert ea.la_causal_varlen_workspace_bytes([0, 70000], 1, 128, 128, 1) == ea.la_causal_workspace_bytes(1, 1, 70000, 128, 128, 1)
    # masked decode needs its flags
    assert lib.la_decode_step_masked(P(0x1000), P(0x2000), P(0x3000), P(0x10000), P(0x20000), P(0x4000), None,
                                     1, 1, 64, 1, None) == -1


def test_validation_decode():
    lib = _lib()
    assert _dec(lib, dtype=5) == -3
    assert _dec(lib, d=100) == -4
    assert _dec(lib, B=0, q=0) == 0
    assert _dec(lib, S=0) == -1
    assert _dec(lib, z=0x20004) == -5
    assert _dec(lib, out=0x10000) == -7                      # out aliases S
    assert _dec(lib, z=0x10000 + 64) == -7                   # z inside S
    assert _dec(lib, S=0x1000) == -7                         # S over q (written in place while q is read)
    assert _dec(lib, z=0x3000) == -7                         # z over v
    # masked: B and H are validated before the flags are looked at
    mk = lambda B, H, act: lib.la_decode_step_masked(P(0x1000), P(0x2000), P(0x3000), P(0x10000), P(0x20000),
                                                     P(0x4000), P(act), B, H, 64, 1, None)
    assert mk(1 << 40, 1 << 40, None) == -2                  # B * H overflows: a shape error
    assert mk(-1, 2, None) == -2
    assert mk(0, 2, None) == 0                               # no heads: no flags needed
    assert mk(1, 1, 0x10000) == -7                           # flags inside S


def test_dtype_codes_outside_the_enum():
    # la_dtype_t covers every int, so any other code is reported, never assumed valid
    lib = _lib()
    for code in (2, 7, -1, -(1 << 31), (1 << 31) - 1):
        assert _nc(lib, dtype=code) == -3
        assert _dec(lib, dtype=code) == -3


def test_segment_sums_shape_is_checked():
    # the binding of la_causal_segments rejects sums of the wrong shape before the library reads
    # them (the kernel reads [B][H][ceil(n / seg_len) - 1][d*d + d] floats)
    torch = pytest.importorskip("torch")
    chk = ea._binding._check_segment_sums
    cpu = torch.device("cpu")
    B, H, n, d, seg = 2, 3, 1000, 64, 256                      # 4 segments: 3 leading sums
    good = torch.zeros((B, H, 3, d * d + d), dtype=torch.float32)
    chk(good, B, H, n, d, seg, cpu)
    for bad in (torch.zeros((B, H, 4, d * d + d)),              # la_state_sums(..., nseg=4) layout
                torch.zeros((B, H, 2, d * d + d)),              # too few: reads past the end
                torch.zeros((B, H, 3, d * d)),                  # z missing
                torch.zeros((B, H, 3, d * d + d), dtype=torch.float64),
                torch.zeros((H, B, 3, d * d + d)).transpose(0, 1),  # not contiguous
                None):
        with pytest.raises(ValueError):
            chk(bad, B, H, n, d, seg, cpu)
    chk(None, B, H, 200, d, seg, cpu)                           # one segment: no sums
    with pytest.raises(ValueError):
        chk(good, B, H, 200, d, seg, cpu)
    with pytest.raises(ValueError):
        chk(good, B, H, n, d, 0, cpu)


def test_causal_plan_and_stage_validation():
    lib = _lib()
    assert ea.la_causal_plan(4, 32, 65536, 128, 128, 1) == 32768     # 2 segments per head
    assert ea.la_causal_plan(64, 8, 4096, 64, 64, 1) == 4096         # batch fills the GPU
    seg = ea.la_causal_plan(1, 1, 4096, 64, 64, 0)
    assert seg % 64 == 0 and 64 <= seg < 4096
    out = ctypes.c_int64(0)
    assert lib.la_causal_plan(1, 1, 100, 64, 96, 1, ctypes.byref(out)) == -4
    assert lib.la_causal_plan(1, 1, 100, 64, 64, 1, None) == -1
    # la_state_sums
    ss = lambda **kw: lib.la_state_sums(P(kw.get("k", 0x2000)), P(kw.get("v", 0x3000)),
                                        P(kw.get("sums", 0x80000)), 1, 1, kw.get("n", 1000), 64, 1,
                                        kw.get("seg_len", 100), kw.get("nseg", 3),
                                        P(kw.get("ws", 0x900000)), kw.get("wsb", 1 << 30), None)
    assert ss(nseg=0) == -2
    assert ss(seg_len=0) == -2
    assert ss(nseg=11) == -2                                  # segment 10 would start at n
    assert ss(sums=0) == -1
    assert ss(sums=0x80004) == -5
    assert ss(sums=0x2000) == -7
    assert ss(n=0, k=0) == 0
    assert ea.la_state_sums_workspace_bytes(1, 1, 1000, 64, 1, 50, 3) == 0        # one tile, one slice each
    assert ea.la_state_sums_workspace_bytes(1, 1, 100000, 64, 1, 50000, 2) > 0    # split slices
    # la_causal_segments
    cs = lambda **kw: lib.la_causal_segments(P(kw.get("q", 0x1000)), P(0x2000), P(0x3000), P(kw.get("out", 0x4000)),
                                             P(kw.get("sums", 0x80000)), 1, 1, kw.get("n", 1000), 64,
                                             kw.get("chunk", 64), 1, kw.get("seg_len", 128), None)
    assert cs(seg_len=100) == -2                              # not a multiple of chunk
    assert cs(chunk=96) == -4
    assert cs(sums=0) == -1                                   # several segments need sums
    assert cs(out=0x80000) == -7                              # out overlaps sums
    assert cs(n=0, q=0) == 0


def _fnc(lib, q=0x1000, k=0x2000, v=0x3000, w=0x5000, out=0x4000, B=1, H=1, n=8, d=64, m=128,
         scale=0.35, dtype=1, ws=0x100000, wsb=1 << 30):
    return lib.la_favor_forward_noncausal(P(q), P(k), P(v), P(w), P(out), B, H, n, d, m, scale, dtype,
                                          P(ws), wsb, None)


def _fdec(lib, q=0x1000, k=0x2000, v=0x3000, w=0x5000, S=0x10000, z=0x80000, c=0x90000, out=0x4000,
          B=1, H=1, d=64, m=128, scale=0.35, dtype=1):
    return lib.la_favor_decode_step(P(q), P(k), P(v), P(w), P(S), P(z), P(c), P(out), B, H, d, m, scale,
                                    dtype, None)


def test_validation_favor():
    lib = _lib()
    assert _fnc(lib, dtype=0) == -4                           # fp32: not supported for FAVOR+
    assert _fnc(lib, dtype=9) == -3
    assert _fnc(lib, d=128, m=256) == -4                       # m * d above 16384
    assert _fnc(lib, m=96) == -4
    assert _fnc(lib, m=-1) == -2
    assert _fnc(lib, scale=0.0) == -9
    assert _fnc(lib, scale=float("inf")) == -9
    assert _fnc(lib, scale=float("nan")) == -9
    assert _fnc(lib, n=0, q=0, w=0) == 0                      # empty: no pointers needed
    assert _fnc(lib, w=0) == -1
    assert _fnc(lib, w=0x5008) == -5
    assert _fnc(lib, ws=0) == -6
    assert _fnc(lib, out=0x5000) == -7                         # out over the projection
    assert _fnc(lib, out=0x100000 + 256) == -7                 # out inside the workspace
    assert ea.la_favor_noncausal_workspace_bytes(1, 1, 8, 64, 128, 1) > 0
    assert ea.la_favor_noncausal_workspace_bytes(1, 1, 8, 64, 128, 0) == 0
    # one per-head record (S, z, c) at least
    assert ea.la_favor_noncausal_workspace_bytes(8, 16, 16384, 64, 256, 1) >= 128 * (256 * 64 + 256 + 4) * 4
    assert _fdec(lib, m=512) == -4
    assert _fdec(lib, scale=-1.0) == -9
    assert _fdec(lib, B=0, q=0) == 0
    assert _fdec(lib, c=0) == -1
    assert _fdec(lib, S=0x10004) == -5
    assert _fdec(lib, z=0x80002) == -5                         # z needs 4-byte alignment only
    assert _fdec(lib, out=0x10000) == -7                       # out over S
    assert _fdec(lib, c=0x10000 + 64) == -7                    # c inside S
    assert _fdec(lib, z=0x5000) == -7                          # z over the projection


def _fca(lib, q=0x1000, k=0x2000, v=0x3000, w=0x5000, out=0x4000, Sn=0, zn=0, cn=0, B=1, H=1, n=8, d=64,
         m=128, chunk=64, scale=0.35, dtype=1, ws=0x100000, wsb=1 << 30):
    return lib.la_favor_forward_causal(P(q), P(k), P(v), P(w), P(out), P(Sn or None), P(zn or None),
                                       P(cn or None), B, H, n, d, m, chunk, scale, dtype, P(ws), wsb, None)


def test_validation_favor_causal():
    lib = _lib()
    S, Z, C = 0x200000, 0x300000, 0x380000
    assert _fca(lib, chunk=96) == -4
    assert _fca(lib, chunk=128, m=256) == -4                   # chunk 128 needs m <= 128
    assert _fca(lib, dtype=0) == -4
    assert _fca(lib, d=128, m=256) == -4
    assert _fca(lib, scale=0.0) == -9
    assert _fca(lib, Sn=S) == -1                               # zn, cn missing
    assert _fca(lib, Sn=S, zn=Z) == -1
    assert _fca(lib, Sn=S + 4, zn=Z, cn=C) == -5
    assert _fca(lib, Sn=S, zn=Z + 2, cn=C) == -5
    assert _fca(lib, Sn=S, zn=S + 64, cn=C) == -7              # zn inside Sn
    assert _fca(lib, Sn=S, zn=Z, cn=C, out=Z) == -7            # out over zn
    assert _fca(lib, Sn=S, zn=Z, cn=C, k=C) == -7              # cn over an input
    assert _fca(lib, w=0) == -1
    assert _fca(lib, out=0x5000) == -7                         # out over the projection
    assert _fca(lib, B=0, Sn=S, zn=Z, cn=C) == 0               # no heads
    assert _fca(lib, n=4096, ws=0) == -6                       # one head: segments need sums
    assert ea.la_favor_causal_workspace_bytes(1, 1, 4096, 64, 128, 64, 1) > 0
    assert ea.la_favor_causal_workspace_bytes(64, 8, 4096, 64, 128, 64, 1) == 0  # one segment per head
    assert ea.la_favor_causal_workspace_bytes(1, 1, 4096, 64, 256, 128, 1) == 0  # invalid chunk
    assert ea.la_favor_causal_workspace_bytes(1, 1, 4096, 64, 128, 128, 1) > 0


def test_validation_ceilings():
    lib = _lib()
    assert lib.la_ceiling_copy(P(0x1000), P(0x100000), 100, None) == -2          # not a multiple of 16
    assert lib.la_ceiling_copy(P(0x1000), P(0x100000), 0, None) == 0
    assert lib.la_ceiling_copy(None, P(0x100000), 64, None) == -1
    assert lib.la_ceiling_copy(P(0x1008), P(0x100000), 64, None) == -5
    assert lib.la_ceiling_copy(P(0x1000), P(0x1010), 64, None) == -7            # overlap
    assert lib.la_ceiling_read_sink_words() > 0
    assert lib.la_ceiling_read(P(0x1000), 48, None, None) == -1
    assert lib.la_ceiling_read(P(0x1000), 48, P(0x1010), None) == -7
    cp = lambda d=128, seg=256, n=1000, out=0x4000000: lib.la_ceiling_causal_pattern(
        P(0x1000000), P(0x2000000), P(0x3000000), P(out), 1, 2, n, d, seg, None)
    assert cp(d=64) == -4
    assert cp(seg=100) == -2
    assert cp(n=0) == 0
    assert cp(out=0x1000000) == -7
