"""The C ABI on the host: the library loads, exports every function the
header declares, and rejects bad arguments before touching the GPU (every
call below fails validation, so no HIP work is enqueued)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qdecode.h")


def _lib():
    import quantized_decode_q4k_amd as qd
    if not os.path.exists(qd.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return qd, qd.lib()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(",
                       src, flags=re.M)
    return sorted(set(n for n in names if n.startswith(("q", "qd_"))))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ["qgemv_q4k", "qgemv_q6k", "qgemv_q8_0", "qffn_gate_up_act", "qgemm_prefill",
              "qdequant", "qdequant_bf16", "qd_status_str", "qd_row_bytes"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    qd, L = _lib()
    for n in declared_functions():
        assert hasattr(L, n), n
        assert n in qd.SIGNATURES, n


def test_block_sizes_and_row_bytes():
    qd, L = _lib()
    assert [L.qd_block_bytes(f) for f in (0, 1, 2)] == [144, 210, 34]
    assert [L.qd_block_elems(f) for f in (0, 1, 2)] == [256, 256, 32]
    assert L.qd_block_bytes(9) == 0
    assert L.qd_row_bytes(0, 2560) == 1440
    assert L.qd_row_bytes(1, 10240) == 8400
    assert L.qd_row_bytes(2, 96) == 102
    assert L.qd_row_bytes(0, 100) == 0
    assert L.qd_row_bytes(2, 0) == 0
    assert L.qd_version() >= 10000
    for s in range(8):
        assert isinstance(L.qd_status_str(s), bytes)


# fake device pointers: never dereferenced because validation fails first
A16 = 0x10000
A16b = 0x20000
A16c = 0x30000


@pytest.mark.parametrize("args,status", [
    ((0, A16, A16b, 4, 256, 1, None), 1),           # null W
    ((A16, 0, A16b, 4, 256, 1, None), 1),           # null x
    ((A16, A16b, 0, 4, 256, 1, None), 1),           # null y
    ((A16, A16b, A16c, 0, 256, 1, None), 2),        # N = 0
    ((A16, A16b, A16c, 4, 100, 1, None), 2),        # K not a multiple of 256
    ((A16, A16b, A16c, 4, 256, 0, None), 2),        # batch 0
    ((A16, A16b, A16c, 4, 256, 65, None), 2),       # batch 65
    ((A16 + 4, A16b, A16c, 4, 256, 1, None), 3),    # W misaligned
    ((A16, A16b + 4, A16c, 4, 256, 1, None), 3),    # x misaligned
    ((A16, A16b, A16c + 2, 4, 256, 1, None), 3),    # y misaligned
    ((A16, A16b, A16b + 512, 4, 256, 1, None), 1),  # y overlaps x
])
def test_gemv_validation(args, status):
    _, L = _lib()
    assert L.qgemv_q4k(*args) == status


def test_q8_0_accepts_k_multiple_of_32_only_in_validation():
    _, L = _lib()
    assert L.qgemv_q8_0(A16, A16b, A16c, 4, 48, 1, None) == 2
    assert L.qgemv(7, A16, A16b, A16c, 4, 256, 1, None) == 1


def test_q8act_validation():
    _, L = _lib()
    f = L.qgemv_q8_0_q8act
    assert f(0, A16b, A16c, 4, 256, 1, None) == 1                    # null W
    assert f(A16, A16b, A16c, 4, 48, 1, None) == 2                   # K not a multiple of 32
    assert f(A16, A16b, A16c, 4, 256, 65, None) == 2                 # batch 65
    assert f(A16, A16b + 4, A16c, 4, 256, 1, None) == 3              # x not 16-byte aligned
    assert f(A16, A16b, A16c + 2, 4, 256, 1, None) == 3              # y misaligned
    assert f(A16, A16b, A16b + 512, 4, 256, 1, None) == 1            # y overlaps x
    big = 0x800000000  # past the 18 GB weight matrix of this shape
    # a quantized row beyond LDS that cannot be split (more than 65536 row tiles)
    assert f(A16, big, big + 0x100000000, 300000, 57344 + 32, 1, None) == 5


def test_quantize_and_preq_validation():
    _, L = _lib()
    f = L.qquantize_q8_act
    X, Q, D = A16, A16b, A16c
    assert f(0, Q, D, 256, 1, None) == 1                             # null x
    assert f(X, Q, 0, 256, 1, None) == 1                             # null d
    assert f(X, Q, D, 48, 1, None) == 2                              # K not a multiple of 32
    assert f(X, Q, D, 256, 65, None) == 2                            # batch 65
    assert f(X, Q + 4, D, 256, 1, None) == 3                         # q not 16-byte aligned
    assert f(X, Q, D + 2, 256, 1, None) == 3                         # d misaligned
    assert f(X, X + 512, D, 256, 1, None) == 1                       # q overlaps x
    assert f(X, Q, Q + 128, 256, 1, None) == 1                       # d overlaps q
    g = L.qgemv_q8_0_preq
    Y = 0x40000
    assert g(A16, Q, D, Y, 4, 256, 0, None) == 2                     # batch 0
    assert g(A16, Q + 8, D, Y, 4, 256, 1, None) == 3                 # q not 16-byte aligned
    assert g(A16, Q, D, Q + 64, 4, 256, 1, None) == 1                # y overlaps q
    assert g(A16, Q, D, D, 4, 256, 1, None) == 1                     # y overlaps d
    big = 0x800000000  # past the 18 GB weight matrix of this shape
    assert g(A16, big, big + 0x100000000, big + 0x200000000, 300000, 57344 + 32, 1, None) == 5  # cannot split


def test_ffn_validation():
    _, L = _lib()
    f = L.qffn_gate_up_act
    # null up
    assert f(0, A16, 0, A16b, None, 1e-6, 0, A16c, None, None, 4, 256, 1, None) == 1
    # bad activation
    assert f(0, A16, A16 + 0x8000, A16b, None, 1e-6, 5, A16c, None, None, 4, 256, 1, None) == 1
    # misaligned norm weight
    assert f(0, A16, A16 + 0x8000, A16b, A16b + 0x1004, 1e-6, 0, A16c, None, None, 4, 256, 1, None) == 3
    # h overlapping g_out
    assert f(0, A16, A16 + 0x8000, A16b, None, 1e-6, 0, A16c, A16c + 4, None, 4, 256, 1, None) == 1


QK, QV = A16 + 0x4000, A16 + 0x8000   # three weight matrices
YQ, YK, YV = A16c, A16c + 0x1000, A16c + 0x2000  # three outputs


def _qkv(L, fq=0, wq=A16, nq=4, fk=0, wk=QK, nk=4, fv=1, wv=QV, nv=4, x=A16b, nw=None,
         q=YQ, k=YK, v=YV, K=256, batch=1):
    return L.qqkv_proj(fq, wq, nq, fk, wk, nk, fv, wv, nv, x, nw, 1e-6, q, k, v, K, batch, None)


@pytest.mark.parametrize("kw,status", [
    (dict(wk=0), 1),                      # null K weights
    (dict(x=0), 1),                       # null x
    (dict(v=0), 1),                       # null v output
    (dict(fv=7), 1),                      # unknown format
    (dict(nk=0), 2),                      # K projection with no rows
    (dict(K=320), 2),                     # K not a multiple of 256 (k-quants)
    (dict(fq=2, fk=2, fv=2, K=48), 2),    # Q8_0 K not a multiple of 32
    (dict(batch=65), 2),                  # batch above 64
    (dict(wv=QV + 8), 3),                 # V weights misaligned
    (dict(x=A16b + 4), 3),                # x misaligned
    (dict(nw=A16b + 0x1004), 3),          # norm weight misaligned
    (dict(k=YK + 2), 3),                  # k output misaligned
    (dict(k=YQ + 8), 1),                  # k overlaps q
    (dict(v=A16b + 64), 1),               # v overlaps x
    (dict(q=QK + 16), 1),                 # q overlaps the K weights
    (dict(nw=A16b + 0x1000, v=A16b + 0x1010), 1),  # v overlaps the norm weight
])
def test_qkv_validation(kw, status):
    _, L = _lib()
    assert _qkv(L, **kw) == status


def test_residual_validation():
    _, L = _lib()
    g = L.qgemv_residual
    R = A16c + 0x4000
    assert g(0, A16, A16b, 0, A16c, 4, 256, 1, None) == 1            # null r
    assert g(0, A16, A16b, R + 2, A16c, 4, 256, 1, None) == 3        # r misaligned
    assert g(0, A16, A16b, A16c + 4, A16c, 4, 256, 1, None) == 1     # r overlaps y, not equal
    assert g(0, A16, A16b, R, A16c, 4, 100, 1, None) == 2            # K not a multiple of 256
    f = L.qffn_decode_residual
    H = A16c + 0x8000
    args = (0, A16, A16 + 0x8000, 1, A16 + 0x10000, A16b, None, 1e-6, 0)
    assert f(*args, 0, A16c, None, 256, 256, 1, None) == 1           # null r
    assert f(*args, A16c + 8, A16c, None, 256, 256, 1, None) == 1    # r overlaps y, not equal
    assert f(*args, H + 4, A16c, H, 256, 256, 1, None) == 1          # r overlaps h_out
    assert f(*args, R + 1, A16c, None, 256, 256, 1, None) == 3       # r misaligned


def test_moe_validation():
    _, L = _lib()
    f = L.qmoe_ffn_decode
    Wg, Wu, Wd = A16, A16 + 0x10000, A16 + 0x20000
    I, C, X, Y = 0x100000, 0x100100, 0x100200, 0x110000
    ok = dict(fg=0, wg=Wg, wu=Wu, fd=1, wd=Wd, ne=2, ids=I, coef=C, ns=2, x=X, nw=None, act=0,
              y=Y, h=None, nff=256, k=256)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["fg"], a["wg"], a["wu"], a["fd"], a["wd"], a["ne"], a["ids"], a["coef"], a["ns"],
                 a["x"], a["nw"], 1e-6, a["act"], a["y"], a["h"], a["nff"], a["k"], None)
    assert call(ids=0) == 1          # null ids
    assert call(coef=0) == 1         # null coef
    assert call(act=4) == 1          # bad activation
    assert call(ne=0) == 2           # no experts
    assert call(ns=0) == 2           # no slots
    assert call(ns=65) == 2          # too many slots
    assert call(nff=100) == 2        # N_ff not a multiple of 256
    assert call(ids=I + 2) == 3      # ids misaligned
    assert call(h=Y + 0x1008) == 3   # h_out misaligned
    assert call(y=Wd + 64) == 1      # y overlaps the down weights
    assert call(h=X) == 1            # h_out overlaps x
    assert call(y=I) == 1            # y overlaps ids
    far = dict(wg=1 << 40, wu=2 << 40, wd=3 << 40, x=4 << 40, y=5 << 40, ids=6 << 40, coef=7 << 40)
    assert call(nff=16384, k=16384, **far) == 5   # rows beyond one workgroup's LDS


def test_dequant_validation():
    _, L = _lib()
    assert L.qdequant(0, 0, A16b, 4, 256, None) == 1
    assert L.qdequant(0, A16 + 1, A16b, 4, 256, None) == 3
    assert L.qdequant_bf16(1, A16, A16b, 4, 300, None) == 2


@pytest.mark.parametrize("args,status", [
    ((0, 0, A16b, A16c, 8, 4, 256, None), 1),           # null W
    ((0, A16, 0, A16c, 8, 4, 256, None), 1),            # null X
    ((0, A16, A16b, 0, 8, 4, 256, None), 1),            # null Y
    ((0, A16, A16b, A16c, 0, 4, 256, None), 2),         # M = 0
    ((0, A16, A16b, A16c, 8, 0, 256, None), 2),         # N = 0
    ((0, A16, A16b, A16c, 8, 4, 320, None), 2),         # K not a multiple of 256
    ((2, A16, A16b, A16c, 8, 4, 48, None), 2),          # Q8_0 K not a multiple of 32
    ((0, A16, A16b, A16c, 1 << 24, 4, 256, None), 2),   # M * K >= 2^31
    ((0, A16 + 4, A16b, A16c, 8, 4, 256, None), 3),     # W misaligned
    ((0, A16, A16b + 8, A16c, 8, 4, 256, None), 3),     # X misaligned (needs 16)
    ((0, A16, A16b, A16c + 2, 8, 4, 256, None), 3),     # Y misaligned
    ((0, A16, A16b, A16b + 256, 8, 4, 256, None), 1),   # Y overlaps X
    ((0, A16, A16b, A16 + 64, 8, 4, 256, None), 1),     # Y overlaps W
    ((7, A16, A16b, A16c, 8, 4, 256, None), 1),         # unknown format
])
def test_prefill_validation(args, status):
    _, L = _lib()
    assert L.qgemm_prefill(*args) == status


def test_prefill_gate_up_validation():
    _, L = _lib()
    f = L.qgemm_prefill_gate_up_act
    U = A16 + 0x8000
    # null up, null H
    assert f(0, A16, 0, A16b, 0, A16c, None, None, 8, 4, 256, None) == 1
    assert f(0, A16, U, A16b, 0, 0, None, None, 8, 4, 256, None) == 1
    # unknown activation
    assert f(0, A16, U, A16b, 3, A16c, None, None, 8, 4, 256, None) == 1
    # H misaligned (2 bytes), g_out misaligned (4 bytes)
    assert f(0, A16, U, A16b, 0, A16c + 1, None, None, 8, 4, 256, None) == 3
    assert f(0, A16, U, A16b, 0, A16c, A16c + 0x1002, None, 8, 4, 256, None) == 3
    # H overlapping g_out, u_out overlapping X
    assert f(0, A16, U, A16b, 0, A16c, A16c + 16, None, 8, 4, 256, None) == 1
    assert f(0, A16, U, A16b, 0, A16c, None, A16b + 64, 8, 4, 256, None) == 1


def test_gemm_override_validation():
    _, L = _lib()
    assert L.qd_set_gemm_override(3, 0) == 1
    assert L.qd_set_gemm_override(0, -1) == 1
    assert L.qd_set_gemm_override(0, 0) == 0
    assert L.qd_set_gemm_streamk(-1) == 1
    assert L.qd_set_gemm_streamk(7) == 0
    assert L.qd_set_gemm_streamk(0) == 0


def test_stream_override_validation():
    _, L = _lib()
    assert L.qd_set_stream_override(9, 0, 0, 0) == 1      # workgroups per CU 1..8
    assert L.qd_set_stream_override(1, 0, 3, 0) == 1      # decoding waves 4 or 8
    assert L.qd_set_stream_override(1, 0, 1, 0) == 1
    assert L.qd_set_stream_override(1, 33, 4, 0) == 1     # depth <= 32 per copying wave
    assert L.qd_set_stream_override(1, 0, 4, 3) == 1      # one, two or four copying waves
    assert L.qd_set_stream_override(1, 0, 8, 8) == 1
    assert L.qd_set_stream_override(1, 0, 8, 4) == 0
    assert L.qd_set_stream_override(1, 1, 8, 1) == 0
    assert L.qd_set_stream_override(1, 16, 8, 2) == 0
    assert L.qd_set_stream_override(2, 3, 0, 0) == 0
    assert L.qd_set_stream_override(0, 0, 0, 0) == 0


def _q8plan(L, N, K, batch):
    import ctypes
    out = (ctypes.c_int32 * 4)()
    st = L.qd_plan_q8act(N, K, batch, out)
    return st, tuple(out)


def test_q8act_plan_terminates_and_fits_lds():
    """The int8-activation GEMV's launch plan, on the host only: large legal K
    (up to the 2^24 the shape check accepts, and around the K at which one
    column's codes stop fitting a workgroup's LDS) gives a plan whose staged
    K-slice fits 63 KB of LDS, whose slices cover K, and every slice is
    non-empty.  An earlier plan loop never ended for some of these K."""
    _, L = _lib()
    budget = 65536 - 1024
    cases = [(4, 1 << 24, 1), (4, 12959776, 1), (4, 12000000, 1), (64, 57344, 1), (64, 57344 + 32, 1),
             (64, 57344 + 256, 1), (64, 65536, 1), (300, 57344 + 32, 8), (262144, 2560, 1),
             (2560, 10240, 8), (5376, 21504, 3), (1, 32, 1)]
    for N, K, batch in cases:
        st, (p, ks, su_per, chunk) = _q8plan(L, N, K, batch)
        assert st == 0, (N, K, batch)
        nsu = (K // 32 + 7) // 8
        assert ks >= 1 and su_per >= 1 and p in (1, 2, 4, 8, 16), (N, K, batch)
        assert (ks - 1) * su_per < nsu <= ks * su_per, (N, K, batch, ks, su_per)
        kslice = min(K, su_per * 256)
        assert chunk >= 1, (N, K, batch)
        lds = (chunk * kslice + 15) // 16 * 16 + chunk * (kslice // 32) * 4
        assert lds <= budget, (N, K, batch, lds)
    # more row tiles than the split-K counters cover: unsupported, not a hang
    st, (_, _, _, chunk) = _q8plan(L, 300000 * 64, 57344 + 32, 1)
    assert st == 0 and chunk == 0
    assert _q8plan(L, 4, 48, 1)[0] == 2
    assert L.qd_plan_q8act(4, 256, 1, None) == 1


def test_launch_override_validation():
    _, L = _lib()
    assert L.qd_set_launch_override(3, 0, 0) == 1
    assert L.qd_set_launch_override(0, 0, 5) == 1
    assert L.qd_set_launch_override(0, 0, 0) == 0


def test_walk_override_validation():
    _, L = _lib()
    assert L.qd_set_walk_override(-1) == 1
    assert L.qd_set_walk_override(65) == 1
    assert L.qd_set_walk_override(8) == 0
    assert L.qd_set_walk_override(0) == 0


def test_python_binding_refuses_cpu_tensors():
    import torch
    qd, _ = _lib()
    W = torch.zeros(144, dtype=torch.uint8)
    x = torch.zeros(256, dtype=torch.float32)
    with pytest.raises(ValueError, match="GPU tensor"):
        qd.qgemv_q4k(W, x)
