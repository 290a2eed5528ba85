"""CPU oracle for block-quantized decode GEMV -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library never imports, links or
calls it, and this package never touches the GPU library: the two share no
code.  The arithmetic lives in ``oracle.c`` (plain C, fp64 accumulation);
this module only builds it with gcc and marshals numpy arrays through ctypes.

Each function names the definition it follows in ``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

Q4_K, Q6_K, Q8_0 = 0, 1, 2
ACT_GELU_TANH, ACT_SILU = 0, 1
FORMATS = {"q4_k": Q4_K, "q6_k": Q6_K, "q8_0": Q8_0}


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (no GPU, no HIP)."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    src = os.path.join(_HERE, "oracle.c")
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared",
           "-fno-fast-math", "-ffp-contract=off", src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        I = ctypes.c_int
        D = ctypes.c_double
        sigs = {
            "orc_block_elems": (I, [I]),
            "orc_block_bytes": (I, [I]),
            "orc_row_bytes": (I64, [I, I64]),
            "orc_f16_to_f32": (ctypes.c_float, [ctypes.c_uint16]),
            "orc_f32_to_bf16": (ctypes.c_uint16, [ctypes.c_float]),
            "orc_bf16_to_f32": (ctypes.c_float, [ctypes.c_uint16]),
            "orc_dequant_q4k_block": (None, [P, P]),
            "orc_dequant_q6k_block": (None, [P, P]),
            "orc_dequant_q8_0_block": (None, [P, P]),
            "orc_q4k_scale_min": (None, [P, I, P, P]),
            "orc_dequant_rows": (I, [I, P, I64, I64, I64, P]),
            "orc_gemv": (I, [I, P, P, I64, I64, I, I64, I64, P, P]),
            "orc_rmsnorm": (None, [P, P, I64, I, D, P]),
            "orc_post_norm_residual": (None, [P, P, P, P, I64, I, D, P, P]),
            "orc_gelu_tanh": (D, [D]),
            "orc_silu": (D, [D]),
            "orc_act": (D, [I, D]),
            "orc_gemm_bf16": (I, [I, P, P, I64, I64, I64, I64, I64, I64, I64, P, P]),
            "orc_quantize_q8_act": (I, [P, I64, I, P, P]),
            "orc_gemv_q8_0_q8act": (I, [P, P, P, I64, I64, I, I64, I64, P, P]),
        }
        for name, (res, args) in sigs.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
        return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _fmt(fmt) -> int:
    return FORMATS[fmt] if isinstance(fmt, str) else int(fmt)


def block_elems(fmt) -> int:
    return _load().orc_block_elems(_fmt(fmt))


def block_bytes(fmt) -> int:
    return _load().orc_block_bytes(_fmt(fmt))


def row_bytes(fmt, K: int) -> int:
    return _load().orc_row_bytes(_fmt(fmt), K)


def f16_to_f32(h: int) -> float:
    return _load().orc_f16_to_f32(h)


def f32_to_bf16(f: float) -> int:
    return _load().orc_f32_to_bf16(f)


def bf16_to_f32(b: int) -> float:
    return _load().orc_bf16_to_f32(b)


def q4k_scale_min(block: np.ndarray, j: int):
    block = np.ascontiguousarray(block, dtype=np.uint8)
    sc = ctypes.c_int()
    m = ctypes.c_int()
    _load().orc_q4k_scale_min(_ptr(block), j, ctypes.byref(sc), ctypes.byref(m))
    return sc.value, m.value


def dequant_block(fmt, block: np.ndarray) -> np.ndarray:
    fmt = _fmt(fmt)
    block = np.ascontiguousarray(block, dtype=np.uint8)
    assert block.size == block_bytes(fmt)
    out = np.empty(block_elems(fmt), dtype=np.float32)
    fn = {Q4_K: "orc_dequant_q4k_block", Q6_K: "orc_dequant_q6k_block",
          Q8_0: "orc_dequant_q8_0_block"}[fmt]
    getattr(_load(), fn)(_ptr(block), _ptr(out))
    return out


def dequant(fmt, W: np.ndarray, K: int, n0: int = 0, n1: int | None = None) -> np.ndarray:
    """fp32 weights of rows [n0, n1) of a row-major quantized matrix."""
    fmt = _fmt(fmt)
    W = np.ascontiguousarray(W, dtype=np.uint8)
    rb = row_bytes(fmt, K)
    if rb <= 0:
        raise ValueError("bad K for format")
    N = W.size // rb
    n1 = N if n1 is None else n1
    out = np.empty((n1 - n0, K), dtype=np.float32)
    if _load().orc_dequant_rows(fmt, _ptr(W), K, n0, n1, _ptr(out)) != 0:
        raise ValueError("orc_dequant_rows failed")
    return out


def gemv(fmt, W: np.ndarray, x: np.ndarray, N: int, K: int,
         n0: int = 0, n1: int | None = None):
    """(y64, S): fp64 y = W x and S = sum |w x| for rows [n0, n1).

    x is [batch, K] (or [K]); outputs are [batch, N] with only rows
    [n0, n1) filled (the rest NaN)."""
    fmt = _fmt(fmt)
    W = np.ascontiguousarray(W, dtype=np.uint8)
    x2 = np.ascontiguousarray(np.atleast_2d(x), dtype=np.float32)
    batch = x2.shape[0]
    assert x2.shape[1] == K
    n1 = N if n1 is None else n1
    y = np.full((batch, N), np.nan, dtype=np.float64)
    S = np.full((batch, N), np.nan, dtype=np.float64)
    rc = _load().orc_gemv(fmt, _ptr(W), _ptr(x2), N, K, batch, n0, n1, _ptr(y), _ptr(S))
    if rc != 0:
        raise ValueError("orc_gemv failed")
    return y, S


def quantize_q8_act(x: np.ndarray):
    """(q, d): x [batch, K] (or [K]) quantized per run of 32 to int8 q and
    fp32 d = max|x| / 127, q = round(x / d) halves away from zero."""
    x2 = np.ascontiguousarray(np.atleast_2d(x), dtype=np.float32)
    batch, K = x2.shape
    q = np.empty((batch, K), dtype=np.int8)
    d = np.empty((batch, K // 32), dtype=np.float32)
    if _load().orc_quantize_q8_act(_ptr(x2), K, batch, _ptr(q), _ptr(d)) != 0:
        raise ValueError("orc_quantize_q8_act failed")
    return q, d


def gemv_q8_0_q8act(W: np.ndarray, q: np.ndarray, d: np.ndarray, N: int, K: int,
                    n0: int = 0, n1: int | None = None):
    """(y64, S) of Q8_0 weights against quantized activations (q, d) for rows
    [n0, n1): y = sum_j dw dx sum qw qx, S over |products|, fp64."""
    W = np.ascontiguousarray(W, dtype=np.uint8)
    q = np.ascontiguousarray(np.atleast_2d(q), dtype=np.int8)
    d = np.ascontiguousarray(np.atleast_2d(d), dtype=np.float32)
    batch = q.shape[0]
    n1 = N if n1 is None else n1
    y = np.full((batch, N), np.nan, dtype=np.float64)
    S = np.full((batch, N), np.nan, dtype=np.float64)
    if _load().orc_gemv_q8_0_q8act(_ptr(W), _ptr(q), _ptr(d), N, K, batch, n0, n1, _ptr(y), _ptr(S)) != 0:
        raise ValueError("orc_gemv_q8_0_q8act failed")
    return y, S


def gemv_rows(fmt, W: np.ndarray, x: np.ndarray, N: int, K: int, rows):
    """Same as gemv, computed only for the listed rows (others NaN)."""
    fmt = _fmt(fmt)
    W = np.ascontiguousarray(W, dtype=np.uint8)
    x2 = np.ascontiguousarray(np.atleast_2d(x), dtype=np.float32)
    batch = x2.shape[0]
    assert x2.shape[1] == K
    y = np.full((batch, N), np.nan, dtype=np.float64)
    S = np.full((batch, N), np.nan, dtype=np.float64)
    lib = _load()
    pW, px, py, pS = _ptr(W), _ptr(x2), _ptr(y), _ptr(S)
    for r in np.asarray(rows, dtype=np.int64):
        if lib.orc_gemv(fmt, pW, px, N, K, batch, int(r), int(r) + 1, py, pS) != 0:
            raise ValueError("orc_gemv failed")
    return y, S


def gemv_threaded(fmt, W, x, N, K, threads: int):
    """Same as gemv over all rows, rows split over `threads` host threads
    (ctypes releases the GIL during the C call)."""
    fmt = _fmt(fmt)
    W = np.ascontiguousarray(W, dtype=np.uint8)
    x2 = np.ascontiguousarray(np.atleast_2d(x), dtype=np.float32)
    batch = x2.shape[0]
    y = np.empty((batch, N), dtype=np.float64)
    S = np.empty((batch, N), dtype=np.float64)
    lib = _load()
    bounds = np.linspace(0, N, threads + 1).astype(np.int64)
    rcs = [0] * threads

    def work(t):
        rcs[t] = lib.orc_gemv(fmt, _ptr(W), _ptr(x2), N, K, batch,
                              int(bounds[t]), int(bounds[t + 1]), _ptr(y), _ptr(S))

    ts = [threading.Thread(target=work, args=(t,)) for t in range(threads)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    if any(rcs):
        raise ValueError("orc_gemv failed")
    return y, S


def rmsnorm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """fp64 RMS-norm of each row of x ([batch, K] or [K])."""
    x2 = np.ascontiguousarray(np.atleast_2d(x), dtype=np.float32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    batch, K = x2.shape
    out = np.empty((batch, K), dtype=np.float64)
    _load().orc_rmsnorm(_ptr(x2), _ptr(w), K, batch, eps, _ptr(out))
    return out


def post_norm_residual(p: np.ndarray, r: np.ndarray, w1: np.ndarray, eps: float, w2=None):
    """(y, y2) of orc_post_norm_residual: y = r + RMSNorm(p; w1), y2 =
    RMSNorm(y; w2) (None without w2); p fp64 [batch, N] or [N]."""
    p2 = np.ascontiguousarray(np.atleast_2d(p), dtype=np.float64)
    r2 = np.ascontiguousarray(np.atleast_2d(r), dtype=np.float32)
    batch, N = p2.shape
    assert r2.shape == (batch, N)
    w1 = np.ascontiguousarray(w1, dtype=np.float32)
    y = np.empty((batch, N), dtype=np.float64)
    y2 = np.empty((batch, N), dtype=np.float64) if w2 is not None else None
    w2c = np.ascontiguousarray(w2, dtype=np.float32) if w2 is not None else None
    _load().orc_post_norm_residual(_ptr(p2), _ptr(r2), _ptr(w1), _ptr(w2c) if w2c is not None else None,
                                   N, batch, eps, _ptr(y), _ptr(y2) if y2 is not None else None)
    return y, y2


def act(kind: int, g: float) -> float:
    return _load().orc_act(kind, g)


def act_vec(kind: int, g: np.ndarray) -> np.ndarray:
    lib = _load()
    flat = np.asarray(g, dtype=np.float64).ravel()
    return np.array([lib.orc_act(kind, float(v)) for v in flat]).reshape(np.shape(g))


def gemm_bf16(fmt, W: np.ndarray, X: np.ndarray, N: int, K: int,
              m0: int = 0, m1: int | None = None, n0: int = 0, n1: int | None = None):
    """(Y64, S) of Y = X bf16(W)^T over the block [m0,m1) x [n0,n1).

    X is uint16 bf16 bits [M, K].  Outputs are [M, N], NaN outside the block."""
    fmt = _fmt(fmt)
    W = np.ascontiguousarray(W, dtype=np.uint8)
    X = np.ascontiguousarray(X, dtype=np.uint16)
    M = X.shape[0]
    assert X.shape[1] == K
    m1 = M if m1 is None else m1
    n1 = N if n1 is None else n1
    Y = np.full((M, N), np.nan, dtype=np.float64)
    S = np.full((M, N), np.nan, dtype=np.float64)
    rc = _load().orc_gemm_bf16(fmt, _ptr(W), _ptr(X), M, N, K, m0, m1, n0, n1, _ptr(Y), _ptr(S))
    if rc != 0:
        raise ValueError("orc_gemm_bf16 failed")
    return Y, S


def gemm_bf16_threaded(fmt, W: np.ndarray, X: np.ndarray, N: int, K: int, threads: int):
    """Same as gemm_bf16 over the whole output, weight rows split over
    `threads` host threads (ctypes releases the GIL during the C call)."""
    fmt = _fmt(fmt)
    W = np.ascontiguousarray(W, dtype=np.uint8)
    X = np.ascontiguousarray(X, dtype=np.uint16)
    M = X.shape[0]
    assert X.shape[1] == K
    Y = np.empty((M, N), dtype=np.float64)
    S = np.empty((M, N), dtype=np.float64)
    lib = _load()
    bounds = np.linspace(0, N, threads + 1).astype(np.int64)
    rcs = [0] * threads

    def work(t):
        rcs[t] = lib.orc_gemm_bf16(fmt, _ptr(W), _ptr(X), M, N, K, 0, M, int(bounds[t]), int(bounds[t + 1]),
                                   _ptr(Y), _ptr(S))

    ts = [threading.Thread(target=work, args=(t,)) for t in range(threads)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    if any(rcs):
        raise ValueError("orc_gemm_bf16 failed")
    return Y, S


def host_threads(cap: int = 16) -> int:
    """Threads for the threaded oracle calls: the cores this process may run
    on, at most `cap`."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(cap, n))


def gemm_bf16_cols(fmt, W: np.ndarray, X: np.ndarray, N: int, K: int, cols):
    """(Y64, S) of Y = X bf16(W)^T for the listed weight rows only: [M, len(cols)]."""
    fmt_id = _fmt(fmt)
    rb = row_bytes(fmt_id, K)
    W = np.ascontiguousarray(W, dtype=np.uint8).reshape(N, rb)
    X = np.ascontiguousarray(X, dtype=np.uint16)
    M = X.shape[0]
    cols = [int(c) for c in cols]
    Y = np.empty((M, len(cols)), dtype=np.float64)
    S = np.empty((M, len(cols)), dtype=np.float64)
    for j, n in enumerate(cols):
        y1, s1 = gemm_bf16(fmt_id, W[n:n + 1], X, 1, K)
        Y[:, j] = y1[:, 0]
        S[:, j] = s1[:, 0]
    return Y, S
