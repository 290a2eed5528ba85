"""Block-quantized decode GEMV for AMD MI355X (gfx950) -- Python binding.

This module only marshals arguments: it checks torch tensors, then passes
their device pointers and the current HIP stream to the C ABI of
``libqdecode.so`` (declared in ``include/qdecode.h``).  Every step of the
computation runs in the library's HIP kernels.  There is no fallback: if the
library is not built, or a tensor is not on the GPU, the call raises.

Entry points (same names as the C ABI):
    qgemv_q4k, qgemv_q6k, qgemv_q8_0, qgemv        y = W x, batch 1..8
    qgemv_residual                                 y = W x + r (r may be y)
    qgemv_post_norm_residual                       y = r + RMSNorm(W x), y2 = RMSNorm(y)
    qffn_decode_post_norm_residual                 the same epilogue on the FFN's down projection
    qgemv_q8_0_q8act                               Q8_0 GEMV on int8-quantized x (opt-in)
    qquantize_q8_act, qgemv_q8_0_preq              its two halves: quantize once, GEMV on the codes
    qqkv_proj                                      q, k, v = Wq xn, Wk xn, Wv xn (one launch)
    qffn_gate_up_act                               h = act(Wg xn) * (Wu xn)
    qffn_decode                                    y = Wd h (whole FFN: gate/up launch, then down)
    qffn_decode_noalloc                            qffn_decode with no allocation (fixed scratch)
    qffn_decode_residual                           y = Wd h + r
    qmoe_ffn_decode                                mixture-of-experts FFN (routed ids on device)
    qgemm_prefill, qgemm_prefill_gate_up_act       bf16 MFMA prefill GEMMs
    qdequant, qdequant_bf16                        decoded weights (tests)
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqdecode.so")

Q4_K, Q6_K, Q8_0 = 0, 1, 2
FORMATS = {"q4_k": Q4_K, "q6_k": Q6_K, "q8_0": Q8_0}
ACT_GELU_TANH, ACT_SILU = 0, 1
ACTS = {"gelu_tanh": ACT_GELU_TANH, "silu": ACT_SILU}
MAX_BATCH = 64
BATCH_CHUNK = 8

QD_OK, QD_EINVAL, QD_ESHAPE, QD_EALIGN, QD_ELAUNCH, QD_EUNSUPPORTED, QD_ENOMEM, QD_ECAPTURE, QD_ETOOBIG = range(9)

# Every function the header declares, with its ctypes signature.
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I = ctypes.c_int
_F = ctypes.c_float
SIGNATURES = {
    "qd_block_elems": (_I, [_I]),
    "qd_block_bytes": (_I, [_I]),
    "qd_row_bytes": (_I64, [_I, _I64]),
    "qd_status_str": (ctypes.c_char_p, [_I]),
    "qd_version": (_I, []),
    "qgemv_q4k": (_I, [_P, _P, _P, _I64, _I64, _I, _P]),
    "qgemv_q6k": (_I, [_P, _P, _P, _I64, _I64, _I, _P]),
    "qgemv_q8_0": (_I, [_P, _P, _P, _I64, _I64, _I, _P]),
    "qgemv": (_I, [_I, _P, _P, _P, _I64, _I64, _I, _P]),
    "qgemv_residual": (_I, [_I, _P, _P, _P, _P, _I64, _I64, _I, _P]),
    "qgemv_post_norm_residual": (_I, [_I, _P, _P, _P, _F, _P, _P, _P, _P, _I64, _I64, _I, _P]),
    "qffn_decode_post_norm_residual": (_I, [_I, _P, _P, _I, _P, _P, _P, _F, _I, _P, _P, _P, _P, _P, _P, _I64,
                                            _I64, _I, _P]),
    "qgemv_q8_0_q8act": (_I, [_P, _P, _P, _I64, _I64, _I, _P]),
    "qquantize_q8_act": (_I, [_P, _P, _P, _I64, _I, _P]),
    "qgemv_q8_0_preq": (_I, [_P, _P, _P, _P, _I64, _I64, _I, _P]),
    "qmoe_ffn_decode": (_I, [_I, _P, _P, _I, _P, _I, _P, _P, _I, _P, _P, _F, _I, _P, _P, _I64, _I64,
                             _P]),
    "qffn_decode_residual": (_I, [_I, _P, _P, _I, _P, _P, _P, _F, _I, _P, _P, _P, _I64, _I64, _I,
                                  _P]),
    "qqkv_proj": (_I, [_I, _P, _I64, _I, _P, _I64, _I, _P, _I64, _P, _P, _F, _P, _P, _P, _I64, _I,
                       _P]),
    "qffn_gate_up_act": (_I, [_I, _P, _P, _P, _P, _F, _I, _P, _P, _P, _I64, _I64, _I, _P]),
    "qffn_decode": (_I, [_I, _P, _P, _I, _P, _P, _P, _F, _I, _P, _P, _I64, _I64, _I, _P]),
    "qffn_decode_noalloc": (_I, [_I, _P, _P, _I, _P, _P, _P, _F, _I, _P, _P, _I64, _I64, _I, _P]),
    "qgemm_prefill": (_I, [_I, _P, _P, _P, _I64, _I64, _I64, _P]),
    "qgemm_prefill_gate_up_act": (_I, [_I, _P, _P, _P, _I, _P, _P, _P, _I64, _I64, _I64, _P]),
    "qdequant": (_I, [_I, _P, _P, _I64, _I64, _P]),
    "qdequant_bf16": (_I, [_I, _P, _P, _I64, _I64, _P]),
    "qd_set_launch_override": (_I, [_I, _I, _I]),
    "qd_set_walk_override": (_I, [_I]),
    "qd_set_gemm_override": (_I, [_I, _I]),
    "qd_set_gemm_streamk": (_I, [_I]),
    "qd_set_stream_override": (_I, [_I, _I, _I, _I]),
    "qd_set_batch_override": (_I, [_I, _I]),
    "qd_plan_q8act": (_I, [_I64, _I64, _I, _P]),
}

_lock = threading.Lock()
_lib = None


class QDError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = lib().qd_status_str(status).decode()
        super().__init__(f"{fn} failed: status {status} ({msg})")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded libqdecode.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is not built; run __graft_entry__.build() "
                    "(hipcc --offload-arch=gfx950) first")
            L = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(L, name)
                fn.restype = res
                fn.argtypes = args
            _lib = L
        return _lib


def _fmt(fmt) -> int:
    v = FORMATS[fmt.lower()] if isinstance(fmt, str) else int(fmt)
    if v not in (Q4_K, Q6_K, Q8_0):
        raise ValueError(f"unknown format {fmt!r}")
    return v


def _act(act) -> int:
    return ACTS[act] if isinstance(act, str) else int(act)


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _dev(t: torch.Tensor, name: str, dtype: torch.dtype):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (no CPU path exists)")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _check(fn: str, status: int):
    if status != QD_OK:
        raise QDError(fn, status)


def block_elems(fmt) -> int:
    return lib().qd_block_elems(_fmt(fmt))


def block_bytes(fmt) -> int:
    return lib().qd_block_bytes(_fmt(fmt))


def row_bytes(fmt, K: int) -> int:
    return lib().qd_row_bytes(_fmt(fmt), K)


def _rows(fmt: int, W: torch.Tensor, K: int) -> int:
    rb = lib().qd_row_bytes(fmt, K)
    if rb <= 0:
        raise ValueError(f"K={K} is not a multiple of the block size")
    if W.numel() % rb:
        raise ValueError("weight bytes are not a whole number of rows")
    return W.numel() // rb


def qgemv(fmt, W: torch.Tensor, x: torch.Tensor, y: torch.Tensor | None = None) -> torch.Tensor:
    """y = W x.  W: uint8 (N rows of blocks); x: fp32 [K] or [batch, K]."""
    f = _fmt(fmt)
    K = x.shape[-1]
    batch = 1 if x.dim() == 1 else x.shape[0]
    N = _rows(f, W, K)
    if y is None:
        y = torch.empty((N,) if x.dim() == 1 else (batch, N), dtype=torch.float32, device=x.device)
    st = lib().qgemv(f, _dev(W, "W", torch.uint8), _dev(x, "x", torch.float32),
                     _dev(y, "y", torch.float32), N, K, batch, _stream())
    _check("qgemv", st)
    return y


def qgemv_residual(fmt, W: torch.Tensor, x: torch.Tensor, r: torch.Tensor,
                   y: torch.Tensor | None = None) -> torch.Tensor:
    """y = W x + r (pass y=r to add in place)."""
    f = _fmt(fmt)
    K = x.shape[-1]
    batch = 1 if x.dim() == 1 else x.shape[0]
    N = _rows(f, W, K)
    if tuple(r.shape) != ((N,) if x.dim() == 1 else (batch, N)):
        raise ValueError("r must have the output's shape")
    if y is None:
        y = torch.empty_like(r)
    st = lib().qgemv_residual(f, _dev(W, "W", torch.uint8), _dev(x, "x", torch.float32),
                              _dev(r, "r", torch.float32), _dev(y, "y", torch.float32), N, K, batch,
                              _stream())
    _check("qgemv_residual", st)
    return y


def qgemv_post_norm_residual(fmt, W: torch.Tensor, x: torch.Tensor, post_w: torch.Tensor, r: torch.Tensor,
                             eps: float = 1e-6, y: torch.Tensor | None = None,
                             next_w: torch.Tensor | None = None, y2: torch.Tensor | None = None):
    """y = r + RMSNorm(W x; post_w) and, with next_w, y2 = RMSNorm(y; next_w).
    Pass y=r to update the residual in place.  Returns y, or (y, y2)."""
    f = _fmt(fmt)
    K = x.shape[-1]
    batch = 1 if x.dim() == 1 else x.shape[0]
    N = _rows(f, W, K)
    if tuple(r.shape) != ((N,) if x.dim() == 1 else (batch, N)):
        raise ValueError("r must have the output's shape")
    if y is None:
        y = torch.empty_like(r)
    if next_w is not None and y2 is None:
        y2 = torch.empty_like(r)
    st = lib().qgemv_post_norm_residual(
        f, _dev(W, "W", torch.uint8), _dev(x, "x", torch.float32), _dev(post_w, "post_w", torch.float32),
        float(eps), _dev(r, "r", torch.float32), _dev(y, "y", torch.float32),
        _dev(next_w, "next_w", torch.float32) if next_w is not None else None,
        _dev(y2, "y2", torch.float32) if next_w is not None else None, N, K, batch, _stream())
    _check("qgemv_post_norm_residual", st)
    return (y, y2) if next_w is not None else y


def qffn_decode_post_norm_residual(fmt_gu, Wg: torch.Tensor, Wu: torch.Tensor, fmt_down, Wd: torch.Tensor,
                                   x: torch.Tensor, post_w: torch.Tensor, r: torch.Tensor,
                                   norm_w: torch.Tensor | None = None, eps: float = 1e-6, act="gelu_tanh",
                                   y: torch.Tensor | None = None, next_w: torch.Tensor | None = None,
                                   y2: torch.Tensor | None = None, h_out: torch.Tensor | None = None):
    """y = r + RMSNorm(Wd h; post_w), h = act(Wg xn) * (Wu xn); with next_w
    also y2 = RMSNorm(y; next_w).  Returns y, or (y, y2)."""
    fg, fd = _fmt(fmt_gu), _fmt(fmt_down)
    K = x.shape[-1]
    batch = 1 if x.dim() == 1 else x.shape[0]
    N = _rows(fg, Wg, K)
    if _rows(fg, Wu, K) != N or _rows(fd, Wd, N) != K:
        raise ValueError("gate/up must be N_ff x K and down K x N_ff")
    if tuple(r.shape) != tuple(x.shape):
        raise ValueError("r must have x's shape")
    if y is None:
        y = torch.empty_like(x)
    if next_w is not None and y2 is None:
        y2 = torch.empty_like(x)
    nw = _dev(norm_w, "norm_w", torch.float32) if norm_w is not None else None
    hp = _dev(h_out, "h_out", torch.float32) if h_out is not None else None
    st = lib().qffn_decode_post_norm_residual(
        fg, _dev(Wg, "Wg", torch.uint8), _dev(Wu, "Wu", torch.uint8), fd, _dev(Wd, "Wd", torch.uint8),
        _dev(x, "x", torch.float32), nw, float(eps), _act(act), _dev(post_w, "post_w", torch.float32),
        _dev(r, "r", torch.float32), _dev(y, "y", torch.float32),
        _dev(next_w, "next_w", torch.float32) if next_w is not None else None,
        _dev(y2, "y2", torch.float32) if next_w is not None else None, hp, N, K, batch, _stream())
    _check("qffn_decode_post_norm_residual", st)
    return (y, y2) if next_w is not None else y


def qgemv_q8_0_q8act(W: torch.Tensor, x: torch.Tensor, y: torch.Tensor | None = None) -> torch.Tensor:
    """y = W q(x): Q8_0 weights against x quantized per 32 to int8 (opt-in;
    differs from qgemv_q8_0 by the activation rounding)."""
    K = x.shape[-1]
    batch = 1 if x.dim() == 1 else x.shape[0]
    N = _rows(Q8_0, W, K)
    if y is None:
        y = torch.empty((N,) if x.dim() == 1 else (batch, N), dtype=torch.float32, device=x.device)
    st = lib().qgemv_q8_0_q8act(_dev(W, "W", torch.uint8), _dev(x, "x", torch.float32),
                                _dev(y, "y", torch.float32), N, K, batch, _stream())
    _check("qgemv_q8_0_q8act", st)
    return y


def qquantize_q8_act(x: torch.Tensor, q: torch.Tensor | None = None, d: torch.Tensor | None = None):
    """(q int8 [.., K], d fp32 [.., K/32]): x quantized per run of 32."""
    K = x.shape[-1]
    batch = 1 if x.dim() == 1 else x.shape[0]
    lead = () if x.dim() == 1 else (batch,)
    if q is None:
        q = torch.empty(lead + (K,), dtype=torch.int8, device=x.device)
    if d is None:
        d = torch.empty(lead + (K // 32,), dtype=torch.float32, device=x.device)
    st = lib().qquantize_q8_act(_dev(x, "x", torch.float32), _dev(q, "q", torch.int8), _dev(d, "d", torch.float32),
                                K, batch, _stream())
    _check("qquantize_q8_act", st)
    return q, d


def qgemv_q8_0_preq(W: torch.Tensor, q: torch.Tensor, d: torch.Tensor, y: torch.Tensor | None = None) -> torch.Tensor:
    """y = W (d, q): Q8_0 weights against activations from qquantize_q8_act."""
    K = q.shape[-1]
    batch = 1 if q.dim() == 1 else q.shape[0]
    N = _rows(Q8_0, W, K)
    if y is None:
        y = torch.empty((N,) if q.dim() == 1 else (batch, N), dtype=torch.float32, device=q.device)
    st = lib().qgemv_q8_0_preq(_dev(W, "W", torch.uint8), _dev(q, "q", torch.int8), _dev(d, "d", torch.float32),
                               _dev(y, "y", torch.float32), N, K, batch, _stream())
    _check("qgemv_q8_0_preq", st)
    return y


def qgemv_q4k(W, x, y=None):
    return qgemv(Q4_K, W, x, y)


def qgemv_q6k(W, x, y=None):
    return qgemv(Q6_K, W, x, y)


def qgemv_q8_0(W, x, y=None):
    return qgemv(Q8_0, W, x, y)


def qqkv_proj(fmts, Wq: torch.Tensor, Wk: torch.Tensor, Wv: torch.Tensor, x: torch.Tensor,
              norm_w: torch.Tensor | None = None, eps: float = 1e-6,
              q: torch.Tensor | None = None, k: torch.Tensor | None = None,
              v: torch.Tensor | None = None):
    """(q, k, v) = (Wq xn, Wk xn, Wv xn), xn = RMSNorm(x) (if norm_w) or x, in
    one launch.  fmts: the three weight formats, e.g. ("q4_k", "q4_k", "q6_k")."""
    f = [_fmt(t) for t in fmts]
    if len(f) != 3:
        raise ValueError("fmts must name three formats (q, k, v)")
    K = x.shape[-1]
    batch = 1 if x.dim() == 1 else x.shape[0]
    Ns = [_rows(fi, W, K) for fi, W in zip(f, (Wq, Wk, Wv))]
    outs = []
    for o, n in zip((q, k, v), Ns):
        shape = (n,) if x.dim() == 1 else (batch, n)
        outs.append(torch.empty(shape, dtype=torch.float32, device=x.device) if o is None else o)
    nw = _dev(norm_w, "norm_w", torch.float32) if norm_w is not None else None
    st = lib().qqkv_proj(f[0], _dev(Wq, "Wq", torch.uint8), Ns[0], f[1], _dev(Wk, "Wk", torch.uint8),
                         Ns[1], f[2], _dev(Wv, "Wv", torch.uint8), Ns[2], _dev(x, "x", torch.float32),
                         nw, float(eps), _dev(outs[0], "q", torch.float32),
                         _dev(outs[1], "k", torch.float32), _dev(outs[2], "v", torch.float32), K,
                         batch, _stream())
    _check("qqkv_proj", st)
    return tuple(outs)


def qffn_gate_up_act(fmt, Wg: torch.Tensor, Wu: torch.Tensor, x: torch.Tensor,
                     norm_w: torch.Tensor | None = None, eps: float = 1e-6, act="gelu_tanh",
                     h: torch.Tensor | None = None, g_out: torch.Tensor | None = None,
                     u_out: torch.Tensor | None = None) -> torch.Tensor:
    """h = act(Wg xn) * (Wu xn) with xn = RMSNorm(x) (if norm_w) or x."""
    f = _fmt(fmt)
    K = x.shape[-1]
    batch = 1 if x.dim() == 1 else x.shape[0]
    N = _rows(f, Wg, K)
    if _rows(f, Wu, K) != N:
        raise ValueError("gate and up must have the same shape")
    shape = (N,) if x.dim() == 1 else (batch, N)
    if h is None:
        h = torch.empty(shape, dtype=torch.float32, device=x.device)
    nw = _dev(norm_w, "norm_w", torch.float32) if norm_w is not None else None
    gp = _dev(g_out, "g_out", torch.float32) if g_out is not None else None
    up = _dev(u_out, "u_out", torch.float32) if u_out is not None else None
    st = lib().qffn_gate_up_act(f, _dev(Wg, "Wg", torch.uint8), _dev(Wu, "Wu", torch.uint8),
                                _dev(x, "x", torch.float32), nw, float(eps), _act(act),
                                _dev(h, "h", torch.float32), gp, up, N, K, batch, _stream())
    _check("qffn_gate_up_act", st)
    return h


def qffn_decode(fmt_gu, Wg: torch.Tensor, Wu: torch.Tensor, fmt_down, Wd: torch.Tensor,
                x: torch.Tensor, norm_w: torch.Tensor | None = None, eps: float = 1e-6,
                act="gelu_tanh", y: torch.Tensor | None = None,
                h_out: torch.Tensor | None = None) -> torch.Tensor:
    """y = Wd (act(Wg xn) * (Wu xn)): the decode FFN of one layer."""
    fg, fd = _fmt(fmt_gu), _fmt(fmt_down)
    K = x.shape[-1]
    batch = 1 if x.dim() == 1 else x.shape[0]
    N = _rows(fg, Wg, K)
    if _rows(fg, Wu, K) != N or _rows(fd, Wd, N) != K:
        raise ValueError("gate/up must be N_ff x K and down K x N_ff")
    if y is None:
        y = torch.empty_like(x)
    nw = _dev(norm_w, "norm_w", torch.float32) if norm_w is not None else None
    hp = _dev(h_out, "h_out", torch.float32) if h_out is not None else None
    st = lib().qffn_decode(fg, _dev(Wg, "Wg", torch.uint8), _dev(Wu, "Wu", torch.uint8), fd,
                           _dev(Wd, "Wd", torch.uint8), _dev(x, "x", torch.float32), nw, float(eps),
                           _act(act), _dev(y, "y", torch.float32), hp, N, K, batch, _stream())
    _check("qffn_decode", st)
    return y


def qffn_decode_noalloc(fmt_gu, Wg: torch.Tensor, Wu: torch.Tensor, fmt_down, Wd: torch.Tensor,
                        x: torch.Tensor, norm_w: torch.Tensor | None, eps: float, act, y: torch.Tensor,
                        h_out: torch.Tensor | None = None) -> torch.Tensor:
    """qffn_decode with h and partial sums in the library's fixed per-GPU
    scratch (no allocation); y must be given."""
    fg, fd = _fmt(fmt_gu), _fmt(fmt_down)
    K = x.shape[-1]
    batch = 1 if x.dim() == 1 else x.shape[0]
    N = _rows(fg, Wg, K)
    if _rows(fg, Wu, K) != N or _rows(fd, Wd, N) != K:
        raise ValueError("gate/up must be N_ff x K and down K x N_ff")
    nw = _dev(norm_w, "norm_w", torch.float32) if norm_w is not None else None
    hp = _dev(h_out, "h_out", torch.float32) if h_out is not None else None
    st = lib().qffn_decode_noalloc(fg, _dev(Wg, "Wg", torch.uint8), _dev(Wu, "Wu", torch.uint8), fd,
                                   _dev(Wd, "Wd", torch.uint8), _dev(x, "x", torch.float32), nw, float(eps),
                                   _act(act), _dev(y, "y", torch.float32), hp, N, K, batch, _stream())
    _check("qffn_decode_noalloc", st)
    return y


def qffn_decode_residual(fmt_gu, Wg: torch.Tensor, Wu: torch.Tensor, fmt_down, Wd: torch.Tensor,
                         x: torch.Tensor, r: torch.Tensor, norm_w: torch.Tensor | None = None,
                         eps: float = 1e-6, act="gelu_tanh", y: torch.Tensor | None = None,
                         h_out: torch.Tensor | None = None) -> torch.Tensor:
    """y = Wd (act(Wg xn) * (Wu xn)) + r (pass y=r to add in place)."""
    fg, fd = _fmt(fmt_gu), _fmt(fmt_down)
    K = x.shape[-1]
    batch = 1 if x.dim() == 1 else x.shape[0]
    N = _rows(fg, Wg, K)
    if _rows(fg, Wu, K) != N or _rows(fd, Wd, N) != K:
        raise ValueError("gate/up must be N_ff x K and down K x N_ff")
    if tuple(r.shape) != tuple(x.shape):
        raise ValueError("r must have x's shape")
    if y is None:
        y = torch.empty_like(x)
    nw = _dev(norm_w, "norm_w", torch.float32) if norm_w is not None else None
    hp = _dev(h_out, "h_out", torch.float32) if h_out is not None else None
    st = lib().qffn_decode_residual(fg, _dev(Wg, "Wg", torch.uint8), _dev(Wu, "Wu", torch.uint8), fd,
                                    _dev(Wd, "Wd", torch.uint8), _dev(x, "x", torch.float32), nw,
                                    float(eps), _act(act), _dev(r, "r", torch.float32),
                                    _dev(y, "y", torch.float32), hp, N, K, batch, _stream())
    _check("qffn_decode_residual", st)
    return y


def qmoe_ffn_decode(fmt_gu, Wg: torch.Tensor, Wu: torch.Tensor, fmt_down, Wd: torch.Tensor,
                    n_experts: int, ids: torch.Tensor, coef: torch.Tensor, x: torch.Tensor,
                    norm_w: torch.Tensor | None = None, eps: float = 1e-6, act="gelu_tanh",
                    y: torch.Tensor | None = None, h_out: torch.Tensor | None = None) -> torch.Tensor:
    """y = sum_z coef[z] Wd[ids[z]] (act(Wg[ids[z]] xn) * (Wu[ids[z]] xn)) for one token.
    Wg, Wu, Wd hold n_experts stacked matrices; ids (int32) and coef (fp32)
    are device tensors of n_sel slots."""
    fg, fd = _fmt(fmt_gu), _fmt(fmt_down)
    K = x.shape[-1]
    if x.dim() != 1:
        raise ValueError("x must be one token, shape [K]")
    if Wg.numel() % n_experts or Wd.numel() % n_experts:
        raise ValueError("weights must hold n_experts equal matrices")
    N = _rows(fg, Wg[: Wg.numel() // n_experts], K)
    if Wu.numel() != Wg.numel() or _rows(fd, Wd[: Wd.numel() // n_experts], N) != K:
        raise ValueError("gate/up must be n_experts x N_ff x K and down n_experts x K x N_ff")
    n_sel = ids.numel()
    if coef.numel() != n_sel:
        raise ValueError("ids and coef must have one entry per slot")
    if y is None:
        y = torch.empty_like(x)
    nw = _dev(norm_w, "norm_w", torch.float32) if norm_w is not None else None
    hp = _dev(h_out, "h_out", torch.float32) if h_out is not None else None
    st = lib().qmoe_ffn_decode(fg, _dev(Wg, "Wg", torch.uint8), _dev(Wu, "Wu", torch.uint8), fd,
                               _dev(Wd, "Wd", torch.uint8), n_experts, _dev(ids, "ids", torch.int32),
                               _dev(coef, "coef", torch.float32), n_sel, _dev(x, "x", torch.float32), nw,
                               float(eps), _act(act), _dev(y, "y", torch.float32), hp, N, K, _stream())
    _check("qmoe_ffn_decode", st)
    return y


def qgemm_prefill(fmt, W: torch.Tensor, X: torch.Tensor, Y: torch.Tensor | None = None) -> torch.Tensor:
    """Y = X bf16(W)^T.  X: bf16 bits as int16/uint16 or torch.bfloat16 [M, K]."""
    f = _fmt(fmt)
    M, K = X.shape
    N = _rows(f, W, K)
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float32, device=X.device)
    st = lib().qgemm_prefill(f, _dev(W, "W", torch.uint8), _dev(X, "X", X.dtype if X.dtype in
                             (torch.bfloat16, torch.int16, torch.uint16) else torch.bfloat16),
                             _dev(Y, "Y", torch.float32), M, N, K, _stream())
    _check("qgemm_prefill", st)
    return Y


def qgemm_prefill_gate_up_act(fmt, Wg, Wu, X, act="gelu_tanh", H=None, g_out=None, u_out=None):
    """H = bf16(act(X Wg^T) * (X Wu^T)); X and H bf16 [M, *]."""
    f = _fmt(fmt)
    M, K = X.shape
    N = _rows(f, Wg, K)
    if _rows(f, Wu, K) != N:
        raise ValueError("gate and up must have the same shape")
    if H is None:
        H = torch.empty((M, N), dtype=torch.bfloat16, device=X.device)
    xdt = X.dtype if X.dtype in (torch.bfloat16, torch.int16, torch.uint16) else torch.bfloat16
    hdt = H.dtype if H.dtype in (torch.bfloat16, torch.int16, torch.uint16) else torch.bfloat16
    gp = _dev(g_out, "g_out", torch.float32) if g_out is not None else None
    up = _dev(u_out, "u_out", torch.float32) if u_out is not None else None
    st = lib().qgemm_prefill_gate_up_act(f, _dev(Wg, "Wg", torch.uint8), _dev(Wu, "Wu", torch.uint8),
                                         _dev(X, "X", xdt), _act(act), _dev(H, "H", hdt), gp, up,
                                         M, N, K, _stream())
    _check("qgemm_prefill_gate_up_act", st)
    return H


def qdequant(fmt, W: torch.Tensor, K: int, out: torch.Tensor | None = None) -> torch.Tensor:
    """fp32 [N, K] dequantised weights."""
    f = _fmt(fmt)
    N = _rows(f, W, K)
    if out is None:
        out = torch.empty((N, K), dtype=torch.float32, device=W.device)
    st = lib().qdequant(f, _dev(W, "W", torch.uint8), _dev(out, "out", torch.float32), N, K, _stream())
    _check("qdequant", st)
    return out


def qdequant_bf16(fmt, W: torch.Tensor, K: int, out: torch.Tensor | None = None) -> torch.Tensor:
    """bf16 bits (int16 tensor) [N, K] of the dequantised weights."""
    f = _fmt(fmt)
    N = _rows(f, W, K)
    if out is None:
        out = torch.empty((N, K), dtype=torch.int16, device=W.device)
    st = lib().qdequant_bf16(f, _dev(W, "W", torch.uint8), _dev(out, "out", out.dtype), N, K, _stream())
    _check("qdequant_bf16", st)
    return out


def set_gemm_override(tm: int = 0, splits: int = 0):
    """Prefill tile override (0 = automatic)."""
    _check("qd_set_gemm_override", lib().qd_set_gemm_override(tm, splits))


def set_gemm_streamk(units_per_wg: int = 0):
    """Prefill stream-K: 0 off, > 0 that many (tile, K-tile) units per workgroup."""
    _check("qd_set_gemm_streamk", lib().qd_set_gemm_streamk(units_per_wg))


def set_stream_override(wg_per_cu: int = 0, depth: int = 0, consumers: int = 0, producers: int = 0):
    """Streaming GEMV shape override (0 = automatic): workgroups per CU, steps
    in flight per copying wave, decoding waves (4 or 8) and copying waves
    (1, 2 or 4)."""
    _check("qd_set_stream_override",
           lib().qd_set_stream_override(wg_per_cu, depth, consumers, producers))


def set_batch_override(mode: int = 0, k_slices: int = 0):
    """Batch 3..64 path: 0 = the matrix-core kernels (automatic), 1 = the fp32
    register kernel in launches of 8 batch rows; k_slices = K-slices of the
    matrix-core kernels (0 = automatic)."""
    _check("qd_set_batch_override", lib().qd_set_batch_override(mode, k_slices))


def set_walk_override(rows_per_group: int = 0):
    """Row slots each lane group of the register-streaming GEMV walks
    (0 = automatic)."""
    _check("qd_set_walk_override", lib().qd_set_walk_override(rows_per_group))


def set_launch_override(p_in: int = 0, p_out: int = 0, nr: int = 0):
    """Force the GEMV launch shape for tuning sweeps (0 = automatic)."""
    _check("qd_set_launch_override", lib().qd_set_launch_override(p_in, p_out, nr))


def plan_q8act(N: int, K: int, batch: int = 1):
    """(lane groups per row, K-slices, superunits per slice, columns per
    launch) of the int8-activation GEMV for this shape; host only."""
    out = (ctypes.c_int32 * 4)()
    _check("qd_plan_q8act", lib().qd_plan_q8act(N, K, batch, out))
    return tuple(out)
