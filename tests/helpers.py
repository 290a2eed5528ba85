"""Helpers shared by the GPU parity tests: device transfer, case banners,
and the output bounds (the 1e-4 * sum|w x| + 1e-6 bar, and its propagation
through the FFN activation)."""
import numpy as np
import torch

import oracle


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def say(msg):
    print(f"[case] {msg}", flush=True)


def assert_bound(name, got, y64, S, rows=None):
    got = np.asarray(got, dtype=np.float64)
    if rows is not None:
        got, y64, S = got[..., rows], y64[..., rows], S[..., rows]
    err = np.abs(got - y64)
    bound = 1e-4 * S + 1e-6
    bad = ~(err <= bound)   # NaN fails
    if bad.any():
        idx = np.unravel_index(np.argmax(err / bound), err.shape)
        raise AssertionError(f"{name}: {bad.sum()} outputs out of bound; worst at {idx}: "
                             f"got {got[idx]!r} ref {y64[idx]!r} err {err[idx]:.3e} bound {bound[idx]:.3e}")
    return float((err / bound).max())


GELU_LIP, SILU_LIP = 1.13, 1.10


def h_tolerance(g64, u64, Sg, Su, act):
    """|act(g) u - act(g~) u~| for |g - g~| <= eg, |u - u~| <= eu, plus the
    fp32 evaluation of act and the product (relative 1e-5)."""
    L = GELU_LIP if act == oracle.ACT_GELU_TANH else SILU_LIP
    eg = 1e-4 * Sg + 1e-6
    eu = 1e-4 * Su + 1e-6
    ag = np.abs(oracle.act_vec(act, g64))
    return L * eg * (np.abs(u64) + eu) + ag * eu + 1e-5 * ag * np.abs(u64) + 1e-7


def pack_q4k_blocks(d, dmin, sc, m, q):
    """Q4_K blocks (uint8 [n, 144]) from per-block d, dmin (values rounded to
    f16), per-sub-block scales and mins (ints 0..63, [n, 8]) and quants
    (ints 0..15, [n, 256]); written from the encoder side of the layout."""
    d = np.asarray(d, np.float16)
    dmin = np.asarray(dmin, np.float16)
    sc = np.asarray(sc, np.int64)
    m = np.asarray(m, np.int64)
    q = np.asarray(q, np.int64)
    n = d.shape[0]
    b = np.zeros((n, 144), np.uint8)
    b[:, 0:2] = d.reshape(n, 1).view(np.uint8)
    b[:, 2:4] = dmin.reshape(n, 1).view(np.uint8)
    s = np.zeros((n, 12), np.int64)
    for j in range(4):
        s[:, j] = sc[:, j] | ((sc[:, j + 4] >> 4) << 6)
        s[:, j + 4] = m[:, j] | ((m[:, j + 4] >> 4) << 6)
        s[:, j + 8] = (sc[:, j + 4] & 15) | ((m[:, j + 4] & 15) << 4)
    b[:, 4:16] = s.astype(np.uint8)
    for run in range(4):
        lo = q[:, 64 * run: 64 * run + 32]
        hi = q[:, 64 * run + 32: 64 * run + 64]
        b[:, 16 + 32 * run: 48 + 32 * run] = (lo | (hi << 4)).astype(np.uint8)
    return b


def cancelling_q4k(N, K, seed, flip_frac=0.0):
    """A Q4_K matrix whose sub-blocks cancel: every sub-block has a constant
    quant q0 and a min with d*sc*q0 == dmin*m exactly (dmin = d or 2d), so
    its weights are zero; with flip_frac > 0 that fraction of quants is
    moved by +-1 from q0, leaving a few weights of +-d*sc among zeros.
    Scales are large (d*sc*q0 up to ~0.6), so the scale and min terms of a
    sub-block are large while the weights are zero or small."""
    rng = np.random.default_rng(seed)
    nblk = N * (K // 256)
    d = rng.uniform(1e-3, 1e-2, nblk).astype(np.float16)
    two = rng.integers(0, 2, nblk).astype(bool)
    dmin = np.where(two, d.astype(np.float32) * 2, d.astype(np.float32)).astype(np.float16)
    sc = np.zeros((nblk, 8), np.int64)
    m = np.zeros((nblk, 8), np.int64)
    q0 = np.zeros((nblk, 8), np.int64)
    for j in range(8):
        qq = rng.integers(1, 16, nblk)                        # constant quant
        hi = 63 // qq                                         # sc * q0 <= 63
        ss = 1 + np.floor(rng.random(nblk) * hi).astype(np.int64)
        need_even = two & (qq % 2 == 1)                       # m = sc * q0 / 2
        ss = np.where(need_even, np.maximum(2, ss - ss % 2), ss)
        prod = ss * qq
        m[:, j] = np.where(two, prod // 2, prod)
        sc[:, j] = ss
        q0[:, j] = qq
    q = np.repeat(q0, 32, axis=1)
    if flip_frac > 0:
        flip = rng.random(q.shape) < flip_frac
        step = np.where(rng.random(q.shape) < 0.5, -1, 1)
        q = np.where(flip, np.clip(q + step, 0, 15), q)
    return pack_q4k_blocks(d, dmin, sc, m, q).reshape(-1)


def post_norm_bound(p64, S, r, w1, eps, y_ref):
    """Bound on |y - y_ref| for y = r + p * w1 / sqrt(mean(p^2) + eps) when p
    carries the GEMV error e = 1e-4 * S + 1e-6 per element (p64, S from the
    oracle; rows are batch columns).  With rho = 1/rms and
    D = sum(2|p| e + e^2) / (sum p^2 + N eps) + 3e-6 (the change of the mean
    square, plus fp32 evaluation of the sum and the root), the relative
    change of rho is at most D, so the normalised term moves by at most
    |w1| rho (e (1 + D) + |p| D); the products and the add round in fp32
    (2^-23 of each magnitude)."""
    p64 = np.atleast_2d(p64)
    S = np.atleast_2d(S)
    N = p64.shape[-1]
    e = 1e-4 * S + 1e-6
    ss = (p64 ** 2).sum(-1, keepdims=True)
    D = (2 * np.abs(p64) * e + e * e).sum(-1, keepdims=True) / (ss + N * eps) + 3e-6
    rho = 1.0 / np.sqrt(ss / N + eps)
    w = np.abs(np.asarray(w1, np.float64))
    n = np.abs(p64) * rho * w
    return w * rho * (e * (1 + D) + np.abs(p64) * D) + 2.0 ** -23 * (n + np.abs(np.atleast_2d(y_ref)))


def rmsnorm_eval_bound(ref):
    """fp32 evaluation error of an RMS-norm of N <= 32768 values computed
    from the same fp32 inputs as the fp64 reference: the sum of squares
    (chains of at most 128 terms plus a 10-level tree), the root, the
    reciprocal and two products, all within 4e-6 relative, plus 1e-30."""
    return 4e-6 * np.abs(ref) + 1e-30
