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
    bad = err > bound
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
