"""Q4_K blocks whose scale and min terms cancel, through every Q4_K kernel
path, against the oracle.

A Q4_K weight is d*sc*q - dmin*m.  In a sub-block with a constant quant q0
and d*sc*q0 == dmin*m exactly, every weight is zero although both terms are
large (up to ~0.6 here); with a few quants moved by +-1, a few weights are
+-d*sc among zeros.  A kernel that applied the scale and the min per
sub-block in fp32 (d*sc*sum(q x) - dmin*m*sum(x)) would carry the rounding
error of those large terms into an output whose bound, 1e-4 * sum|w x| +
1e-6, is set by the small weights alone (1e-6 for an all-zero row).  The
batch-1..2 paths form sum(q X) and sum(X) exactly in integers and combine
the two terms in fp64 (one rounding of the exact value), the batch-3..8
paths form each weight first; either way all-zero rows come out as exact
zeros and the rest within the bound: the register GEMV (several launch shapes, split-K across
workgroups, row walks, batch 1-8), the LDS-streaming GEMV (automatic at
K >= 8192 and forced at K = 2560 / 5376), the fused gate/up, the fused
Q/K/V launch, the mixture-of-experts launches and the prefill GEMM.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import assert_bound, cancelling_q4k, dev, h_tolerance, say

pytestmark = pytest.mark.gpu

SEED = 0x5EED


@pytest.fixture(scope="module")
def qd(gpu):
    import quantized_decode_q4k_amd as qd
    qd.lib()
    yield qd
    qd.set_launch_override(0, 0, 0)
    qd.set_walk_override(0)
    qd.set_stream_override(0, 0, 0, 0)


def _check(name, y, W, x, N, K, zero_rows_exact):
    y64, S = oracle.gemv("q4_k", W, x, N, K)
    assert_bound(name, y, y64, S)
    if zero_rows_exact:
        assert not np.asarray(y).any(), f"{name}: all-zero weights gave a non-zero output"


@pytest.mark.parametrize("flip", [0.0, 0.03])
@pytest.mark.parametrize("N,K", [(300, 2560), (64, 5376), (40, 10240)])
@pytest.mark.parametrize("batch", [1, 2, 8, 40])
def test_cancel_gemv_automatic(qd, flip, N, K, batch):
    say(f"q4k cancel gemv N={N} K={K} batch={batch} flip={flip}")
    W = cancelling_q4k(N, K, seed=N + K + batch, flip_frac=flip)
    x = synth.normal((batch, K), SEED, tensor_id=201)
    y = qd.qgemv_q4k(dev(W), dev(x)).cpu().numpy()
    _check(f"auto {N}x{K} b{batch} flip={flip}", y, W, x, N, K, flip == 0.0)


# (p_in, p_out, nr, row slots per lane group)
SHAPES = [(1, 1, 1, 1), (2, 1, 2, 2), (4, 3, 1, 1), (16, 1, 1, 1), (1, 4, 2, 3), (8, 2, 1, 2)]


@pytest.mark.parametrize("flip", [0.0, 0.03])
@pytest.mark.parametrize("batch", [1, 3])
def test_cancel_gemv_forced_shapes(qd, flip, batch):
    N, K = 130, 2560
    W = cancelling_q4k(N, K, seed=7, flip_frac=flip)
    x = synth.normal((batch, K), SEED, tensor_id=202)
    Wd, xd = dev(W), dev(x)
    try:
        for p_in, p_out, nr, rpg in SHAPES:
            say(f"q4k cancel forced p_in={p_in} p_out={p_out} nr={nr} rpg={rpg} batch={batch} flip={flip}")
            qd.set_launch_override(p_in, p_out, nr)
            qd.set_walk_override(rpg)
            y = qd.qgemv_q4k(Wd, xd).cpu().numpy()
            _check(f"forced {p_in}/{p_out}/{nr}/{rpg}", y, W, x, N, K, flip == 0.0)
    finally:
        qd.set_launch_override(0, 0, 0)
        qd.set_walk_override(0)


@pytest.mark.parametrize("flip", [0.0, 0.03])
@pytest.mark.parametrize("K", [2560, 5376])
@pytest.mark.parametrize("batch", [1, 2])
def test_cancel_gemv_streaming_forced(qd, flip, K, batch):
    N = 257
    W = cancelling_q4k(N, K, seed=11, flip_frac=flip)
    x = synth.normal((batch, K), SEED, tensor_id=203)
    Wd, xd = dev(W), dev(x)
    try:
        for wpc, cons, prod in ((1, 8, 2), (2, 4, 2), (1, 4, 4)):
            say(f"q4k cancel stream K={K} batch={batch} wpc={wpc} cons={cons} prod={prod} flip={flip}")
            qd.set_stream_override(wpc, 0, cons, prod)
            y = qd.qgemv_q4k(Wd, xd).cpu().numpy()
            _check(f"stream {wpc}/{cons}/{prod}", y, W, x, N, K, flip == 0.0)
    finally:
        qd.set_stream_override(0, 0, 0, 0)


@pytest.mark.parametrize("N,K,batch", [(10240, 2560, 1), (512, 2560, 8), (300, 10240, 2)])
def test_cancel_gate_up(qd, N, K, batch):
    """Fused gate/up with cancelling gate and up: g and u within the bound
    (exact zeros where every weight is zero), h within the propagated bound."""
    say(f"q4k cancel gate/up N={N} K={K} batch={batch}")
    Wg = cancelling_q4k(N, K, seed=21, flip_frac=0.02)
    Wu = cancelling_q4k(N, K, seed=22, flip_frac=0.0)
    x = synth.normal((batch, K), SEED, tensor_id=204)
    nw = synth.normal((K,), SEED, tensor_id=205, mean=1.0, std=0.1)
    g = torch.empty((batch, N), device="cuda")
    u = torch.empty((batch, N), device="cuda")
    h = qd.qffn_gate_up_act("q4_k", dev(Wg), dev(Wu), dev(x), dev(nw), 1e-6, "gelu_tanh",
                            g_out=g, u_out=u).cpu().numpy()
    xn = oracle.rmsnorm(x, nw, 1e-6).astype(np.float32)
    g64, Sg = oracle.gemv("q4_k", Wg, xn, N, K)
    u64, Su = oracle.gemv("q4_k", Wu, xn, N, K)
    assert_bound("gate", g.cpu().numpy(), g64, Sg)
    uu = u.cpu().numpy()
    assert_bound("up", uu, u64, Su)
    assert not uu.any(), "all-zero up weights gave a non-zero output"
    tol = h_tolerance(g64, u64, Sg, Su, oracle.ACT_GELU_TANH)
    href = oracle.act_vec(oracle.ACT_GELU_TANH, g64) * u64
    assert (np.abs(h - href) <= tol).all()


def test_cancel_qkv(qd):
    K = 2560
    say("q4k cancel qkv")
    Ws = [cancelling_q4k(n, K, seed=30 + i, flip_frac=f) for i, (n, f) in
          enumerate(((2048, 0.0), (1024, 0.03), (1024, 0.0)))]
    x = synth.normal((1, K), SEED, tensor_id=206)
    nw = synth.normal((K,), SEED, tensor_id=207, mean=1.0, std=0.1)
    q, k, v = qd.qqkv_proj(("q4_k",) * 3, *(dev(W) for W in Ws), dev(x), dev(nw), 1e-6)
    xn = oracle.rmsnorm(x, nw, 1e-6).astype(np.float32)
    for name, W, out, n, exact in (("q", Ws[0], q, 2048, True), ("k", Ws[1], k, 1024, False),
                                   ("v", Ws[2], v, 1024, True)):
        _check(f"qkv {name}", out.cpu().numpy(), W, xn, n, K, exact)


def test_cancel_moe(qd):
    """Mixture-of-experts with cancelling Q4_K experts: every h exactly zero
    (gate weights zero), so y is exactly zero too."""
    n_exp, ff, hidden = 6, 512, 512
    say("q4k cancel moe")
    Wg = cancelling_q4k(n_exp * ff, hidden, seed=41)
    Wu = cancelling_q4k(n_exp * ff, hidden, seed=42, flip_frac=0.05)
    Wd = cancelling_q4k(n_exp * hidden, ff, seed=43, flip_frac=0.05)
    x = synth.normal((hidden,), SEED, tensor_id=208)
    ids = torch.tensor([1, 4, 0], dtype=torch.int32, device="cuda")
    coef = torch.tensor([0.5, 0.3, 0.2], dtype=torch.float32, device="cuda")
    h = torch.empty((3, ff), device="cuda")
    y = qd.qmoe_ffn_decode("q4_k", dev(Wg), dev(Wu), "q4_k", dev(Wd), n_exp, ids, coef, dev(x), None, 1e-6,
                           "silu", h_out=h).cpu().numpy()
    assert not h.cpu().numpy().any()
    assert not y.any()


def test_cancel_prefill(qd):
    """The prefill GEMM on cancelling Q4_K weights: bf16(w) of a zero weight
    is zero, so all-zero rows give exact zero columns."""
    M, N, K = 64, 256, 512
    say("q4k cancel prefill")
    W = cancelling_q4k(N, K, seed=51)
    X = synth.normal_bf16((M, K), SEED, tensor_id=209)
    Y = qd.qgemm_prefill("q4_k", dev(W), dev(X.view(np.int16))).cpu().numpy()
    assert not Y.any()
