"""GPU parity of the prefill GEMMs (qgemm_prefill, qgemm_prefill_gate_up_act)
against the oracle's dequantise -> bf16 (nearest even) -> fp64 contraction.

Bars:
  * the bf16 weights are bit-exact: with identity activations (X = I) every
    output is one product 1 * bf16(w), so Y = bf16(W)^T exactly;
  * |Y - Y64| <= 1e-4 * sum_k |bf16(w) x| + 1e-6, Y64 and the sum in fp64;
  * H = bf16(act(g) u): g and u meet the bar above, and H meets the bound
    propagated through the activation plus its own bf16 rounding (2^-8
    relative).
The Gemma-4-31B prefill case (512 tokens, hidden 5376, intermediate 21504)
runs in the launch configuration bench.py times and is checked on every
output; the down projection is checked on the GPU's own H.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import assert_bound, dev, h_tolerance, say

pytestmark = pytest.mark.gpu

SEED = 0x5EED
BF16_ONE = 0x3F80


@pytest.fixture(scope="module")
def qd(gpu):
    import quantized_decode_q4k_amd as qd
    qd.lib()
    yield qd
    qd.set_gemm_override(0, 0)


def xdev(X):
    """bf16 bits (uint16) to a device int16 tensor (the binding takes either)."""
    return dev(np.ascontiguousarray(X).view(np.int16))


def bf16_of(ref32):
    """Nearest-even bf16 of each fp32 value, as fp32 (oracle rounding)."""
    flat = np.array([oracle.f32_to_bf16(float(v)) for v in ref32.ravel()], np.uint32)
    return (flat << 16).view(np.float32).reshape(ref32.shape)


def h_bound(g64, u64, Sg, Su, aid):
    tol = h_tolerance(g64, u64, Sg, Su, aid)
    href = oracle.act_vec(aid, g64) * u64
    return href, tol + 2.0 ** -8 * (np.abs(href) + tol)


def act_id(act):
    return oracle.ACT_GELU_TANH if act == "gelu_tanh" else oracle.ACT_SILU


def run_override(qd, tm, splits, fn):
    qd.set_gemm_override(tm, splits)
    try:
        return fn()
    finally:
        qd.set_gemm_override(0, 0)


# ----------------------------------------------------- bf16 weights exact ---

@pytest.mark.parametrize("fmt,K", [("q4_k", 512), ("q6_k", 512), ("q8_0", 160), ("q8_0", 512)])
@pytest.mark.parametrize("splits", [1, 2])
def test_prefill_identity_gives_bf16_weights(qd, fmt, K, splits):
    N = 300
    say(f"prefill identity {fmt} N={N} K={K} splits={splits}")
    W = synth.quant_weights(fmt, N, K, SEED, tensor_id=61)
    X = np.zeros((K, K), np.uint16)
    X[np.arange(K), np.arange(K)] = BF16_ONE
    Y = run_override(qd, 0, splits, lambda: qd.qgemm_prefill(fmt, dev(W), xdev(X)).cpu().numpy())
    ref = bf16_of(oracle.dequant(fmt, W, K)).T  # [K tokens][N]
    # +0.0 normalises the sign of zero (a sum of +0 and -0 products is +0)
    assert np.array_equal((Y + 0.0).view(np.uint32), (ref + 0.0).view(np.uint32))


# ------------------------------------------------------------ small GEMM ---

SMALL = [("q4_k", 77, 300, 768), ("q4_k", 1, 40, 256), ("q6_k", 130, 513, 512),
         ("q6_k", 5, 64, 768), ("q8_0", 77, 300, 416), ("q8_0", 33, 257, 96),
         ("q8_0", 1, 7, 32)]


@pytest.mark.parametrize("fmt,M,N,K", SMALL)
@pytest.mark.parametrize("tm,splits", [(0, 0), (2, 1), (4, 3)])
def test_prefill_small(qd, fmt, M, N, K, tm, splits):
    say(f"prefill {fmt} M={M} N={N} K={K} tm={tm} splits={splits}")
    W = synth.quant_weights(fmt, N, K, SEED, tensor_id=62)
    X = synth.normal_bf16((M, K), SEED, tensor_id=63)
    Y = run_override(qd, tm, splits, lambda: qd.qgemm_prefill(fmt, dev(W), xdev(X)).cpu().numpy())
    y64, S = oracle.gemm_bf16(fmt, W, X, N, K)
    assert_bound(f"prefill {fmt}", Y, y64, S)


def test_prefill_split_k_deterministic(qd):
    fmt, M, N, K = "q4_k", 200, 700, 2048
    say(f"prefill split-K determinism {fmt} M={M} N={N} K={K}")
    W = synth.quant_weights(fmt, N, K, SEED, tensor_id=64)
    X = synth.normal_bf16((M, K), SEED, tensor_id=65)
    Wd, Xd = dev(W), xdev(X)
    runs = [run_override(qd, 4, 4, lambda: qd.qgemm_prefill(fmt, Wd, Xd).cpu().numpy())
            for _ in range(3)]
    assert all(np.array_equal(runs[0].view(np.uint32), r.view(np.uint32)) for r in runs[1:])
    y64, S = oracle.gemm_bf16(fmt, W, X, N, K)
    assert_bound("split-K", runs[0], y64, S)
    one = run_override(qd, 4, 1, lambda: qd.qgemm_prefill(fmt, Wd, Xd).cpu().numpy())
    assert_bound("no split", one, y64, S)


# ------------------------------------------------------------- stream-K ---

def run_streamk(qd, per, fn, tm=0):
    qd.set_gemm_streamk(per)
    qd.set_gemm_override(tm, 0)
    try:
        return fn()
    finally:
        qd.set_gemm_streamk(0)
        qd.set_gemm_override(0, 0)


@pytest.mark.parametrize("fmt,M,N,K", [("q4_k", 300, 700, 2048), ("q6_k", 130, 513, 1536),
                                       ("q8_0", 77, 300, 416)])
@pytest.mark.parametrize("per", [3, 5, 16, 37])
def test_prefill_streamk(qd, fmt, M, N, K, per):
    """Stream-K runs of units shorter and longer than a tile's K-tiles (16,
    12 and 4 of them here): tiles shared by up to six workgroups, workgroups
    holding only the middle of one tile, several whole tiles, ragged ends and
    a K-tile past K.  Repeat calls are bitwise equal; every output is within
    the bound."""
    say(f"prefill stream-K {fmt} M={M} N={N} K={K} per={per}")
    W = synth.quant_weights(fmt, N, K, SEED, tensor_id=66)
    X = synth.normal_bf16((M, K), SEED, tensor_id=67)
    Wd, Xd = dev(W), xdev(X)
    runs = [run_streamk(qd, per, lambda: qd.qgemm_prefill(fmt, Wd, Xd).cpu().numpy()) for _ in range(2)]
    assert np.array_equal(runs[0].view(np.uint32), runs[1].view(np.uint32))
    y64, S = oracle.gemm_bf16(fmt, W, X, N, K)
    assert_bound(f"stream-K {fmt}", runs[0], y64, S)


@pytest.mark.parametrize("per,tm", [(7, 4), (3, 2)])
def test_prefill_ffn_streamk(qd, per, tm):
    qd.set_gemm_streamk(per)
    try:
        check_prefill_ffn(qd, "q4_k", 200, 300, 1536, "silu", f"stream-K {per}", tm=tm)
    finally:
        qd.set_gemm_streamk(0)


# --------------------------------------------------------- gate/up + act ---

def check_prefill_ffn(qd, fmt, M, N, K, act, tag, cols=None, tm=0, splits=0):
    Wg = synth.quant_weights(fmt, N, K, SEED, tensor_id=71)
    Wu = synth.quant_weights(fmt, N, K, SEED, tensor_id=72)
    X = synth.normal_bf16((M, K), SEED, tensor_id=73)
    say(f"prefill ffn {tag} {fmt} M={M} N={N} K={K} act={act}")
    import torch
    g = torch.empty((M, N), device="cuda")
    u = torch.empty((M, N), device="cuda")
    Wgd, Wud, Xd = dev(Wg), dev(Wu), xdev(X)
    H = run_override(qd, tm, splits, lambda: qd.qgemm_prefill_gate_up_act(
        fmt, Wgd, Wud, Xd, act, g_out=g, u_out=u))
    H2 = run_override(qd, tm, splits, lambda: qd.qgemm_prefill_gate_up_act(fmt, Wgd, Wud, Xd, act))
    H = H.view(torch.int16).cpu().numpy().view(np.uint16)
    H2 = H2.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(H, H2), "H depends on whether g/u are written"
    g, u = g.cpu().numpy(), u.cpu().numpy()
    if cols is None:
        cols = np.arange(N)
        th = oracle.host_threads()
        g64, Sg = oracle.gemm_bf16_threaded(fmt, Wg, X, N, K, th)
        u64, Su = oracle.gemm_bf16_threaded(fmt, Wu, X, N, K, th)
    else:
        g64, Sg = oracle.gemm_bf16_cols(fmt, Wg, X, N, K, cols)
        u64, Su = oracle.gemm_bf16_cols(fmt, Wu, X, N, K, cols)
    assert_bound(f"{tag} gate", g[:, cols], g64, Sg)
    assert_bound(f"{tag} up", u[:, cols], u64, Su)
    href, bound = h_bound(g64, u64, Sg, Su, act_id(act))
    hgot = (H[:, cols].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    err = np.abs(hgot - href)
    assert (err <= bound).all(), f"{tag} H: worst {np.max(err / bound):.3f} of the bound"
    return H


@pytest.mark.parametrize("fmt,K", [("q4_k", 512), ("q6_k", 256), ("q8_0", 416)])
@pytest.mark.parametrize("act", ["gelu_tanh", "silu"])
def test_prefill_ffn_small(qd, fmt, K, act):
    check_prefill_ffn(qd, fmt, 130, 300, K, act, "small")


def test_prefill_ffn_split_k(qd):
    check_prefill_ffn(qd, "q4_k", 70, 200, 1536, "gelu_tanh", "split", tm=2, splits=3)


# ------------------------------------------- Gemma-4-31B prefill (512 tok) ---

def test_config_gemma4_31b_prefill_gate_up(qd):
    """Every (token, row) of the Gemma-4-31B prefill gate/up (512 tokens x
    21504 rows of each) against the oracle, the oracle's rows split over the
    host threads."""
    M, hidden, ff = 512, synth.GEMMA4_HIDDEN, synth.GEMMA4_FF
    check_prefill_ffn(qd, "q4_k", M, ff, hidden, "gelu_tanh", "gemma4 gate/up")


def test_config_gemma4_31b_prefill_down(qd):
    """Every output of the Gemma-4-31B prefill down projection (512 tokens x
    5376 rows, K = 21504) on the GPU's own H."""
    M, hidden, ff = 512, synth.GEMMA4_HIDDEN, synth.GEMMA4_FF
    Wg = synth.quant_weights("q4_k", ff, hidden, SEED, tensor_id=71)
    Wu = synth.quant_weights("q4_k", ff, hidden, SEED, tensor_id=72)
    X = synth.normal_bf16((M, hidden), SEED, tensor_id=73)
    H = qd.qgemm_prefill_gate_up_act("q4_k", dev(Wg), dev(Wu), xdev(X), "gelu_tanh")
    H = H.view(torch.int16).cpu().numpy().view(np.uint16)
    Wd = synth.quant_weights("q6_k", hidden, ff, SEED, tensor_id=74)
    say(f"prefill gemma4 down q6_k {hidden}x{ff} M={M}")
    Y = qd.qgemm_prefill("q6_k", dev(Wd), xdev(H)).cpu().numpy()
    y64, S = oracle.gemm_bf16_threaded("q6_k", Wd, H, hidden, ff, oracle.host_threads())
    assert_bound("gemma4 down", Y, y64, S)
