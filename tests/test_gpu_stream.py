"""GPU parity of the streaming GEMV path (weights copied through an LDS ring,
one workgroup per row range) against the oracle.

The path applies to batch 1 and 2 when the matrix is a whole number of
16-byte chunks; it is taken automatically for long rows (K >= 8192; at
batch 2 only from 4096 rows, fewer go to the register kernel) and
forced here with the stream override on shapes chosen to split rows
unevenly over workgroups, leave partial last steps and run fewer rows than
workgroups, with 4 and 8 decoding waves and one, two or four copying waves
(one and two workgroups per CU).  The Gemma-3 down
and gate/up shapes at two workgroups per CU hold more steps than the ring
has slots, so the copying waves reuse slots; a depth override of 1 keeps a
single step in flight per copying wave.  A launch override forces the
register-streaming kernel, run on the same inputs as a second check.
Bar: |y - y_ref| <= 1e-4 * sum|w x| + 1e-6 per output, h within the bound
propagated through the activation; two runs of one launch shape agree bit
for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import assert_bound, dev, h_tolerance, say

pytestmark = pytest.mark.gpu

SEED = 0x5EED


@pytest.fixture(scope="module")
def qd(gpu):
    import quantized_decode_q4k_amd as qd
    qd.lib()
    yield qd
    qd.set_launch_override(0, 0, 0)
    qd.set_stream_override(0, 0, 0, 0)


def forced(qd, wpc, fn, consumers=8, depth=0, producers=0):
    qd.set_stream_override(wpc, depth, consumers, producers)
    try:
        return fn()
    finally:
        qd.set_stream_override(0, 0, 0, 0)


# (workgroups per CU, decoding waves, copying waves)
VARIANTS = [(1, 4, 1), (1, 4, 2), (1, 4, 4), (2, 4, 2), (1, 8, 1), (1, 8, 2), (1, 8, 4), (2, 8, 2)]


def streams(fmt, N, K):
    return (N * synth.row_bytes(fmt, K)) % 16 == 0 and K % 256 == 0


# N = 1 (one workgroup), 37 (fewer rows than workgroups), 256, 257 and 600
# (rows split unevenly); K = 2048 keeps every Q6_K matrix a multiple of 16 bytes
CASES = [(fmt, N, K) for fmt in ("q4_k", "q6_k", "q8_0") for N, K in
         ((1, 2048), (37, 2048), (256, 2048), (257, 2048), (600, 2048), (64, 10240))]


@pytest.mark.parametrize("fmt,N,K", CASES)
@pytest.mark.parametrize("batch", [1, 2])
def test_stream_gemv(qd, fmt, N, K, batch):
    assert streams(fmt, N, K)
    say(f"stream gemv {fmt} N={N} K={K} batch={batch}")
    W = synth.quant_weights(fmt, N, K, SEED, tensor_id=81)
    x = synth.normal((batch, K), SEED, tensor_id=82)
    Wd, xd = dev(W), dev(x)
    y64, S = oracle.gemv(fmt, W, x, N, K)
    for wpc, cons, prod in VARIANTS:
        y = forced(qd, wpc, lambda: qd.qgemv(fmt, Wd, xd).cpu().numpy(), cons, 0, prod)
        assert_bound(f"stream {fmt} wpc={wpc} consumers={cons} producers={prod}", y, y64, S)
        again = forced(qd, wpc, lambda: qd.qgemv(fmt, Wd, xd).cpu().numpy(), cons, 0, prod)
        assert np.array_equal(y.view(np.uint32), again.view(np.uint32))
    auto = qd.qgemv(fmt, Wd, xd).cpu().numpy()
    assert_bound(f"automatic {fmt}", auto, y64, S)
    qd.set_launch_override(2, 1, 1)
    try:
        legacy = qd.qgemv(fmt, Wd, xd).cpu().numpy()
    finally:
        qd.set_launch_override(0, 0, 0)
    assert_bound(f"legacy {fmt}", legacy, y64, S)


@pytest.mark.parametrize("fmt,N,K", [("q4_k", 300, 2048), ("q8_0", 40, 2560), ("q6_k", 48, 1024)])
@pytest.mark.parametrize("batch,act,norm", [(1, "gelu_tanh", True), (2, "silu", True),
                                            (1, "silu", False)])
@pytest.mark.parametrize("consumers,producers", [(4, 1), (4, 2), (8, 2), (8, 4)])
def test_stream_gate_up(qd, fmt, N, K, batch, act, norm, consumers, producers):
    assert streams(fmt, N, K)
    say(f"stream gate/up {fmt} N={N} K={K} batch={batch} act={act} norm={norm} consumers={consumers}")
    Wg = synth.quant_weights(fmt, N, K, SEED, tensor_id=83)
    Wu = synth.quant_weights(fmt, N, K, SEED, tensor_id=84)
    x = synth.normal((batch, K), SEED, tensor_id=85)
    nw = synth.normal((K,), SEED, tensor_id=86, mean=1.0, std=0.1)
    g = torch.empty((batch, N), device="cuda")
    u = torch.empty((batch, N), device="cuda")
    h = forced(qd, 1, lambda: qd.qffn_gate_up_act(fmt, dev(Wg), dev(Wu), dev(x),
                                                   dev(nw) if norm else None, 1e-6, act,
                                                   g_out=g, u_out=u).cpu().numpy(), consumers, 0,
               producers)
    g, u = g.cpu().numpy(), u.cpu().numpy()
    xn = (oracle.rmsnorm(x, nw, 1e-6) if norm else x.astype(np.float64)).astype(np.float32)
    g64, Sg = oracle.gemv(fmt, Wg, xn, N, K)
    u64, Su = oracle.gemv(fmt, Wu, xn, N, K)
    assert_bound("gate", g, g64, Sg)
    assert_bound("up", u, u64, Su)
    aid = oracle.ACT_GELU_TANH if act == "gelu_tanh" else oracle.ACT_SILU
    href = oracle.act_vec(aid, g64) * u64
    tol = h_tolerance(g64, u64, Sg, Su, aid)
    err = np.abs(h - href)
    assert (err <= tol).all(), f"h: worst {np.max(err / tol):.3f} of tolerance"


# Gemma-3 down (Q6_K 2560 x 10240) and gate/up (Q4_K 10240 x 2560): at two
# workgroups per CU a workgroup's steps outnumber the ring slots.
@pytest.mark.parametrize("consumers", [4, 8])
@pytest.mark.parametrize("depth", [0, 1])
@pytest.mark.parametrize("producers", [1, 2, 4])
def test_stream_ring_reuse_down(qd, consumers, depth, producers):
    fmt, N, K = "q6_k", 2560, 10240
    say(f"stream ring reuse {fmt} N={N} K={K} consumers={consumers} depth={depth}")
    W = synth.quant_weights(fmt, N, K, SEED, tensor_id=87)
    x = synth.normal((1, K), SEED, tensor_id=88)
    y64, S = oracle.gemv(fmt, W, x, N, K)
    Wd, xd = dev(W), dev(x)
    for wpc in (1, 2):
        y = forced(qd, wpc, lambda: qd.qgemv(fmt, Wd, xd).cpu().numpy(), consumers, depth, producers)
        assert_bound(f"down wpc={wpc}", y, y64, S)


@pytest.mark.parametrize("consumers", [4, 8])
@pytest.mark.parametrize("depth", [0, 1])
@pytest.mark.parametrize("producers", [1, 2, 4])
def test_stream_ring_reuse_gate_up(qd, consumers, depth, producers):
    fmt, N, K = "q4_k", 10240, 2560
    say(f"stream ring reuse gate/up {fmt} N={N} K={K} consumers={consumers} depth={depth}")
    Wg = synth.quant_weights(fmt, N, K, SEED, tensor_id=89)
    Wu = synth.quant_weights(fmt, N, K, SEED, tensor_id=90)
    x = synth.normal((1, K), SEED, tensor_id=91)
    nw = synth.normal((K,), SEED, tensor_id=92, mean=1.0, std=0.1)
    xn = oracle.rmsnorm(x, nw, 1e-6).astype(np.float32)
    g64, Sg = oracle.gemv(fmt, Wg, xn, N, K)
    u64, Su = oracle.gemv(fmt, Wu, xn, N, K)
    aid = oracle.ACT_GELU_TANH
    href = oracle.act_vec(aid, g64) * u64
    tol = h_tolerance(g64, u64, Sg, Su, aid)
    for wpc in (1, 2):
        g = torch.empty((1, N), device="cuda")
        u = torch.empty((1, N), device="cuda")
        h = forced(qd, wpc, lambda: qd.qffn_gate_up_act(fmt, dev(Wg), dev(Wu), dev(x), dev(nw), 1e-6,
                                                       "gelu_tanh", g_out=g, u_out=u).cpu().numpy(),
                   consumers, depth, producers)
        assert_bound(f"gate wpc={wpc}", g.cpu().numpy(), g64, Sg)
        assert_bound(f"up wpc={wpc}", u.cpu().numpy(), u64, Su)
        err = np.abs(h - href)
        assert (err <= tol).all(), f"h wpc={wpc}: worst {np.max(err / tol):.3f} of tolerance"


# Batch 2 over long rows and few of them (the Gemma-3 down shape, 2560 rows
# of K = 10240) runs on the register kernel with four K-slices across
# workgroups, the automatic choice there; 4096 rows stay on the streaming
# kernel.  Every output row is checked.
@pytest.mark.parametrize("fmt", ["q4_k", "q6_k", "q8_0"])
@pytest.mark.parametrize("N", [2560, 4096])
def test_long_rows_batch2_automatic(qd, fmt, N):
    K, batch = 10240, 2
    say(f"automatic gemv {fmt} N={N} K={K} batch={batch}")
    W = synth.quant_weights(fmt, N, K, SEED, tensor_id=83)
    x = synth.normal((batch, K), SEED, tensor_id=84)
    Wd, xd = dev(W), dev(x)
    y64, S = oracle.gemv(fmt, W, x, N, K)
    y = qd.qgemv(fmt, Wd, xd).cpu().numpy()
    assert_bound(f"automatic {fmt} N={N}", y, y64, S)
    again = qd.qgemv(fmt, Wd, xd).cpu().numpy()
    assert np.array_equal(y.view(np.uint32), again.view(np.uint32))


# The fused gate/up at batch 2 over rows of K >= 4096 runs on the register
# kernel (one lane group per row, two K-slices across workgroups), the
# automatic choice there; K = 2560 stays on the streaming kernel.
@pytest.mark.parametrize("fmt,N,K", [("q4_k", 1500, 5376), ("q4_k", 700, 4096), ("q6_k", 300, 4096),
                                     ("q8_0", 333, 4096), ("q4_k", 1024, 2560)])
def test_gate_up_batch2_automatic(qd, fmt, N, K):
    batch, act = 2, "gelu_tanh"
    say(f"automatic gate/up {fmt} N={N} K={K} batch={batch}")
    Wg = synth.quant_weights(fmt, N, K, SEED, tensor_id=88)
    Wu = synth.quant_weights(fmt, N, K, SEED, tensor_id=89)
    x = synth.normal((batch, K), SEED, tensor_id=90)
    nw = synth.normal((K,), SEED, tensor_id=91, mean=1.0, std=0.1)
    g = torch.empty((batch, N), device="cuda")
    u = torch.empty((batch, N), device="cuda")
    h = qd.qffn_gate_up_act(fmt, dev(Wg), dev(Wu), dev(x), dev(nw), 1e-6, act,
                            g_out=g, u_out=u).cpu().numpy()
    g, u = g.cpu().numpy(), u.cpu().numpy()
    xn = oracle.rmsnorm(x, nw, 1e-6).astype(np.float32)
    g64, Sg = oracle.gemv(fmt, Wg, xn, N, K)
    u64, Su = oracle.gemv(fmt, Wu, xn, N, K)
    assert_bound("gate", g, g64, Sg)
    assert_bound("up", u, u64, Su)
    href = oracle.act_vec(oracle.ACT_GELU_TANH, g64) * u64
    tol = h_tolerance(g64, u64, Sg, Su, oracle.ACT_GELU_TANH)
    err = np.abs(h - href)
    assert (err <= tol).all(), f"h: worst {np.max(err / tol):.3f} of tolerance"
