"""GPU parity for batches above 8 columns: every column of the GEMV, the
fused gate/up, the decode FFN (one matrix-core launch per projection over
groups of 8 batch rows, a ragged last group at 9, 17 and 23 columns, the
64-column limit) and the fused Q/K/V projection (successive launches of up
to 8 columns) against the oracle.  The bar is the oracle bound for every
column.  The decode FFN's down projection reads h as the digits the gate/up
launch wrote: its output must not depend on whether h is also kept.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

SEED = 0x5EED


@pytest.fixture(scope="module")
def qd(gpu):
    import quantized_decode_q4k_amd as qd
    qd.lib()
    return qd


from helpers import assert_bound, dev, h_tolerance, say  # noqa: E402


@pytest.mark.parametrize("fmt,N,K", [("q4_k", 300, 2560), ("q6_k", 130, 10240), ("q8_0", 77, 1024)])
@pytest.mark.parametrize("batch", [9, 23, 64])
def test_gemv_large_batch(qd, fmt, N, K, batch):
    W = synth.quant_weights(fmt, N, K, SEED, tensor_id=111)
    x = synth.normal((batch, K), SEED, tensor_id=112)
    say(f"gemv {fmt} {N}x{K} batch={batch}")
    y = torch.full((batch, N), float("nan"), device="cuda")
    qd.qgemv(fmt, dev(W), dev(x), y)
    y64, S = oracle.gemv(fmt, W, x, N, K)
    assert_bound(f"{fmt} b{batch}", y.cpu().numpy(), y64, S)


@pytest.mark.parametrize("batch", [9, 17])
def test_gate_up_and_ffn_decode_large_batch(qd, batch):
    hidden, ff = 512, 1280
    Wg = synth.quant_weights("q4_k", ff, hidden, SEED, tensor_id=113)
    Wu = synth.quant_weights("q4_k", ff, hidden, SEED, tensor_id=114)
    Wd = synth.quant_weights("q6_k", hidden, ff, SEED, tensor_id=115)
    x = synth.normal((batch, hidden), SEED, tensor_id=116)
    nw = synth.normal((hidden,), SEED, tensor_id=117, mean=1.0, std=0.1)
    r = synth.normal((batch, hidden), SEED, tensor_id=118)
    say(f"ffn decode batch={batch}")
    h = torch.full((batch, ff), float("nan"), device="cuda")
    y = qd.qffn_decode_residual("q4_k", dev(Wg), dev(Wu), "q6_k", dev(Wd), dev(x), dev(r), dev(nw), 1e-6,
                                "silu", h_out=h)
    h, y = h.cpu().numpy(), y.cpu().numpy()
    xn32 = oracle.rmsnorm(x, nw, 1e-6).astype(np.float32)
    g64, Sg = oracle.gemv("q4_k", Wg, xn32, ff, hidden)
    u64, Su = oracle.gemv("q4_k", Wu, xn32, ff, hidden)
    href = oracle.act_vec(oracle.ACT_SILU, g64) * u64
    tol = h_tolerance(g64, u64, Sg, Su, oracle.ACT_SILU)
    assert (np.abs(h - href) <= tol).all(), "h out of tolerance"
    y64, Sy = oracle.gemv("q6_k", Wd, h, hidden, ff)
    ref = y64 + r
    err = np.abs(y - ref)
    assert (err <= 1e-4 * Sy + 1e-6 + 2.0 ** -23 * np.abs(ref)).all(), "y out of bound"
    # the fused gate/up alone, at the same batch
    g = torch.empty((batch, ff), device="cuda")
    hh = qd.qffn_gate_up_act("q4_k", dev(Wg), dev(Wu), dev(x), dev(nw), 1e-6, "silu", g_out=g)
    assert_bound("gate b%d" % batch, g.cpu().numpy(), g64, Sg)
    assert np.array_equal(hh.cpu().numpy().view(np.uint32), h.view(np.uint32))


@pytest.mark.parametrize("batch", [3, 8, 19])
def test_ffn_decode_h_kept_or_not(qd, batch):
    hidden, ff = 768, 2048
    Wg = synth.quant_weights("q4_k", ff, hidden, SEED, tensor_id=130)
    Wu = synth.quant_weights("q4_k", ff, hidden, SEED, tensor_id=131)
    Wd = synth.quant_weights("q6_k", hidden, ff, SEED, tensor_id=132)
    x = synth.normal((batch, hidden), SEED, tensor_id=133)
    nw = synth.normal((hidden,), SEED, tensor_id=134, mean=1.0, std=0.1)
    say(f"ffn decode h kept or not batch={batch}")
    h = torch.full((batch, ff), float("nan"), device="cuda")
    y1 = qd.qffn_decode("q4_k", dev(Wg), dev(Wu), "q6_k", dev(Wd), dev(x), dev(nw), 1e-6, "gelu_tanh", h_out=h)
    y2 = qd.qffn_decode("q4_k", dev(Wg), dev(Wu), "q6_k", dev(Wd), dev(x), dev(nw), 1e-6, "gelu_tanh")
    y1, y2, h = y1.cpu().numpy(), y2.cpu().numpy(), h.cpu().numpy()
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    y64, Sy = oracle.gemv("q6_k", Wd, h, hidden, ff)
    assert_bound(f"down b{batch}", y1, y64, Sy)


def test_qkv_large_batch(qd):
    fm, Ns, K, batch = ("q4_k", "q4_k", "q6_k"), (96, 32, 32), 2560, 11
    Ws = [synth.quant_weights(f, n, K, SEED, tensor_id=120 + i) for i, (f, n) in enumerate(zip(fm, Ns))]
    x = synth.normal((batch, K), SEED, tensor_id=123)
    nw = synth.normal((K,), SEED, tensor_id=124, mean=1.0, std=0.1)
    say(f"qkv batch={batch}")
    outs = qd.qqkv_proj(fm, *[dev(W) for W in Ws], dev(x), dev(nw))
    xn32 = oracle.rmsnorm(x, nw, 1e-6).astype(np.float32)
    for name, f, n, W, o in zip("qkv", fm, Ns, Ws, outs):
        y64, S = oracle.gemv(f, W, xn32, n, K)
        assert_bound(f"qkv {name}", o.cpu().numpy(), y64, S)
