"""GPU parity of the residual-add epilogues (qgemv_residual,
qffn_decode_residual) against the oracle.

y must equal W x + r within the GEMV bound 1e-4 * sum|w x| + 1e-6 plus one
fp32 rounding of the sum (2^-24 |y|, taken as 2^-23 |y_ref| for slack), with
W x from the oracle in fp64 and r added in fp64.  Each case runs out of place
and in place (y = r), through every kernel that can write the output: the
register GEMV with and without a split across workgroups, the LDS-streaming
GEMV (K >= 8192), and the decode FFN's two-launch, grid-barrier and
single-launch forms.
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
    yield qd
    qd.set_launch_override(0, 0, 0)


from helpers import dev, h_tolerance, say  # noqa: E402


def assert_residual(name, got, y64, S, r):
    ref = y64 + r.astype(np.float64)
    err = np.abs(np.asarray(got, np.float64) - ref)
    bound = 1e-4 * S + 1e-6 + 2.0 ** -23 * np.abs(ref)
    bad = err > bound
    assert not bad.any(), f"{name}: {bad.sum()} outputs out of bound, worst {np.max(err / bound):.3f}"


@pytest.mark.parametrize("fmt,N,K,batch,shape", [
    ("q4_k", 2560, 2048, 1, None),        # O projection shape (register GEMV)
    ("q6_k", 2560, 10240, 1, None),       # down shape (LDS-streaming GEMV)
    ("q8_0", 37, 512, 3, None),           # ragged rows, batch 3
    ("q4_k", 300, 2560, 8, (2, 2, 1)),    # split across two workgroups
    ("q6_k", 130, 2048, 2, (4, 3, 1)),    # split across three workgroups
])
@pytest.mark.parametrize("inplace", [False, True])
def test_gemv_residual(qd, fmt, N, K, batch, shape, inplace):
    W = synth.quant_weights(fmt, N, K, SEED, tensor_id=81)
    x = synth.normal((batch, K), SEED, tensor_id=82)
    r = synth.normal((batch, N), SEED, tensor_id=83)
    say(f"gemv_residual {fmt} {N}x{K} batch={batch} shape={shape} inplace={inplace}")
    if shape:
        qd.set_launch_override(*shape)
    try:
        rd = dev(r)
        y = qd.qgemv_residual(fmt, dev(W), dev(x), rd, y=rd if inplace else None)
        got = y.cpu().numpy()
    finally:
        qd.set_launch_override(0, 0, 0)
    y64, S = oracle.gemv(fmt, W, x, N, K)
    assert_residual(f"{fmt} residual", got, y64, S, r)


@pytest.mark.parametrize("inplace", [False, True])
def test_ffn_decode_residual(qd, inplace):
    hidden, ff, batch = 2560, 10240, 1
    Wg = synth.quant_weights("q4_k", ff, hidden, SEED, tensor_id=84)
    Wu = synth.quant_weights("q4_k", ff, hidden, SEED, tensor_id=85)
    Wd = synth.quant_weights("q6_k", hidden, ff, SEED, tensor_id=86)
    x = synth.normal((batch, hidden), SEED, tensor_id=87)
    nw = synth.normal((hidden,), SEED, tensor_id=88, mean=1.0, std=0.1)
    r = synth.normal((batch, hidden), SEED, tensor_id=89)
    say(f"ffn_decode_residual gemma3 inplace={inplace}")
    h = torch.empty((batch, ff), device="cuda")
    rd = dev(r)
    y = qd.qffn_decode_residual("q4_k", dev(Wg), dev(Wu), "q6_k", dev(Wd), dev(x), rd, dev(nw), 1e-6,
                                "gelu_tanh", y=rd if inplace else None, h_out=h)
    got, hh = y.cpu().numpy(), h.cpu().numpy()
    xn32 = oracle.rmsnorm(x, nw, 1e-6).astype(np.float32)
    g64, Sg = oracle.gemv("q4_k", Wg, xn32, ff, hidden)
    u64, Su = oracle.gemv("q4_k", Wu, xn32, ff, hidden)
    href = oracle.act_vec(oracle.ACT_GELU_TANH, g64) * u64
    tol = h_tolerance(g64, u64, Sg, Su, oracle.ACT_GELU_TANH)
    assert (np.abs(hh - href) <= tol).all(), "h out of tolerance"
    y64, Sy = oracle.gemv("q6_k", Wd, hh, hidden, ff)
    assert_residual("ffn residual", got, y64, Sy, r)
