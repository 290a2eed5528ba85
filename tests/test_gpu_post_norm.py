"""GPU parity of the post-norm, residual and next-norm epilogue (the
post_attn_residual_norm_store / post_ffn_norm_residual_add steps of the larql
Gemma 3 table) against the oracle.

    y  = r + RMSNorm(W x; post_w)       y2 = RMSNorm(y; next_w)

y is checked against the oracle's y computed from the exact projection, with
the GEMV bound carried through the norm (post_norm_bound); y2 is checked
stage by stage against the oracle's RMS-norm of the GPU's own y.  Shapes:
the Gemma-3-4B O projection (Q4_K 2560 x 2048, register GEMV) and down
projection (Q6_K 2560 x 10240, LDS-streaming GEMV), batches 1-12 (chunked
above 8), split-K launch shapes, in place (y = r), the FFN form, and
repeated calls (the completion counter returns to zero).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import dev, h_tolerance, post_norm_bound, rmsnorm_eval_bound, say

pytestmark = pytest.mark.gpu

SEED = 0x5EED
EPS = 1e-6


@pytest.fixture(scope="module")
def qd(gpu):
    import quantized_decode_q4k_amd as qd
    qd.lib()
    yield qd
    qd.set_launch_override(0, 0, 0)


def check_post(name, y, y2, p64, S, r, w1, w2):
    yref, _ = oracle.post_norm_residual(p64, r, w1, EPS)
    bound = post_norm_bound(p64, S, r, w1, EPS, yref)
    y = np.atleast_2d(np.asarray(y, np.float64))
    err = np.abs(y - yref)
    assert (err <= bound).all(), f"{name} y: worst {np.max(err / bound):.3f} of the bound"
    if w2 is not None:
        y2ref = oracle.rmsnorm(y.astype(np.float32), w2, EPS)
        b2 = rmsnorm_eval_bound(y2ref)
        err2 = np.abs(np.atleast_2d(y2) - y2ref)
        assert (err2 <= b2).all(), f"{name} y2: worst {np.max(err2 / b2):.3f} of the bound"


CASES = [
    # fmt, N, K, batch, forced (p_in, p_out, nr) or None
    ("q4_k", 2560, 2048, 1, None),      # Gemma-3 O projection
    ("q6_k", 2560, 10240, 1, None),     # Gemma-3 down (streaming kernel)
    ("q6_k", 2560, 10240, 2, None),     # streaming kernel, two columns
    ("q4_k", 2560, 2048, 3, None),
    ("q8_0", 700, 1024, 8, None),
    ("q4_k", 300, 2560, 12, None),      # two launches of columns
    ("q4_k", 300, 2560, 2, (2, 3, 1)),  # split across three workgroups
    ("q6_k", 129, 2048, 1, (16, 4, 1)),
]


@pytest.mark.parametrize("fmt,N,K,batch,shape", CASES)
@pytest.mark.parametrize("inplace", [False, True])
@pytest.mark.parametrize("with_next", [False, True])
def test_gemv_post_norm(qd, fmt, N, K, batch, shape, inplace, with_next):
    say(f"post-norm gemv {fmt} {N}x{K} batch={batch} shape={shape} inplace={inplace} next={with_next}")
    W = synth.quant_weights(fmt, N, K, SEED, tensor_id=211)
    x = synth.normal((batch, K), SEED, tensor_id=212)
    r = synth.normal((batch, N), SEED, tensor_id=213)
    w1 = synth.normal((N,), SEED, tensor_id=214, mean=1.0, std=0.1)
    w2 = synth.normal((N,), SEED, tensor_id=215, mean=1.0, std=0.1) if with_next else None
    if shape:
        qd.set_launch_override(*shape)
    try:
        rd = dev(r)
        Wd, xd, w1d = dev(W), dev(x), dev(w1)
        outs = []
        for rep in range(2):
            rr = rd.clone() if inplace else rd
            out = qd.qgemv_post_norm_residual(fmt, Wd, xd, w1d, rr, EPS, y=rr if inplace else None,
                                              next_w=dev(w2) if with_next else None)
            y, y2 = out if with_next else (out, None)
            outs.append((y.cpu().numpy(), None if y2 is None else y2.cpu().numpy()))
    finally:
        qd.set_launch_override(0, 0, 0)
    p64, S = oracle.gemv_threaded(fmt, W, x, N, K, oracle.host_threads())
    check_post(f"{fmt} {N}x{K} b{batch}", outs[0][0], outs[0][1], p64, S, r, w1, w2)
    assert np.array_equal(outs[0][0].view(np.uint32), outs[1][0].view(np.uint32)), "not deterministic"
    if with_next:
        assert np.array_equal(outs[0][1].view(np.uint32), outs[1][1].view(np.uint32))


@pytest.mark.parametrize("batch", [1, 3])
def test_ffn_decode_post_norm(qd, batch):
    """The Gemma-3 FFN with the post-FFN norm and residual on its down
    projection: h against the oracle, y on the GPU's own h, y2 on the GPU's
    own y."""
    hidden, ff = 2560, 10240
    say(f"post-norm ffn gemma3 batch={batch}")
    Wg = synth.quant_weights("q4_k", ff, hidden, SEED, tensor_id=216)
    Wu = synth.quant_weights("q4_k", ff, hidden, SEED, tensor_id=217)
    Wd = synth.quant_weights("q6_k", hidden, ff, SEED, tensor_id=218)
    x = synth.normal((batch, hidden), SEED, tensor_id=219)
    r = synth.normal((batch, hidden), SEED, tensor_id=220)
    w1 = synth.normal((hidden,), SEED, tensor_id=221, mean=1.0, std=0.1)
    w2 = synth.normal((hidden,), SEED, tensor_id=222, mean=1.0, std=0.1)
    h = torch.empty((batch, ff), device="cuda")
    rd = dev(r)
    y, y2 = qd.qffn_decode_post_norm_residual("q4_k", dev(Wg), dev(Wu), "q6_k", dev(Wd), dev(x), dev(w1), rd,
                                              None, EPS, "gelu_tanh", y=rd, next_w=dev(w2), h_out=h)
    hh, y, y2 = h.cpu().numpy(), y.cpu().numpy(), y2.cpu().numpy()
    th = oracle.host_threads()
    g64, Sg = oracle.gemv_threaded("q4_k", Wg, x, ff, hidden, th)
    u64, Su = oracle.gemv_threaded("q4_k", Wu, x, ff, hidden, th)
    href = oracle.act_vec(oracle.ACT_GELU_TANH, g64) * u64
    tol = h_tolerance(g64, u64, Sg, Su, oracle.ACT_GELU_TANH)
    assert (np.abs(hh - href) <= tol).all(), "h out of tolerance"
    p64, S = oracle.gemv_threaded("q6_k", Wd, hh, hidden, ff, th)
    check_post("ffn", y, y2, p64, S, r, w1, w2)


def test_post_norm_zero_projection_keeps_residual(qd):
    """x = 0: the projection is zero, its norm is zero (eps > 0), so y = r
    bit for bit and y2 = RMSNorm(r)."""
    N, K = 2560, 2048
    say("post-norm zero projection")
    W = synth.quant_weights("q4_k", N, K, SEED, tensor_id=223)
    r = synth.normal((1, N), SEED, tensor_id=224)
    w1 = synth.normal((N,), SEED, tensor_id=225, mean=1.0, std=0.1)
    w2 = synth.normal((N,), SEED, tensor_id=226, mean=1.0, std=0.1)
    y, y2 = qd.qgemv_post_norm_residual("q4_k", dev(W), dev(np.zeros((1, K), np.float32)), dev(w1), dev(r),
                                        EPS, next_w=dev(w2))
    assert np.array_equal(y.cpu().numpy().view(np.uint32), r.view(np.uint32))
    y2ref = oracle.rmsnorm(r, w2, EPS)
    assert (np.abs(y2.cpu().numpy() - y2ref) <= rmsnorm_eval_bound(y2ref)).all()
