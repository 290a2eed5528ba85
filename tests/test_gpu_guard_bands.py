"""Out-of-bounds stores: every output is a window of a larger device buffer
whose 4 KB margins on both sides, and the window itself, start filled with a
sentinel NaN pattern.  After each call the margins must still hold the
sentinel bit for bit (no kernel wrote past its output) and the window must
hold none (every output element was written).  Each entry point runs through
the kernels its shapes select: register GEMV with and without split-K,
LDS-streaming GEMV and fused gate/up, the decode FFN's three forms, fused
Q/K/V, MoE, prefill GEMMs, the dequantisers, and the int8-activation
quantizer and GEMV.
"""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

SEED = 0x5EED
GUARD = 1024                 # elements per margin (4 KB of fp32)
SENT32 = 0x7FBADBAD          # a quiet NaN no kernel computes
SENT16 = 0x7FBD              # bf16 NaN pattern


@pytest.fixture(scope="module")
def qd(gpu):
    import quantized_decode_q4k_amd as qd
    qd.lib()
    yield qd
    qd.set_launch_override(0, 0, 0)


from helpers import dev, say  # noqa: E402


class Guarded:
    """A device buffer [GUARD | window | GUARD] filled with the sentinel."""

    def __init__(self, shape, bf16=False):
        self.n = int(np.prod(shape))
        self.bf16 = bf16
        if bf16:
            self.buf = torch.full((2 * GUARD + self.n,), SENT16, dtype=torch.int16, device="cuda")
        else:
            bits = torch.full((2 * GUARD + self.n,), SENT32, dtype=torch.int32, device="cuda")
            self.buf = bits.view(torch.float32)
        self.view = self.buf[GUARD:GUARD + self.n].view(shape)

    def check(self, name):
        torch.cuda.synchronize()
        raw = self.buf.cpu().numpy().view(np.uint16 if self.bf16 else np.uint32)
        sent = SENT16 if self.bf16 else SENT32
        lo, win, hi = raw[:GUARD], raw[GUARD:GUARD + self.n], raw[GUARD + self.n:]
        assert (lo == sent).all(), f"{name}: {np.count_nonzero(lo != sent)} stores below the output"
        assert (hi == sent).all(), f"{name}: {np.count_nonzero(hi != sent)} stores above the output"
        assert not (win == sent).any(), f"{name}: {np.count_nonzero(win == sent)} outputs never written"


@pytest.mark.parametrize("fmt,N,K,batch,shape", [
    ("q4_k", 300, 2560, 1, None),        # register GEMV
    ("q6_k", 2560, 10240, 1, None),      # LDS-streaming GEMV
    ("q6_k", 257, 2048, 2, None),        # streaming, batch 2, uneven rows
    ("q8_0", 77, 1024, 3, None),         # register, batch 3
    ("q4_k", 300, 2560, 8, (2, 2, 1)),   # split across workgroups
    ("q4_k", 40, 512, 11, None),         # two launches of 8 + 3 columns
])
def test_gemv_guard_bands(qd, fmt, N, K, batch, shape):
    say(f"guard gemv {fmt} {N}x{K} batch={batch} shape={shape}")
    W = dev(synth.quant_weights(fmt, N, K, SEED, tensor_id=131))
    x = dev(synth.normal((batch, K), SEED, tensor_id=132))
    y = Guarded((batch, N))
    if shape:
        qd.set_launch_override(*shape)
    try:
        qd.qgemv(fmt, W, x, y.view)
    finally:
        qd.set_launch_override(0, 0, 0)
    y.check(f"qgemv {fmt}")
    # in-place residual add on a guarded y
    r = Guarded((batch, N))
    r.view.copy_(dev(synth.normal((batch, N), SEED, tensor_id=133)))
    qd.qgemv_residual(fmt, W, x, r.view, y=r.view)
    r.check(f"qgemv_residual {fmt}")


@pytest.mark.parametrize("fmt,N,K,batch", [("q4_k", 10240, 2560, 1), ("q8_0", 512, 2560, 2),
                                           ("q4_k", 96, 512, 9)])
def test_gate_up_guard_bands(qd, fmt, N, K, batch):
    say(f"guard gate/up {fmt} {N}x{K} batch={batch}")
    Wg = dev(synth.quant_weights(fmt, N, K, SEED, tensor_id=134))
    Wu = dev(synth.quant_weights(fmt, N, K, SEED, tensor_id=135))
    x = dev(synth.normal((batch, K), SEED, tensor_id=136))
    nw = dev(synth.normal((K,), SEED, tensor_id=137, mean=1.0, std=0.1))
    h, g, u = Guarded((batch, N)), Guarded((batch, N)), Guarded((batch, N))
    qd.qffn_gate_up_act(fmt, Wg, Wu, x, nw, 1e-6, "gelu_tanh", h=h.view, g_out=g.view, u_out=u.view)
    for t, name in ((h, "h"), (g, "g"), (u, "u")):
        t.check(f"qffn_gate_up_act {name}")


def test_ffn_decode_guard_bands(qd):
    hidden, ff = 2560, 10240
    say("guard ffn_decode")
    Wg = dev(synth.quant_weights("q4_k", ff, hidden, SEED, tensor_id=138))
    Wu = dev(synth.quant_weights("q4_k", ff, hidden, SEED, tensor_id=139))
    Wd = dev(synth.quant_weights("q6_k", hidden, ff, SEED, tensor_id=140))
    x = dev(synth.normal((1, hidden), SEED, tensor_id=141))
    nw = dev(synth.normal((hidden,), SEED, tensor_id=142, mean=1.0, std=0.1))
    y, h = Guarded((1, hidden)), Guarded((1, ff))
    qd.qffn_decode("q4_k", Wg, Wu, "q6_k", Wd, x, nw, 1e-6, "gelu_tanh", y=y.view, h_out=h.view)
    y.check("qffn_decode y")
    h.check("qffn_decode h")


@pytest.mark.parametrize("kernel", ["stream", "register"])
def test_qkv_and_moe_guard_bands(qd, kernel):
    """Batch 1 runs on the streaming kernel; a forced launch shape keeps the
    register kernel."""
    say(f"guard qkv and moe ({kernel} kernel)")
    if kernel == "register":
        qd.set_launch_override(4, 0, 0)
    try:
        _qkv_and_moe(qd)
    finally:
        qd.set_launch_override(0, 0, 0)


def _qkv_and_moe(qd):
    fm, Ns, K = ("q4_k", "q4_k", "q6_k"), (2048, 1024, 1024), 2560
    Ws = [dev(synth.quant_weights(f, n, K, SEED, tensor_id=143 + i)) for i, (f, n) in enumerate(zip(fm, Ns))]
    x = dev(synth.normal((1, K), SEED, tensor_id=146))
    nw = dev(synth.normal((K,), SEED, tensor_id=147, mean=1.0, std=0.1))
    outs = [Guarded((1, n)) for n in Ns]
    qd.qqkv_proj(fm, *Ws, x, nw, 1e-6, q=outs[0].view, k=outs[1].view, v=outs[2].view)
    for o, name in zip(outs, "qkv"):
        o.check(f"qqkv_proj {name}")
    E, ff = 6, 512
    Wg = dev(synth.quant_weights("q4_k", E * ff, K, SEED, tensor_id=148))
    Wu = dev(synth.quant_weights("q4_k", E * ff, K, SEED, tensor_id=149))
    Wd = dev(synth.quant_weights("q6_k", E * K, ff, SEED, tensor_id=150))
    ids = torch.tensor([4, 1, -3, 5], dtype=torch.int32, device="cuda")
    coef = torch.tensor([0.4, 0.3, 0.2, 0.1], dtype=torch.float32, device="cuda")
    y, h = Guarded((K,)), Guarded((4, ff))
    qd.qmoe_ffn_decode("q4_k", Wg, Wu, "q6_k", Wd, E, ids, coef, x[0], nw, 1e-6, "silu", y=y.view, h_out=h.view)
    y.check("qmoe_ffn_decode y")
    h.check("qmoe_ffn_decode h")


@pytest.mark.parametrize("fmt,M,N,K", [("q4_k", 130, 300, 768), ("q6_k", 77, 513, 512), ("q8_0", 33, 257, 96)])
def test_prefill_and_dequant_guard_bands(qd, fmt, M, N, K):
    say(f"guard prefill/dequant {fmt} M={M} N={N} K={K}")
    W = dev(synth.quant_weights(fmt, N, K, SEED, tensor_id=151))
    Wu = dev(synth.quant_weights(fmt, N, K, SEED, tensor_id=152))
    X = torch.from_numpy(synth.normal_bf16((M, K), SEED, tensor_id=153).view(np.int16)).cuda()
    Y = Guarded((M, N))
    qd.qgemm_prefill(fmt, W, X, Y=Y.view)
    Y.check(f"qgemm_prefill {fmt}")
    H, g, u = Guarded((M, N), bf16=True), Guarded((M, N)), Guarded((M, N))
    qd.qgemm_prefill_gate_up_act(fmt, W, Wu, X, "gelu_tanh", H=H.view.view(torch.bfloat16), g_out=g.view,
                                 u_out=u.view)
    for t, name in ((H, "H"), (g, "g"), (u, "u")):
        t.check(f"qgemm_prefill_gate_up_act {name} {fmt}")
    D, Db = Guarded((N, K)), Guarded((N, K), bf16=True)
    qd.qdequant(fmt, W, K, out=D.view)
    qd.qdequant_bf16(fmt, W, K, out=Db.view)
    D.check(f"qdequant {fmt}")
    Db.check(f"qdequant_bf16 {fmt}")


@pytest.mark.parametrize("N,K,batch", [(300, 2560, 1), (77, 96, 3), (40, 16384, 5), (64, 512, 11)])
def test_int8_activation_guard_bands(qd, N, K, batch):
    say(f"guard int8 activations {N}x{K} batch={batch}")
    W = dev(synth.quant_weights("q8_0", N, K, SEED, tensor_id=154))
    x = dev(synth.normal((batch, K), SEED, tensor_id=155))
    y = Guarded((batch, N))
    qd.qgemv_q8_0_q8act(W, x, y.view)
    y.check("qgemv_q8_0_q8act")
    # codes: an int8 buffer seen as bytes inside a guarded fp32 buffer
    qb, d = Guarded(((batch * K) // 4,)), Guarded((batch, K // 32))
    qd.qquantize_q8_act(x, q=qb.view.view(torch.int8).view(batch, K), d=d.view)
    d.check("qquantize_q8_act d")
    raw = qb.buf.cpu().numpy().view(np.uint32)
    assert (raw[:GUARD] == SENT32).all() and (raw[GUARD + qb.n:] == SENT32).all(), "codes written outside q"
    y2 = Guarded((batch, N))
    qd.qgemv_q8_0_preq(W, qb.view.view(torch.int8).view(batch, K), d.view, y2.view)
    y2.check("qgemv_q8_0_preq")
