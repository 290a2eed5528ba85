"""The allocation-free decode FFN (qffn_decode_noalloc) through the C ABI,
against the entry point it mirrors (qffn_decode, which keeps h and partial
sums in the stream's workspace) and against the oracle.

Two calls in a row on one stream, the second with a smaller input (the
scratch keeps the first call's contents; the second must not see them),
then the reverse order; a split-K shape (batch 8, partial sums in the
scratch); a call beyond the scratch's size (QD_ETOOBIG, nothing enqueued);
and the call captured in a graph on a fresh stream (no workspace exists
there, so qffn_decode would return QD_ECAPTURE) and replayed.
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
    return qd


class Ffn:
    def __init__(self, hidden, ff, batch, tid, fd="q6_k"):
        self.hidden, self.ff, self.batch, self.fd = hidden, ff, batch, fd
        self.Wg = synth.quant_weights("q4_k", ff, hidden, SEED, tensor_id=tid)
        self.Wu = synth.quant_weights("q4_k", ff, hidden, SEED, tensor_id=tid + 1)
        self.Wd = synth.quant_weights(fd, hidden, ff, SEED, tensor_id=tid + 2)
        self.x = synth.normal((batch, hidden), SEED, tensor_id=tid + 3)
        self.nw = synth.normal((hidden,), SEED, tensor_id=tid + 4, mean=1.0, std=0.1)
        self.d = [dev(a) for a in (self.Wg, self.Wu, self.Wd, self.x, self.nw)]

    def run(self, qd, noalloc, h_out=None):
        Wg, Wu, Wd, x, nw = self.d
        y = torch.empty((self.batch, self.hidden), device="cuda")
        if noalloc:
            qd.qffn_decode_noalloc("q4_k", Wg, Wu, self.fd, Wd, x, nw, 1e-6, "gelu_tanh", y, h_out=h_out)
        else:
            qd.qffn_decode("q4_k", Wg, Wu, self.fd, Wd, x, nw, 1e-6, "gelu_tanh", y=y, h_out=h_out)
        return y

    def check_oracle(self, qd):
        """h and y of the allocation-free call against the oracle (y on the
        GPU's own h)."""
        h = torch.empty((self.batch, self.ff), device="cuda")
        y = self.run(qd, True, h_out=h).cpu().numpy()
        hh = h.cpu().numpy()
        th = oracle.host_threads()
        xn = oracle.rmsnorm(self.x, self.nw, 1e-6).astype(np.float32)
        g64, Sg = oracle.gemv_threaded("q4_k", self.Wg, xn, self.ff, self.hidden, th)
        u64, Su = oracle.gemv_threaded("q4_k", self.Wu, xn, self.ff, self.hidden, th)
        href = oracle.act_vec(oracle.ACT_GELU_TANH, g64) * u64
        tol = h_tolerance(g64, u64, Sg, Su, oracle.ACT_GELU_TANH)
        assert (np.abs(hh - href) <= tol).all(), "h out of tolerance"
        y64, Sy = oracle.gemv_threaded(self.fd, self.Wd, hh, self.hidden, self.ff, th)
        assert_bound("noalloc y", y, y64, Sy)


def same(a, b, what):
    assert np.array_equal(a.cpu().numpy().view(np.uint32), b.cpu().numpy().view(np.uint32)), what


def test_noalloc_matches_workspace_entry_two_calls(qd):
    big = Ffn(2560, 10240, 1, 231)           # Gemma-3-4B FFN, LDS-streaming kernels, h in the scratch
    small = Ffn(512, 1024, 8, 236, "q4_k")   # register kernels, batch 8
    for order in ((big, small), (small, big)):
        for f in order:
            say(f"noalloc ffn hidden={f.hidden} ff={f.ff} batch={f.batch}")
            a = f.run(qd, True)
            b = f.run(qd, False)
            same(a, b, f"hidden={f.hidden}: noalloc differs from qffn_decode")
    big.check_oracle(qd)
    small.check_oracle(qd)


def test_noalloc_split_k_partials_in_scratch(qd):
    """Gemma-4-31B shape at batch 8: the register kernels split K across
    workgroups (partial sums and tile counters in the scratch), then a
    smaller call."""
    f = Ffn(5376, 21504, 8, 241)
    g = Ffn(512, 1536, 3, 246)
    for ff in (f, g, f):
        say(f"noalloc split-K hidden={ff.hidden} ff={ff.ff} batch={ff.batch}")
        same(ff.run(qd, True), ff.run(qd, False), f"hidden={ff.hidden}: noalloc differs from qffn_decode")
    g.check_oracle(qd)


def test_noalloc_rejects_calls_beyond_the_scratch(qd):
    """A call whose h and partial sums exceed the scratch returns QD_ETOOBIG
    and enqueues nothing (the weights are never read)."""
    hidden, ff, batch = 2560, 131072, 8
    say("noalloc too big")
    Wg = torch.empty(ff * synth.row_bytes("q4_k", hidden), dtype=torch.uint8, device="cuda")
    Wu = torch.empty_like(Wg)
    Wd = torch.empty(hidden * synth.row_bytes("q6_k", ff), dtype=torch.uint8, device="cuda")
    x = torch.zeros((batch, hidden), device="cuda")
    y = torch.full((batch, hidden), 7.0, device="cuda")
    with pytest.raises(qd.QDError) as e:
        qd.qffn_decode_noalloc("q4_k", Wg, Wu, "q6_k", Wd, x, None, 1e-6, "gelu_tanh", y)
    assert e.value.status == qd.QD_ETOOBIG
    torch.cuda.synchronize()
    assert bool((y == 7.0).all()), "a rejected call wrote its output"


def test_noalloc_captured_on_a_fresh_stream(qd):
    """On a stream with no workspace the allocation-free call can be
    captured; every replay reproduces the eager result."""
    f = Ffn(512, 1024, 2, 251)
    Wg, Wu, Wd, x, nw = f.d
    ref = f.run(qd, False)
    torch.cuda.synchronize()
    y = torch.empty_like(ref)
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            qd.qffn_decode_noalloc("q4_k", Wg, Wu, "q6_k", Wd, x, nw, 1e-6, "gelu_tanh", y)
        for rep in range(3):
            y.fill_(float("nan"))
            f.run(qd, True)                   # the scratch rewritten between replays
            g.replay()
            s.synchronize()
            same(y, ref, f"replay {rep}")
