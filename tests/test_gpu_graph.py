"""Calls captured in a HIP graph and replayed: every replay must reproduce the
eager result bit for bit (the kernels sum in a fixed order).  Between
replays the outputs are refilled with NaN by a fill kernel and the same entry
point runs eagerly on other inputs, so the workspace's partial sums and
counters are rewritten in between; a replay that depended on stale workspace
state, or on a counter left non-zero, would differ.  Each case makes one
uncaptured call first, so the workspace has its final size before capture.
Cases: the decode FFN (LDS-streaming kernels, h in the workspace), a split-K
GEMV, the fused Q/K/V projection, the MoE FFN (split-K over slots), a
split-K prefill GEMM, and the int8-activation GEMV (codes in the workspace).
"""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

SEED = 0x5EED


@pytest.fixture(scope="module")
def qd(gpu):
    import quantized_decode_q4k_amd as qd
    qd.lib()
    yield qd
    qd.set_launch_override(0, 0, 0)
    qd.set_gemm_override(0, 0)


from helpers import dev, say  # noqa: E402


def check_replays(name, run, outs, perturb, replays=3):
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        run()
        s.synchronize()
        ref = [o.clone() for o in outs]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            run()
        for rep in range(replays):
            for o in outs:
                o.fill_(float("nan"))
            perturb()
            g.replay()
            s.synchronize()
            for i, (o, r) in enumerate(zip(outs, ref)):
                a = o.cpu().numpy().view(np.uint32 if o.dtype == torch.float32 else np.uint16)
                b = r.cpu().numpy().view(np.uint32 if r.dtype == torch.float32 else np.uint16)
                assert np.array_equal(a, b), f"{name}: replay {rep} output {i} differs from the eager call"


def test_graph_ffn_decode(qd):
    hidden, ff = 2560, 10240
    say("graph ffn_decode gemma3")
    Wg = dev(synth.quant_weights("q4_k", ff, hidden, SEED, tensor_id=161))
    Wu = dev(synth.quant_weights("q4_k", ff, hidden, SEED, tensor_id=162))
    Wd = dev(synth.quant_weights("q6_k", hidden, ff, SEED, tensor_id=163))
    nw = dev(synth.normal((hidden,), SEED, tensor_id=164, mean=1.0, std=0.1))
    x, x2 = dev(synth.normal((1, hidden), SEED, tensor_id=165)), dev(synth.normal((1, hidden), SEED, tensor_id=166))
    y, y2 = torch.empty((1, hidden), device="cuda"), torch.empty((1, hidden), device="cuda")
    run = lambda: qd.qffn_decode("q4_k", Wg, Wu, "q6_k", Wd, x, nw, 1e-6, "gelu_tanh", y=y)
    perturb = lambda: qd.qffn_decode("q4_k", Wg, Wu, "q6_k", Wd, x2, nw, 1e-6, "gelu_tanh", y=y2)
    check_replays("qffn_decode", run, [y], perturb)


def test_graph_split_k_gemv_and_qkv(qd):
    say("graph split-K gemv and qkv")
    W = dev(synth.quant_weights("q4_k", 300, 2560, SEED, tensor_id=167))
    x, x2 = dev(synth.normal((8, 2560), SEED, tensor_id=168)), dev(synth.normal((8, 2560), SEED, tensor_id=169))
    y, y2 = torch.empty((8, 300), device="cuda"), torch.empty((8, 300), device="cuda")
    qd.set_launch_override(2, 3, 1)
    try:
        check_replays("split-K qgemv", lambda: qd.qgemv("q4_k", W, x, y), [y],
                      lambda: qd.qgemv("q4_k", W, x2, y2))
    finally:
        qd.set_launch_override(0, 0, 0)
    fm, Ns = ("q4_k", "q4_k", "q6_k"), (2048, 1024, 1024)
    Ws = [dev(synth.quant_weights(f, n, 2560, SEED, tensor_id=170 + i)) for i, (f, n) in enumerate(zip(fm, Ns))]
    nw = dev(synth.normal((2560,), SEED, tensor_id=173, mean=1.0, std=0.1))
    outs = [torch.empty((1, n), device="cuda") for n in Ns]
    outs2 = [torch.empty((1, n), device="cuda") for n in Ns]
    check_replays("qqkv_proj", lambda: qd.qqkv_proj(fm, *Ws, x[:1], nw, 1e-6, q=outs[0], k=outs[1], v=outs[2]),
                  outs, lambda: qd.qqkv_proj(fm, *Ws, x2[:1], nw, 1e-6, q=outs2[0], k=outs2[1], v=outs2[2]))


def test_graph_moe_and_prefill(qd):
    say("graph moe and split-K prefill")
    E, ff, hidden = 16, 1024, 2560
    Wg = dev(synth.quant_weights("q4_k", E * ff, hidden, SEED, tensor_id=174))
    Wu = dev(synth.quant_weights("q4_k", E * ff, hidden, SEED, tensor_id=175))
    Wd = dev(synth.quant_weights("q6_k", E * hidden, ff, SEED, tensor_id=176))
    x, x2 = dev(synth.normal((hidden,), SEED, tensor_id=177)), dev(synth.normal((hidden,), SEED, tensor_id=178))
    nw = dev(synth.normal((hidden,), SEED, tensor_id=179, mean=1.0, std=0.1))
    ids = torch.tensor([3, 9, 0, 15, 7, 3], dtype=torch.int32, device="cuda")
    ids2 = torch.tensor([1, 2, 4, 8, 10, 11], dtype=torch.int32, device="cuda")
    coef = torch.tensor([0.3, 0.2, 0.15, 0.15, 0.1, 0.1], dtype=torch.float32, device="cuda")
    y, y2 = torch.empty((hidden,), device="cuda"), torch.empty((hidden,), device="cuda")
    check_replays("qmoe_ffn_decode",
                  lambda: qd.qmoe_ffn_decode("q4_k", Wg, Wu, "q6_k", Wd, E, ids, coef, x, nw, 1e-6, "gelu_tanh", y=y),
                  [y], lambda: qd.qmoe_ffn_decode("q4_k", Wg, Wu, "q6_k", Wd, E, ids2, coef, x2, nw, 1e-6,
                                                  "gelu_tanh", y=y2))
    M, N, K = 64, 300, 2048
    W = dev(synth.quant_weights("q6_k", N, K, SEED, tensor_id=180))
    X = torch.from_numpy(synth.normal_bf16((M, K), SEED, tensor_id=181).view(np.int16)).cuda()
    X2 = torch.from_numpy(synth.normal_bf16((M, K), SEED, tensor_id=182).view(np.int16)).cuda()
    Y, Y2 = torch.empty((M, N), device="cuda"), torch.empty((M, N), device="cuda")
    qd.set_gemm_override(2, 3)
    try:
        check_replays("split-K qgemm_prefill", lambda: qd.qgemm_prefill("q6_k", W, X, Y=Y), [Y],
                      lambda: qd.qgemm_prefill("q6_k", W, X2, Y=Y2))
    finally:
        qd.set_gemm_override(0, 0)
    qd.set_gemm_streamk(5)
    try:
        check_replays("stream-K qgemm_prefill", lambda: qd.qgemm_prefill("q6_k", W, X, Y=Y), [Y],
                      lambda: qd.qgemm_prefill("q6_k", W, X2, Y=Y2))
    finally:
        qd.set_gemm_streamk(0)


def test_graph_int8_activations(qd):
    say("graph int8-activation gemv")
    N, K = 513, 2560
    W = dev(synth.quant_weights("q8_0", N, K, SEED, tensor_id=183))
    x, x2 = dev(synth.normal((8, K), SEED, tensor_id=184)), dev(synth.normal((8, K), SEED, tensor_id=185))
    y, y2 = torch.empty((8, N), device="cuda"), torch.empty((8, N), device="cuda")
    check_replays("qgemv_q8_0_q8act", lambda: qd.qgemv_q8_0_q8act(W, x, y), [y],
                  lambda: qd.qgemv_q8_0_q8act(W, x2, y2))


def test_capture_without_workspace_returns_status(qd):
    """A call made while its stream is capturing, which would have to create
    the stream's workspace, returns QD_ECAPTURE and enqueues nothing: the
    capture stays valid, and the graph (holding only the other call, a
    dequantisation that uses no workspace) replays with correct results.
    After one uncaptured call on the stream the same call can be captured."""
    say("capture without workspace")
    hidden, ff = 512, 1024
    Wg = dev(synth.quant_weights("q4_k", ff, hidden, SEED, tensor_id=186))
    Wu = dev(synth.quant_weights("q4_k", ff, hidden, SEED, tensor_id=187))
    Wd = dev(synth.quant_weights("q6_k", hidden, ff, SEED, tensor_id=188))
    W = dev(synth.quant_weights("q4_k", 64, hidden, SEED, tensor_id=189))
    x = dev(synth.normal((1, hidden), SEED, tensor_id=190))
    w_out = torch.empty((64, hidden), device="cuda")
    y_ffn = torch.empty((1, hidden), device="cuda")
    s = torch.cuda.Stream()   # a fresh stream: no workspace yet
    with torch.cuda.stream(s):
        ref_w = qd.qdequant("q4_k", W, hidden).clone()
        s.synchronize()
        g = torch.cuda.CUDAGraph()
        status = None
        with torch.cuda.graph(g, stream=s):
            try:
                qd.qffn_decode("q4_k", Wg, Wu, "q6_k", Wd, x, None, 1e-6, "gelu_tanh", y=y_ffn)
            except qd.QDError as e:
                status = e.status
            qd.qdequant("q4_k", W, hidden, out=w_out)
        assert status == qd.QD_ECAPTURE, status
        for rep in range(3):
            w_out.fill_(float("nan"))
            g.replay()
            s.synchronize()
            assert np.array_equal(w_out.cpu().numpy().view(np.uint32), ref_w.cpu().numpy().view(np.uint32))
        # one uncaptured call creates the workspace; the captured call then works
        ref_ffn = qd.qffn_decode("q4_k", Wg, Wu, "q6_k", Wd, x, None, 1e-6, "gelu_tanh").clone()
        s.synchronize()
        g2 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g2, stream=s):
            qd.qffn_decode("q4_k", Wg, Wu, "q6_k", Wd, x, None, 1e-6, "gelu_tanh", y=y_ffn)
        for rep in range(3):
            y_ffn.fill_(float("nan"))
            g2.replay()
            s.synchronize()
            assert np.array_equal(y_ffn.cpu().numpy().view(np.uint32), ref_ffn.cpu().numpy().view(np.uint32))
