"""Activations with a large dynamic range, through the paths that stage x as
per-run digits (an exponent per run of 32 and a 31-bit integer per
activation): the batch-1..2 GEMVs and the batch 3..64 matrix-core kernels,
against the oracle.

Each run of 32 activations carries one outlier 10^4 times the others (and
some runs 10^5), so every other activation of the run is rounded at 2^-31 of
the outlier.  Where an outlier meets a zero weight (Q8_0 rows whose quant at
the outlier's column is zeroed), the output bound 1e-4 * sum|w x| + 1e-6 is
set by the small activations alone: the rounding must stay below it there
too.  Shapes: the register GEMV (K = 2560), the LDS-streaming GEMV (K =
10240) and the fused gate/up; batch 1 and 2, and 3, 8 and 19 on the
matrix cores (one and three groups of 8 batch rows).  Also: a run holding an
infinity gives a non-finite output on every row, as fp32 arithmetic would.
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


def spiky(batch, K, tensor_id, big=1e4, huge=1e5):
    """N(0,1) activations, one outlier per run of 32 (x big, every 7th run x huge)."""
    x = synth.normal((batch, K), SEED, tensor_id=tensor_id).astype(np.float64)
    rng = np.random.default_rng(tensor_id)
    runs = K // 32
    cols = np.arange(runs) * 32 + rng.integers(0, 32, size=runs)
    for b in range(batch):
        x[b, cols] *= big
        x[b, cols[::7]] *= huge / big
    return x.astype(np.float32), cols


def zero_q80_columns(W, N, K, cols, rows):
    """Q8_0 rows `rows` get quant 0 (weight 0) at columns `cols`."""
    W = W.copy().reshape(N, K // 32 * 34)
    for j in cols:
        W[rows, (j // 32) * 34 + 2 + (j % 32)] = 0
    return W.reshape(-1)


@pytest.mark.parametrize("fmt", ["q4_k", "q6_k", "q8_0"])
@pytest.mark.parametrize("N,K", [(256, 2560), (64, 10240)])
@pytest.mark.parametrize("batch", [1, 2, 3, 8, 19])
def test_gemv_outliers(qd, fmt, N, K, batch):
    say(f"outliers gemv {fmt} {N}x{K} batch={batch}")
    W = synth.quant_weights(fmt, N, K, SEED, tensor_id=301)
    x, cols = spiky(batch, K, tensor_id=302)
    if fmt == "q8_0":
        W = zero_q80_columns(W, N, K, cols, np.arange(0, N, 2))
    y = qd.qgemv(fmt, dev(W), dev(x)).cpu().numpy()
    y64, S = oracle.gemv(fmt, W, x, N, K)
    assert_bound(f"{fmt} {N}x{K} b{batch} outliers", y, y64, S)


@pytest.mark.parametrize("batch", [1, 2, 8])
def test_gate_up_outliers(qd, batch):
    ff, hidden = 1024, 2560
    say(f"outliers gate/up q4_k {ff}x{hidden} batch={batch}")
    Wg = synth.quant_weights("q4_k", ff, hidden, SEED, tensor_id=303)
    Wu = synth.quant_weights("q4_k", ff, hidden, SEED, tensor_id=304)
    x, _ = spiky(batch, hidden, tensor_id=305)
    g = torch.empty((batch, ff), device="cuda")
    u = torch.empty((batch, ff), device="cuda")
    h = qd.qffn_gate_up_act("q4_k", dev(Wg), dev(Wu), dev(x), None, 1e-6, "silu", g_out=g, u_out=u)
    h, g, u = (t.cpu().numpy() for t in (h, g, u))
    g64, Sg = oracle.gemv("q4_k", Wg, x, ff, hidden)
    u64, Su = oracle.gemv("q4_k", Wu, x, ff, hidden)
    assert_bound("gate outliers", g, g64, Sg)
    assert_bound("up outliers", u, u64, Su)
    href = oracle.act_vec(oracle.ACT_SILU, g64) * u64
    assert (np.abs(h - href) <= h_tolerance(g64, u64, Sg, Su, oracle.ACT_SILU)).all()


@pytest.mark.parametrize("fmt", ["q4_k", "q6_k", "q8_0"])
@pytest.mark.parametrize("K", [2560, 10240])
@pytest.mark.parametrize("batch", [1, 4])
def test_gemv_nonfinite_activation(qd, fmt, K, batch):
    N = 64
    say(f"non-finite activation {fmt} {N}x{K} batch={batch}")
    W = synth.quant_weights(fmt, N, K, SEED, tensor_id=306)
    x = synth.normal((batch, K), SEED, tensor_id=307)
    x[0, 77] = np.inf
    y = qd.qgemv(fmt, dev(W), dev(x)).cpu().numpy()
    assert not np.isfinite(y[0]).any(), f"{fmt} K={K}: an infinite activation left finite outputs"
    if batch > 1:  # the other batch rows are untouched by row 0's infinity
        y64, S = oracle.gemv(fmt, W, x[1:], N, K)
        assert_bound(f"{fmt} {N}x{K} rows 1..{batch - 1}", y[1:], y64, S)
