"""GPU parity of the opt-in int8-activation Q8_0 GEMV (qgemv_q8_0_q8act).

Two bars, both against the oracle:
- the quantized computation: the oracle quantizes x per run of 32 (fp32
  d = max|x| / 127, q = round(x / d) halves away from zero), then sums
  dw dx sum(qw qx) in fp64; the GPU result must be within
  1e-4 * S + 1e-6 of it, S the sum of |products|.  The kernel takes the same
  fp32 rounding decisions (correctly rounded division, round half away), so
  its int8 codes match the oracle's and only the float accumulation differs;
- the exact fp32 GEMV: the activation rounding moves each x by at most d/2,
  so |y - W x| <= sum_j d_j/2 sum_i |w_ji| + 1e-4 * S_exact + 1e-6 (checked
  with the oracle's dequantized weights), and for N(0,1) activations that
  distance stays below 5e-2 * sum|w x|.
The two halves are also checked apart: qquantize_q8_act's codes and scales
must equal the oracle's bit for bit, and qgemv_q8_0_preq, fed the oracle's
own codes, must meet the bound, with K unsplit and split across workgroups
(forced slice counts, ragged last slices, the per-tile counters reused by
consecutive calls).
Shapes: ragged rows, K not a multiple of 256 (ragged superunits), batch 1, 3,
8 and 11 (two launches), K = 16384 where LDS holds three quantized columns,
all-zero and half-way activation runs, and the lm_head shape
262144 x 2560 on sampled rows.
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


from helpers import assert_bound, dev, say  # noqa: E402


def check(name, W, x, got, N, K, n0=0, n1=None):
    n1 = N if n1 is None else n1
    q, d = oracle.quantize_q8_act(x)
    y64, S = oracle.gemv_q8_0_q8act(W, q, d, N, K, n0, n1)
    assert_bound(name, got[:, n0:n1], y64[:, n0:n1], S[:, n0:n1])
    # distance from the exact GEMV, bounded by the activation rounding
    ye, Se = oracle.gemv("q8_0", W, x, N, K, n0, n1)
    Wf = oracle.dequant("q8_0", W, K, n0, n1).astype(np.float64)            # [rows, K]
    half_d = np.repeat(d.astype(np.float64) / 2, 32, axis=1)                 # [batch, K]
    shift = half_d @ np.abs(Wf).T                                            # [batch, rows]
    err = np.abs(got[:, n0:n1].astype(np.float64) - ye[:, n0:n1])
    bound = shift + 1e-4 * Se[:, n0:n1] + 1e-6
    assert (err <= bound).all(), f"{name}: {(err > bound).sum()} outputs beyond the activation-rounding bound"
    return err, Se[:, n0:n1]


@pytest.mark.parametrize("N,K,batch", [
    (300, 2560, 1),      # ragged rows, hidden-size K
    (77, 96, 3),         # K = 3 blocks: one ragged superunit
    (513, 1056, 8),      # 33 blocks: ragged last superunit, batch 8
    (64, 512, 11),       # two launches of 8 + 3 columns
    (40, 16384, 5),      # LDS holds 3 columns: launches of 3 + 2
    (70, 65536, 1),      # one column beyond LDS: K split until a slice fits
])
def test_q8act_parity(qd, N, K, batch):
    say(f"q8act {N}x{K} batch={batch}")
    W = synth.quant_weights("q8_0", N, K, SEED, tensor_id=191)
    x = synth.normal((batch, K), SEED, tensor_id=192)
    y = qd.qgemv_q8_0_q8act(dev(W), dev(x)).cpu().numpy().reshape(batch, N)
    err, Se = check(f"q8act {N}x{K} b{batch}", W, x, y, N, K)
    assert (err <= 5e-2 * Se + 1e-6).all()


def test_q8act_special_runs(qd):
    """An all-zero run (d = 0, q = 0), runs whose x / d lands on a half
    (x = k + 1/2 times d with d a power of two), and negative halves."""
    N, K = 70, 256
    say("q8act special runs")
    W = synth.quant_weights("q8_0", N, K, SEED, tensor_id=193)
    x = synth.normal((2, K), SEED, tensor_id=194)
    x[0, 32:64] = 0.0
    d = 2.0 ** -4
    run = (np.arange(32, dtype=np.float32) - 15.5) * d     # -15.5 d .. 15.5 d
    run[31] = 127 * d                                       # max |x| = 127 d, so the scale is exactly d
    x[1, 0:32] = run
    x[1, 64:96] = -run
    got = qd.qgemv_q8_0_q8act(dev(W), dev(x)).cpu().numpy()
    q, dd = oracle.quantize_q8_act(x)
    assert dd[0, 1] == 0.0 and not q[0, 32:64].any()
    assert dd[1, 0] == np.float32(d) and q[1, 0] == -16 and q[1, 15] == -1 and q[1, 16] == 1
    check("q8act special runs", W, x, got, N, K)


def test_q8act_lm_head_sampled(qd):
    """The Q8_0 lm_head shape 262144 x 2560, batch 1 and 8, on three row
    windows (start, a middle span, the end)."""
    N, K = 262144, 2560
    W = synth.quant_weights("q8_0", N, K, SEED, tensor_id=195)
    Wd = dev(W)
    for batch in (1, 8):
        say(f"q8act lm_head batch={batch}")
        x = synth.normal((batch, K), SEED, tensor_id=196 + batch)
        y = qd.qgemv_q8_0_q8act(Wd, dev(x)).cpu().numpy().reshape(batch, N)
        assert np.isfinite(y).all()
        for n0, n1 in ((0, 300), (131000, 131300), (N - 300, N)):
            check(f"q8act lm_head b{batch} rows {n0}..{n1}", W, x, y, N, K, n0, n1)


def test_q8act_codes_match_fp32_path_on_exact_inputs(qd):
    """Activations that are already int8 multiples of a power-of-two scale
    (max |x| = 127 d in every run) quantize without rounding, so the int8
    path must agree with the fp32 GEMV to the usual bound."""
    N, K = 200, 512
    say("q8act exact inputs")
    rng = np.random.default_rng(SEED)
    W = synth.quant_weights("q8_0", N, K, SEED, tensor_id=199)
    qv = rng.integers(-127, 128, size=(1, K)).astype(np.float32)
    qv[0, ::32] = 127.0
    x = (qv * np.float32(2.0 ** -6)).astype(np.float32)
    got = qd.qgemv_q8_0_q8act(dev(W), dev(x)).cpu().numpy().reshape(1, N)
    ye, Se = oracle.gemv("q8_0", W, x, N, K)
    assert_bound("q8act exact inputs vs fp32 GEMV", got, ye, Se)


@pytest.mark.parametrize("batch,K", [(1, 2560), (3, 96), (64, 512), (8, 10240), (2, 32)])
def test_quantize_codes_bit_exact(qd, batch, K):
    say(f"qquantize_q8_act batch={batch} K={K}")
    x = synth.normal((batch, K), SEED, tensor_id=200) * np.float32(3.0)
    x[0, :32] = 0.0                                            # an all-zero run
    if K >= 96:
        d = np.float32(2.0 ** -3)
        x[-1, 64:96] = (np.arange(32, dtype=np.float32) - 15.5) * d   # exact halves
        x[-1, 95] = 127 * d
    q_ref, d_ref = oracle.quantize_q8_act(x)
    q, dd = qd.qquantize_q8_act(dev(x))
    q, dd = q.cpu().numpy(), dd.cpu().numpy()
    assert np.array_equal(q, q_ref), f"{np.count_nonzero(q != q_ref)} codes differ"
    assert np.array_equal(dd.view(np.uint32), d_ref.view(np.uint32)), "scales differ"


@pytest.mark.parametrize("N,K,batch", [(300, 2560, 1), (2560, 10240, 8), (77, 96, 3), (100, 16384, 7)])
def test_preq_gemv_on_oracle_codes(qd, N, K, batch):
    say(f"qgemv_q8_0_preq {N}x{K} batch={batch}")
    W = synth.quant_weights("q8_0", N, K, SEED, tensor_id=201)
    x = synth.normal((batch, K), SEED, tensor_id=202)
    q, d = oracle.quantize_q8_act(x)
    y = qd.qgemv_q8_0_preq(dev(W), dev(q), dev(d)).cpu().numpy().reshape(batch, N)
    y64, S = oracle.gemv_q8_0_q8act(W, q, d, N, K)
    assert_bound(f"qgemv_q8_0_preq {N}x{K} b{batch}", y, y64, S)


@pytest.mark.parametrize("N,K,batch,p,ks", [
    (513, 1056, 8, 2, 3),     # 5 superunits in slices of 2, 2, 1 (the last ragged)
    (300, 10240, 4, 1, 8),    # 40 superunits, 8 slices of 5
    (77, 2560, 1, 4, 2),      # one column, split
    (2560, 10240, 8, 1, 7),   # 7 slices of 6, 6, ..., 4
    (130, 5376, 3, 1, 21),    # 21 superunits, one per slice
])
def test_preq_split_k(qd, N, K, batch, p, ks):
    say(f"qgemv_q8_0_preq split {N}x{K} batch={batch} p={p} ks={ks}")
    W = synth.quant_weights("q8_0", N, K, SEED, tensor_id=203)
    x = synth.normal((batch, K), SEED, tensor_id=204)
    q, d = oracle.quantize_q8_act(x)
    y64, S = oracle.gemv_q8_0_q8act(W, q, d, N, K)
    Wd, qd_, dd = dev(W), dev(q), dev(d)
    qd.set_launch_override(p, ks, 0)
    try:
        for rep in range(2):  # the tile counters must be back at zero for the second call
            y = qd.qgemv_q8_0_preq(Wd, qd_, dd).cpu().numpy().reshape(batch, N)
            assert_bound(f"preq split {N}x{K} b{batch} p{p} ks{ks} call {rep}", y, y64, S)
    finally:
        qd.set_launch_override(0, 0, 0)
