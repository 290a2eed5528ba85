"""GPU parity of the fused Q/K/V projection (qqkv_proj) against the oracle.

Each of q, k and v must meet the GEMV bound |y - y_ref| <= 1e-4 * sum|w x| +
1e-6 against the oracle's GEMV of the oracle's RMS-normalised x (rounded to
fp32).  Cases: the Gemma-3-4B attention shapes (Q 2048, K 1024, V 1024 rows
over K = 2560) in the Q4_K/Q4_K/Q6_K mix and in Q8_0; small ragged row counts
that leave partial tiles, batch 1..8, with and without the norm; and the
shapes that fall back to three GEMV launches (K beyond one workgroup's LDS,
Q8_0 with K not a multiple of 256).

At batch 1 with rows of whole 256-weight superunits the three matrices run
on the streaming kernel in one launch; other batches, other rows and any
forced launch shape take the register kernel, which the `register_kernel`
cases run on the batch-1 shapes.
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


from helpers import assert_bound, dev, say  # noqa: E402


@pytest.fixture
def register_kernel(qd):
    """A forced launch shape keeps Q/K/V on the register kernel."""
    qd.set_launch_override(4, 0, 0)
    yield
    qd.set_launch_override(0, 0, 0)


def check_qkv(qd, fmts, Ns, K, batch, with_norm=True, tag="", rows=None):
    Ws = [synth.quant_weights(f, n, K, SEED, tensor_id=60 + i) for i, (f, n) in enumerate(zip(fmts, Ns))]
    x = synth.normal((batch, K), SEED, tensor_id=63)
    nw = synth.normal((K,), SEED, tensor_id=64, mean=1.0, std=0.1)
    say(f"qkv {tag} {fmts} rows={Ns} K={K} batch={batch} norm={with_norm}")
    # outputs pre-filled with NaN: every element must be written
    outs = [torch.full((batch, n), float("nan"), device="cuda") for n in Ns]
    qd.qqkv_proj(fmts, *[dev(W) for W in Ws], dev(x), dev(nw) if with_norm else None, 1e-6,
                 q=outs[0], k=outs[1], v=outs[2])
    torch.cuda.synchronize()
    xn = oracle.rmsnorm(x, nw, 1e-6) if with_norm else x.astype(np.float64)
    xn32 = xn.astype(np.float32)
    for name, f, n, W, o in zip("qkv", fmts, Ns, Ws, outs):
        got = o.cpu().numpy()
        assert np.isfinite(got).all(), f"{tag} {name}: unwritten outputs"
        r = rows if rows is not None and n > 4096 else None
        if r is None:
            y64, S = oracle.gemv(f, W, xn32, n, K)
            assert_bound(f"{tag} {name}", got, y64, S)
        else:
            y64, S = oracle.gemv_rows(f, W, xn32, n, K, r)
            assert_bound(f"{tag} {name}", got, y64, S, r)


@pytest.mark.parametrize("variant", ["kquant", "q8_0"])
def test_qkv_gemma3_4b(qd, variant):
    fm = ("q4_k", "q4_k", "q6_k") if variant == "kquant" else ("q8_0",) * 3
    check_qkv(qd, fm, (2048, 1024, 1024), 2560, 1, tag=f"gemma3 {variant}")


@pytest.mark.parametrize("fmts", [("q4_k", "q4_k", "q6_k"), ("q6_k", "q8_0", "q4_k"),
                                  ("q8_0", "q6_k", "q8_0")])
@pytest.mark.parametrize("batch", [1, 3, 8])
def test_qkv_ragged_rows(qd, fmts, batch):
    check_qkv(qd, fmts, (37, 5, 130), 512, batch, tag="ragged")


def test_qkv_single_rows_without_norm(qd):
    check_qkv(qd, ("q4_k", "q6_k", "q8_0"), (1, 1, 1), 768, 2, with_norm=False, tag="one row")


def test_qkv_gemma4_31b_shapes(qd):
    # Gemma-4-31B hidden size: a long activation row that still fits one tile
    check_qkv(qd, ("q4_k", "q4_k", "q6_k"), (512, 256, 256), 5376, 1, tag="gemma4 K=5376")


@pytest.mark.parametrize("fmts,K,batch", [(("q4_k", "q4_k", "q6_k"), 16384, 2),
                                          (("q8_0", "q8_0", "q8_0"), 96, 1)])
def test_qkv_three_launch_fallback(qd, fmts, K, batch):
    check_qkv(qd, fmts, (40, 24, 24), K, batch, tag="fallback")


def test_qkv_long_rows_streaming(qd):
    """K = 16384 at batch 1: beyond the register kernel's staging, on the
    streaming kernel."""
    check_qkv(qd, ("q4_k", "q4_k", "q6_k"), (40, 24, 24), 16384, 1, tag="stream K=16384")


def test_qkv_more_rows_than_cus(qd):
    """Fewer rows than workgroups for one matrix, many rows per workgroup for
    another."""
    check_qkv(qd, ("q6_k", "q4_k", "q8_0"), (3000, 2, 700), 1024, 1, tag="uneven shares")


@pytest.mark.parametrize("variant", ["kquant", "q8_0"])
def test_qkv_register_kernel_gemma3_4b(qd, register_kernel, variant):
    fm = ("q4_k", "q4_k", "q6_k") if variant == "kquant" else ("q8_0",) * 3
    check_qkv(qd, fm, (2048, 1024, 1024), 2560, 1, tag=f"register kernel {variant}")


def test_qkv_register_kernel_ragged(qd, register_kernel):
    check_qkv(qd, ("q6_k", "q8_0", "q4_k"), (37, 5, 130), 512, 1, tag="register kernel ragged")


@pytest.mark.parametrize("batch", [1, 2])
def test_qkv_repeatable_bitwise(qd, batch):
    fm = ("q4_k", "q4_k", "q6_k")
    Ws = [dev(synth.quant_weights(f, n, 2560, SEED, tensor_id=70 + i)) for i, (f, n) in
          enumerate(zip(fm, (300, 100, 100)))]
    x = dev(synth.normal((batch, 2560), SEED, tensor_id=73))
    nw = dev(synth.normal((2560,), SEED, tensor_id=74, mean=1.0, std=0.1))
    a = [t.cpu().numpy() for t in qd.qqkv_proj(fm, *Ws, x, nw)]
    b = [t.cpu().numpy() for t in qd.qqkv_proj(fm, *Ws, x, nw)]
    for u, w in zip(a, b):
        assert np.array_equal(u.view(np.uint32), w.view(np.uint32))
