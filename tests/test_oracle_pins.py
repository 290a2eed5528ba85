"""Pins for the CPU oracle: each test checks the oracle against something
other than itself -- a hand-built block whose weights are known in closed
form, the encoder side of a packing, a library routine, brute force on tiny
inputs, or an exact invariant.

Format layouts follow the GGUF k-quant reading (larql "Architecture -> Metal
shader map", dispatch predicate table: 144-byte GGUF-direct Q4_K blocks;
dotLLM PR #320: 34-byte Q8_0 blocks).  Agreement with real GGUF files is
parity unpinned: no such file is available.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_cases.json")


def f16(v: float) -> int:
    return int(np.float16(v).view(np.uint16))


# ------------------------------------------------------------ encoders ---
# Written from the encoder side of each layout, independent of oracle.c.

def pack_q4k(d, dmin, sc, m, q):
    """Pack one Q4_K block from d, dmin (floats), 8 scales, 8 mins (0..63)
    and 256 quants (0..15)."""
    b = np.zeros(144, dtype=np.uint8)
    b[0:2] = np.frombuffer(np.float16(d).tobytes(), np.uint8)
    b[2:4] = np.frombuffer(np.float16(dmin).tobytes(), np.uint8)
    s = np.zeros(12, dtype=np.int64)
    for j in range(4):
        # low 6 bits of s[j]: scale j; top 2 bits: bits 4..5 of scale j+4
        s[j] = sc[j] | ((sc[j + 4] >> 4) << 6)
        # low 6 bits of s[j+4]: min j; top 2 bits: bits 4..5 of min j+4
        s[j + 4] = m[j] | ((m[j + 4] >> 4) << 6)
        # s[j+8]: low nibble of scale j+4, then low nibble of min j+4
        s[j + 8] = (sc[j + 4] & 15) | ((m[j + 4] & 15) << 4)
    b[4:16] = s.astype(np.uint8)
    qs = np.zeros(128, dtype=np.int64)
    for i in range(256):
        run, pos = divmod(i, 64)
        idx = 32 * run + (pos % 32)
        qs[idx] |= (q[i] & 15) << (0 if pos < 32 else 4)
    b[16:144] = qs.astype(np.uint8)
    return b


def pack_q6k(d, scales, q):
    """Pack one Q6_K block from d, 16 int8 scales and 256 quants (0..63)."""
    b = np.zeros(210, dtype=np.uint8)
    ql = np.zeros(128, dtype=np.int64)
    qh = np.zeros(64, dtype=np.int64)
    for i in range(256):
        h, r = divmod(i, 128)
        g, l = divmod(r, 32)
        lo, hi = q[i] & 15, q[i] >> 4
        idx = 64 * h + 32 * (g % 2) + l
        ql[idx] |= lo << (0 if g < 2 else 4)
        qh[32 * h + l] |= hi << (2 * g)
    b[0:128] = ql.astype(np.uint8)
    b[128:192] = qh.astype(np.uint8)
    b[192:208] = np.asarray(scales, dtype=np.int8).view(np.uint8)
    b[208:210] = np.frombuffer(np.float16(d).tobytes(), np.uint8)
    return b


def pack_q8_0(d, q):
    b = np.zeros(34, dtype=np.uint8)
    b[0:2] = np.frombuffer(np.float16(d).tobytes(), np.uint8)
    b[2:34] = np.asarray(q, dtype=np.int8).view(np.uint8)
    return b


# ---------------------------------------------------------------- f16 ---

def test_f16_all_bit_patterns_match_numpy():
    """binary16 decode of all 65536 patterns equals numpy's conversion."""
    lib = oracle._load()
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    got = np.array([lib.orc_f16_to_f32(int(h)) for h in bits], dtype=np.float32)
    same = (got.view(np.uint32) == ref.view(np.uint32)) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


@pytest.mark.parametrize("bits,val", [(0x3C00, 1.0), (0x0001, 2.0 ** -24), (0x0400, 2.0 ** -14),
                                      (0x7BFF, 65504.0), (0xC000, -2.0), (0x3555, 0.333251953125)])
def test_f16_known_values(bits, val):
    assert oracle.f16_to_f32(bits) == val


# --------------------------------------------------------------- bf16 ---

@pytest.mark.parametrize("x,bits", [
    (1.0, 0x3F80),
    (1.0 + 2.0 ** -8, 0x3F80),        # tie between 1 (even) and 1+2^-7 -> 1
    (1.0 + 3 * 2.0 ** -8, 0x3F82),    # tie between 1+2^-7 (odd) and 1+2^-6 -> even
    (1.0 + 2.0 ** -8 + 2.0 ** -20, 0x3F81),  # just above the tie -> up
    (-1.0 - 2.0 ** -8, 0xBF80),
    (3.3895313892515355e38, 0x7F7F),  # largest finite bf16
])
def test_bf16_rounding_closed_forms(x, bits):
    assert oracle.f32_to_bf16(float(np.float32(x))) == bits


def test_bf16_overflow_midpoint_rounds_to_inf():
    # (2 - 2^-8) * 2^127 is the midpoint between the largest bf16 (odd) and
    # 2^128: ties-to-even rounds up, i.e. to infinity
    mid = np.uint32(0x7F7F8000).view(np.float32)
    below = np.uint32(0x7F7F7FFF).view(np.float32)
    assert oracle.f32_to_bf16(float(mid)) == 0x7F80
    assert oracle.f32_to_bf16(float(below)) == 0x7F7F


def test_bf16_matches_exact_nearest_on_random_values():
    """Nearest bf16 by exhaustive comparison with the two neighbours,
    computed with Python's exact fractions."""
    from fractions import Fraction
    rng = np.random.default_rng(1)
    vals = np.concatenate([rng.standard_normal(300), rng.standard_normal(100) * 1e-38,
                           rng.standard_normal(100) * 1e30]).astype(np.float32)
    for v in vals:
        u = int(np.float32(v).view(np.uint32))
        cands = [(u & 0xFFFF0000), (u & 0xFFFF0000) + 0x10000]
        fv = Fraction(float(v))
        best = None
        for c in cands:
            cv = Fraction(float(np.uint32(c).view(np.float32)))
            dist = abs(cv - fv)
            if best is None or dist < best[0] or (dist == best[0] and ((c >> 16) & 1) == 0):
                best = (dist, c >> 16)
        assert oracle.f32_to_bf16(float(v)) == best[1]
        assert oracle.bf16_to_f32(best[1]) == float(np.uint32(best[1] << 16).view(np.float32))


# --------------------------------------------------------------- Q4_K ---

SC = [1, 2, 3, 4, 17, 33, 49, 63]
MN = [0, 5, 10, 63, 16, 32, 48, 60]


def test_q4k_handbuilt_block():
    """d = 1, dmin = 0.5, known scales/mins/quants -> w = sc*q - 0.5*m."""
    q = [(i * 7 + 3) % 16 for i in range(256)]
    blk = pack_q4k(1.0, 0.5, SC, MN, q)
    w = oracle.dequant_block("q4_k", blk)
    exp = np.array([SC[i // 32] * q[i] - 0.5 * MN[i // 32] for i in range(256)], np.float32)
    assert np.array_equal(w, exp)


def test_q4k_scale_min_exhaustive_roundtrip():
    """Every (scale, min) pair at every sub-block survives pack -> decode."""
    lib = oracle._load()
    import ctypes
    sc_out, m_out = ctypes.c_int(), ctypes.c_int()
    q = [0] * 256
    for j in range(8):
        for s in range(64):
            for m in range(64):
                sc = [(7 * k + 11) % 64 for k in range(8)]
                mn = [(13 * k + 5) % 64 for k in range(8)]
                sc[j], mn[j] = s, m
                blk = pack_q4k(1.0, 1.0, sc, mn, q)
                lib.orc_q4k_scale_min(blk.ctypes.data_as(ctypes.c_void_p), j,
                                      ctypes.byref(sc_out), ctypes.byref(m_out))
                assert (sc_out.value, m_out.value) == (s, m)
                if s % 21 == 0 and m % 21 == 0:
                    # neighbours are untouched
                    for k in range(8):
                        assert oracle.q4k_scale_min(blk, k) == (sc[k], mn[k])


def test_q4k_every_nibble_position_alone():
    """q_i = 15 at one position, all others 0, m = 0: exactly one weight."""
    sc = [1, 2, 3, 4, 5, 6, 7, 8]
    for i in range(256):
        q = [0] * 256
        q[i] = 15
        w = oracle.dequant_block("q4_k", pack_q4k(0.25, 0.0, sc, [0] * 8, q))
        exp = np.zeros(256, np.float32)
        exp[i] = 0.25 * sc[i // 32] * 15
        assert np.array_equal(w, exp), i


def test_q4k_min_only_and_scale_zero():
    """q = 0 everywhere -> w = -dmin*m per sub-block; sc = 0 kills the d term."""
    w = oracle.dequant_block("q4_k", pack_q4k(3.0, 0.125, [0] * 8, MN, [9] * 256))
    exp = np.repeat(np.array([-0.125 * m for m in MN], np.float32), 32)
    assert np.array_equal(w, exp)


def test_q4k_single_rounding():
    """w is the correctly rounded fp32 of the exact real d*sc*q - dmin*m."""
    from fractions import Fraction
    rng = np.random.default_rng(7)
    for _ in range(20):
        d = float(np.float16(rng.uniform(1e-3, 1e-2)))
        dm = float(np.float16(rng.uniform(1e-3, 1e-2)))
        sc = list(rng.integers(0, 64, 8))
        mn = list(rng.integers(0, 64, 8))
        q = list(rng.integers(0, 16, 256))
        w = oracle.dequant_block("q4_k", pack_q4k(d, dm, sc, mn, q))
        for i in range(0, 256, 5):
            exact = Fraction(d) * int(sc[i // 32]) * int(q[i]) - Fraction(dm) * int(mn[i // 32])
            # nearest fp32: compare against float32 neighbours
            f = np.float32(float(exact))
            cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
            best = min(cands, key=lambda c: (abs(Fraction(float(c)) - exact)))
            assert w[i] == best


# --------------------------------------------------------------- Q6_K ---

def test_q6k_handbuilt_block():
    """d = 1/64, scale t = t - 8, q_i = i mod 64 -> w = (t-8)(q-32)/64."""
    scales = [t - 8 for t in range(16)]
    q = [i % 64 for i in range(256)]
    w = oracle.dequant_block("q6_k", pack_q6k(1.0 / 64, scales, q))
    exp = np.array([scales[i // 16] * (q[i] - 32) / 64.0 for i in range(256)], np.float32)
    assert np.array_equal(w, exp)


def test_q6k_every_bit_position():
    """Each of the 6 quant bits of each weight, set alone on top of q = 0."""
    scales = [1] * 16
    for i in range(256):
        for bit in range(6):
            q = [0] * 256
            q[i] = 1 << bit
            w = oracle.dequant_block("q6_k", pack_q6k(1.0, scales, q))
            exp = np.full(256, -32.0, np.float32)
            exp[i] = (1 << bit) - 32
            assert np.array_equal(w, exp), (i, bit)


def test_q6k_scales_are_signed_per_16():
    q = [40] * 256
    scales = [-128, 127, -64, 63, -1, 1, 0, 5, -5, 100, -100, 2, -2, 3, -3, 4]
    w = oracle.dequant_block("q6_k", pack_q6k(0.5, scales, q))
    exp = np.repeat(np.array([0.5 * s * 8 for s in scales], np.float32), 16)
    assert np.array_equal(w, exp)


# --------------------------------------------------------------- Q8_0 ---

def test_q8_0_handbuilt_block():
    q = [i - 16 for i in range(32)]
    q[5] = -128
    q[6] = 127
    w = oracle.dequant_block("q8_0", pack_q8_0(0.25, q))
    assert np.array_equal(w, np.array([0.25 * v for v in q], np.float32))


def test_q8_0_regression_shapes_row_stride():
    """The pages' odd-block regression rows: row n must start at n*K/32*34."""
    cases = json.load(open(GOLDEN))["q8_0_row_stride_regression"]["cases_rows_K"]
    for M, K in cases:
        nb = K // 32
        blocks = []
        for n in range(M):
            for b in range(nb):
                blocks.append(pack_q8_0(float(n + 1), [(n * 3 + b + i) % 7 - 3 for i in range(32)]))
        W = np.concatenate(blocks)
        assert W.size == M * nb * 34
        w = oracle.dequant("q8_0", W, K)
        for n in range(M):
            for b in range(nb):
                exp = np.array([(n + 1) * ((n * 3 + b + i) % 7 - 3) for i in range(32)], np.float32)
                assert np.array_equal(w[n, 32 * b:32 * b + 32], exp)


# --------------------------------------------------------------- GEMV ---

@pytest.mark.parametrize("fmt,K", [("q4_k", 512), ("q6_k", 512), ("q8_0", 96)])
def test_gemv_one_hot_returns_column(fmt, K):
    N = 5
    W = synth.quant_weights(fmt, N, K, seed=3)
    wd = oracle.dequant(fmt, W, K)
    for k in [0, 1, 31, 32, 63, K - 1]:
        x = np.zeros(K, np.float32)
        x[k] = 1.0
        y, S = oracle.gemv(fmt, W, x, N, K)
        assert np.array_equal(y[0], wd[:, k].astype(np.float64))
        assert np.array_equal(S[0], np.abs(wd[:, k]).astype(np.float64))


@pytest.mark.parametrize("fmt,K", [("q4_k", 256), ("q6_k", 256), ("q8_0", 64)])
def test_gemv_brute_force_tiny(fmt, K):
    """Against an independent numpy float64 matmul of the decoded matrix."""
    N, B = 7, 3
    W = synth.quant_weights(fmt, N, K, seed=11)
    x = synth.normal((B, K), seed=12)
    y, S = oracle.gemv(fmt, W, x, N, K)
    wd = oracle.dequant(fmt, W, K).astype(np.float64)
    ref = x.astype(np.float64) @ wd.T
    refS = np.abs(x.astype(np.float64)) @ np.abs(wd).T
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S, refS, rtol=1e-12, atol=1e-12)


def test_gemv_all_ones_gives_row_sums_of_handbuilt_block():
    q = [(i * 5) % 16 for i in range(256)]
    blk = pack_q4k(0.5, 0.25, SC, MN, q)
    W = np.concatenate([blk, blk])
    y, _ = oracle.gemv("q4_k", W, np.ones(256, np.float32), 2, 256)
    exp = sum(0.5 * SC[i // 32] * q[i] - 0.25 * MN[i // 32] for i in range(256))
    assert y[0, 0] == exp and y[0, 1] == exp


def test_gemv_scaling_is_exact_and_rows_independent():
    K, N = 512, 9
    W = synth.quant_weights("q6_k", N, K, seed=5)
    x = synth.normal((K,), seed=6)
    y1, _ = oracle.gemv("q6_k", W, x, N, K)
    y2, _ = oracle.gemv("q6_k", W, 2 * x, N, K)
    assert np.array_equal(2 * y1, y2)
    # rows computed one range at a time equal the whole computation
    yr, _ = oracle.gemv("q6_k", W, x, N, K, n0=4, n1=9)
    assert np.array_equal(yr[0, 4:], y1[0, 4:])
    assert np.isnan(yr[0, :4]).all()


def test_gemv_rejects_bad_shapes():
    lib = oracle._load()
    W = np.zeros(144, np.uint8)
    x = np.zeros(256, np.float32)
    p = oracle._ptr
    assert lib.orc_gemv(0, p(W), p(x), 1, 100, 1, 0, 1, None, None) == -1
    assert lib.orc_gemv(0, p(W), p(x), 1, 256, 0, 0, 1, None, None) == -1
    assert lib.orc_gemv(7, p(W), p(x), 1, 256, 1, 0, 1, None, None) == -1
    assert oracle.row_bytes("q8_0", 96) == 102
    assert oracle.row_bytes("q4_k", 2560) == 1440
    assert oracle.row_bytes("q6_k", 10240) == 8400


# ----------------------------------------------------------- RMS-norm ---

def test_rmsnorm_constant_vector_closed_form():
    K, c, eps = 64, 3.0, 1e-6
    x = np.full(K, c, np.float32)
    w = np.linspace(0.5, 1.5, K).astype(np.float32)
    out = oracle.rmsnorm(x, w, eps)[0]
    exp = w.astype(np.float64) * c / math.sqrt(c * c + eps)
    np.testing.assert_allclose(out, exp, rtol=1e-15)


def test_rmsnorm_unit_rms_and_weight_direct():
    """With w = 1 the output has mean square K/(K + eps*K/ms) ~ 1; w enters
    linearly (no 1 + w offset)."""
    x = synth.normal((2, 256), seed=2)
    ones = np.ones(256, np.float32)
    out = oracle.rmsnorm(x, ones, 0.0)
    np.testing.assert_allclose((out ** 2).mean(axis=1), 1.0, rtol=1e-12)
    out2 = oracle.rmsnorm(x, 2 * ones, 0.0)
    np.testing.assert_array_equal(out2, 2 * out)


# ------------------------------------------------- Post-norm residual ---

def test_post_norm_constant_projection_closed_form():
    """p = c * 1: the normalised projection is w1 * c / sqrt(c^2 + eps), so
    y = r + w1 * c / sqrt(c^2 + eps); the sign of c carries through."""
    N, eps = 96, 1e-6
    r = synth.normal((2, N), seed=5)
    w1 = np.linspace(0.5, 1.5, N).astype(np.float32)
    for c in (3.0, -0.25):
        p = np.full((2, N), c)
        y, _ = oracle.post_norm_residual(p, r, w1, eps)
        exp = r.astype(np.float64) + w1.astype(np.float64) * c / math.sqrt(c * c + eps)
        np.testing.assert_allclose(y, exp, rtol=1e-14, atol=1e-15)


def test_post_norm_zero_projection_is_residual():
    """p = 0 adds nothing (the norm of zero is zero for eps > 0), so y = r
    exactly; y2 is then the RMS-norm of r, which equals orc_rmsnorm of r."""
    N = 128
    r = synth.normal((3, N), seed=6)
    w1 = synth.normal((N,), seed=7, mean=1.0, std=0.1)
    w2 = synth.normal((N,), seed=8, mean=1.0, std=0.1)
    y, y2 = oracle.post_norm_residual(np.zeros((3, N)), r, w1, 1e-6, w2)
    np.testing.assert_array_equal(y, r.astype(np.float64))
    np.testing.assert_array_equal(y2, oracle.rmsnorm(r, w2, 1e-6))


def test_post_norm_scale_invariance_and_unit_rms():
    """With eps = 0 the normalised projection does not depend on the scale
    of p (p -> 2^k p gives the same y exactly), and with w2 = 1 the second
    output has mean square 1; the weights enter linearly (no 1 + w)."""
    N = 256
    p = synth.normal((2, N), seed=9).astype(np.float64)
    r = synth.normal((2, N), seed=10)
    w1 = synth.normal((N,), seed=11, mean=1.0, std=0.1)
    ones = np.ones(N, np.float32)
    y, y2 = oracle.post_norm_residual(p, r, w1, 0.0, ones)
    y8, _ = oracle.post_norm_residual(8.0 * p, r, w1, 0.0)
    np.testing.assert_array_equal(y, y8)
    np.testing.assert_allclose((y2 ** 2).mean(axis=1), 1.0, rtol=1e-12)
    z0, _ = oracle.post_norm_residual(p, np.zeros_like(r), w1, 0.0)
    z1, _ = oracle.post_norm_residual(p, np.zeros_like(r), 2 * w1, 0.0)
    np.testing.assert_array_equal(z1, 2 * z0)
    # the normalised part has unit RMS before the weight: w1 = 1, r = 0
    u, _ = oracle.post_norm_residual(p, np.zeros_like(r), ones, 0.0)
    np.testing.assert_allclose((u ** 2).mean(axis=1), 1.0, rtol=1e-12)


# -------------------------------------------------------- Activations ---

def test_activations_against_torch_float64():
    import torch
    g = np.linspace(-12, 12, 2001)
    gelu = oracle.act_vec(oracle.ACT_GELU_TANH, g)
    silu = oracle.act_vec(oracle.ACT_SILU, g)
    tg = torch.tensor(g, dtype=torch.float64)
    ref_gelu = torch.nn.functional.gelu(tg, approximate="tanh").numpy()
    ref_silu = torch.nn.functional.silu(tg).numpy()
    np.testing.assert_allclose(gelu, ref_gelu, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(silu, ref_silu, rtol=1e-14, atol=1e-15)


def test_activation_special_values():
    assert oracle.act(oracle.ACT_GELU_TANH, 0.0) == 0.0
    assert oracle.act(oracle.ACT_SILU, 0.0) == 0.0
    assert abs(oracle.act(oracle.ACT_GELU_TANH, 30.0) - 30.0) < 1e-12
    assert abs(oracle.act(oracle.ACT_GELU_TANH, -30.0)) < 1e-12
    assert abs(oracle.act(oracle.ACT_SILU, 1.0) - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16


# ------------------------------------------------------- bf16 GEMM ------

def test_gemm_bf16_against_numpy_of_rounded_operands():
    fmt, N, K, M = "q4_k", 6, 512, 4
    W = synth.quant_weights(fmt, N, K, seed=21)
    X = synth.normal_bf16((M, K), seed=22)
    Y, S = oracle.gemm_bf16(fmt, W, X, N, K)
    wd = oracle.dequant(fmt, W, K)
    # bf16 rounding of the weights done here with the bit trick (a separate
    # implementation from the oracle's distance-based rounding)
    wb = (synth.bf16_bits(wd).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    xb = (X.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    np.testing.assert_allclose(Y, xb @ wb.T, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S, np.abs(xb) @ np.abs(wb).T, rtol=1e-12, atol=1e-12)


def test_gemm_bf16_m1_reduces_to_gemv_on_bf16_weights():
    fmt, N, K = "q6_k", 5, 256
    W = synth.quant_weights(fmt, N, K, seed=31)
    X = synth.normal_bf16((1, K), seed=32)
    Y, _ = oracle.gemm_bf16(fmt, W, X, N, K)
    # gemv on the same operands: bf16 weights as a dense matrix via numpy
    wd = oracle.dequant(fmt, W, K)
    wb = (synth.bf16_bits(wd).astype(np.uint32) << 16).view(np.float32)
    xb = (X.astype(np.uint32) << 16).view(np.float32)
    exact = [sum(float(a) * float(b) for a, b in zip(wb[n], xb[0])) for n in range(N)]
    np.testing.assert_allclose(Y[0], exact, rtol=1e-12)


# ------------------------------------------- int8-quantized activations ---
# dotLLM PR #320 (CPU Q8_0 kernels: GemmQ8_0 on pre-quantized input).  Pins of
# the quantizer: worked values, exact power-of-two scaling, sign symmetry and
# range; of the Q8_0 x int8 GEMV: an independent numpy float64 evaluation from
# the raw bytes, and closeness to the unquantized GEMV.

def test_q8_act_quantizer_worked_values():
    x = np.zeros((1, 64), np.float32)
    x[0, :6] = [127.0, -63.5, 2.5, -2.5, 0.4, -0.5]
    q, d = oracle.quantize_q8_act(x)
    assert d[0, 0] == np.float32(1.0) and d[0, 1] == 0.0          # amax 127 -> d 1; zero run -> d 0
    assert list(q[0, :6]) == [127, -64, 3, -3, 0, -1]              # halves away from zero
    assert not q[0, 32:].any()


def test_q8_act_quantizer_scaling_sign_and_range():
    x = synth.normal((3, 256), 0x5EED, tensor_id=201)
    q, d = oracle.quantize_q8_act(x)
    for k in (-7, 3):                                              # x * 2^k: same q, d * 2^k exactly
        q2, d2 = oracle.quantize_q8_act((x * np.float32(2.0 ** k)).astype(np.float32))
        assert np.array_equal(q2, q) and np.array_equal(d2, d * np.float32(2.0 ** k))
    qn, dn = oracle.quantize_q8_act(-x)
    assert np.array_equal(qn, -q) and np.array_equal(dn, d)
    assert np.abs(q).max() <= 127
    assert (np.abs(q).reshape(3, 8, 32).max(axis=2) == 127).all()  # every run reaches the full range
    # each value is within half a step of its quantized value
    err = np.abs(x.reshape(3, 8, 32) - q.reshape(3, 8, 32) * d[:, :, None])
    assert (err <= 0.5 * d[:, :, None] * (1 + 1e-6)).all()


def test_q8_act_gemv_against_numpy_from_bytes():
    N, K = 5, 96
    W = synth.quant_weights("q8_0", N, K, 0x5EED, tensor_id=202)
    x = synth.normal((2, K), 0x5EED, tensor_id=203)
    q, d = oracle.quantize_q8_act(x)
    y, S = oracle.gemv_q8_0_q8act(W, q, d, N, K)
    blocks = W.reshape(N, K // 32, 34)
    dw = blocks[:, :, :2].copy().view(np.float16)[:, :, 0].astype(np.float64)   # numpy's f16 decode
    qw = blocks[:, :, 2:].view(np.int8).astype(np.float64)
    qx = q.reshape(2, K // 32, 32).astype(np.float64)
    prod = dw[None, :, :, None] * d.astype(np.float64)[:, None, :, None] * qw[None] * qx[:, None]
    assert np.allclose(y, prod.sum(axis=(2, 3)), rtol=1e-13, atol=0)
    assert np.allclose(S, np.abs(prod).sum(axis=(2, 3)), rtol=1e-13, atol=0)


def test_q8_act_gemv_close_to_exact_gemv():
    N, K = 64, 2560
    W = synth.quant_weights("q8_0", N, K, 0x5EED, tensor_id=204)
    x = synth.normal((1, K), 0x5EED, tensor_id=205)
    q, d = oracle.quantize_q8_act(x)
    yq, _ = oracle.gemv_q8_0_q8act(W, q, d, N, K)
    y, S = oracle.gemv("q8_0", W, x, N, K)
    assert (np.abs(yq - y) <= 5e-2 * S + 1e-6).all()


def test_cancelling_q4k_blocks_decode_to_zero():
    """The cancelling Q4_K blocks the GPU tests build (constant quant q0 per
    sub-block, d*sc*q0 == dmin*m exactly) decode to exact zeros, and moving
    a quant by +-1 gives +-d*sc exactly: the oracle's single rounding of
    d*sc*q - dmin*m is exact here, whatever the size of the two terms."""
    import sys
    sys.path.insert(0, os.path.dirname(__file__))
    from helpers import cancelling_q4k
    W = cancelling_q4k(16, 1024, seed=3)
    assert not oracle.dequant("q4_k", W, 1024).any()
    Wf = cancelling_q4k(16, 1024, seed=4, flip_frac=0.1)
    w = oracle.dequant("q4_k", Wf, 1024)
    blocks = Wf.reshape(-1, 144)
    for bi in range(0, blocks.shape[0], 7):
        d = float(np.frombuffer(blocks[bi, 0:2].tobytes(), np.float16)[0])
        for j in range(8):
            sc, _ = oracle.q4k_scale_min(blocks[bi], j)
            row, col = divmod(bi, 1024 // 256)
            sub = w[row, 256 * col + 32 * j: 256 * col + 32 * j + 32]
            assert set(np.unique(np.abs(sub)).tolist()) <= {0.0, float(np.float32(d * sc))}
