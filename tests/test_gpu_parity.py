"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Bars:
  * dequantised weights (fp32 and bf16) are bit-exact;
  * every GEMV output meets |y - y_ref| <= 1e-4 * sum|w x| + 1e-6 with y_ref
    and the sum taken in fp64 by the oracle;
  * the fused FFN's g and u meet that bound against the oracle's GEMV of the
    oracle's RMS-normalised x, and h = act(g) u meets the bound propagated
    through the activation (see h_tolerance);
  * the down projection is checked on the GPU's own h (stage by stage).
Full-size cases run in the launch configuration bench.py times (automatic
launch shapes); small cases also sweep forced launch shapes.
"""
import json
import os

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
    qd.set_walk_override(0)


from helpers import GELU_LIP, SILU_LIP, assert_bound, dev, h_tolerance, say  # noqa: E402


# ------------------------------------------------------------ dequant ---

DEQ_CASES = [("q4_k", 7, 512), ("q4_k", 3, 2560), ("q6_k", 7, 512), ("q6_k", 5, 2560),
             ("q6_k", 2, 21504), ("q8_0", 8, 32), ("q8_0", 4, 96), ("q8_0", 2, 160),
             ("q8_0", 5, 2560), ("q8_0", 3, 2592)]


@pytest.mark.parametrize("fmt,N,K", DEQ_CASES)
def test_dequant_fp32_bit_exact(qd, fmt, N, K):
    say(f"dequant fp32 {fmt} N={N} K={K}")
    W = synth.quant_weights(fmt, N, K, SEED, tensor_id=11)
    got = qd.qdequant(fmt, dev(W), K).cpu().numpy()
    ref = oracle.dequant(fmt, W, K)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("fmt,N,K", [("q4_k", 2, 512), ("q6_k", 3, 512), ("q8_0", 3, 96)])
def test_dequant_bf16_bit_exact(qd, fmt, N, K):
    say(f"dequant bf16 {fmt} N={N} K={K}")
    W = synth.quant_weights(fmt, N, K, SEED, tensor_id=12)
    got = qd.qdequant_bf16(fmt, dev(W), K).cpu().numpy().view(np.uint16)
    ref32 = oracle.dequant(fmt, W, K)
    ref = np.array([oracle.f32_to_bf16(float(v)) for v in ref32.ravel()], np.uint16).reshape(ref32.shape)
    assert np.array_equal(got, ref)


def test_dequant_fp8_nibble_unit_all_values(qd):
    """Every 4-bit quant value through the in-register converter: a Q4_K block
    with d = 1, dmin = 0, scale 1 and quant i % 16 decodes to i % 16."""
    say("dequant nibble unit")
    blk = np.zeros(144, np.uint8)
    blk[0:2] = np.frombuffer(np.float16(1.0).tobytes(), np.uint8)
    blk[4:8] = 1                      # scales of sub-blocks 0..3 = 1, mins 0
    blk[12:16] = 1                    # scales of sub-blocks 4..7 = 1 (low nibble of s[8..11])
    qs = np.zeros(128, np.uint8)
    for i in range(256):
        run, pos = divmod(i, 64)
        qs[32 * run + pos % 32] |= (i % 16) << (0 if pos < 32 else 4)
    blk[16:] = qs
    got = qd.qdequant("q4_k", dev(blk), 256).cpu().numpy()[0]
    assert np.array_equal(got, np.array([i % 16 for i in range(256)], np.float32))


# --------------------------------------------------------------- GEMV ---

GEMV_SMALL = [("q4_k", 257, 512), ("q4_k", 64, 2560), ("q6_k", 257, 512), ("q6_k", 33, 2560),
              ("q8_0", 257, 96), ("q8_0", 70, 2592), ("q8_0", 64, 2560)]


@pytest.mark.parametrize("fmt,N,K", GEMV_SMALL)
@pytest.mark.parametrize("batch", [1, 3, 8])
def test_gemv_small(qd, fmt, N, K, batch):
    say(f"gemv {fmt} N={N} K={K} batch={batch}")
    W = synth.quant_weights(fmt, N, K, SEED, tensor_id=21)
    x = synth.normal((batch, K), SEED, tensor_id=22)
    y = qd.qgemv(fmt, dev(W), dev(x)).cpu().numpy()
    y64, S = oracle.gemv(fmt, W, x, N, K)
    assert_bound(f"{fmt} {N}x{K} b{batch}", y, y64, S)


PAGE_CASES = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_cases.json")))


@pytest.mark.parametrize("case", PAGE_CASES["q8_0_row_stride_regression"]["cases_rows_K"])
def test_gemv_q8_0_page_regression_rows(qd, case):
    """dotLLM's odd-block regression rows (rows past 0 read at the right stride)."""
    N, K = case
    say(f"gemv q8_0 regression N={N} K={K}")
    W = synth.quant_weights("q8_0", N, K, SEED, tensor_id=23)
    x = synth.normal((K,), SEED, tensor_id=24)
    y = qd.qgemv_q8_0(dev(W), dev(x)).cpu().numpy()
    y64, S = oracle.gemv("q8_0", W, x, N, K)
    assert_bound("q8_0 regression", y, y64[0], S[0])


SHAPES = [(1, 1, 1), (2, 1, 1), (4, 1, 2), (16, 1, 1), (1, 2, 1), (2, 4, 2), (1, 5, 1), (8, 3, 2)]


@pytest.mark.parametrize("fmt", ["q4_k", "q6_k", "q8_0"])
def test_gemv_forced_launch_shapes(qd, fmt):
    """Every (p_in, p_out, nr) gives results within the bound, including
    split-K across workgroups with its workspace reduction."""
    N, K = 300, 2560
    W = synth.quant_weights(fmt, N, K, SEED, tensor_id=25)
    x = synth.normal((2, K), SEED, tensor_id=26)
    y64, S = oracle.gemv(fmt, W, x, N, K)
    Wd, xd = dev(W), dev(x)
    try:
        for p_in, p_out, nr in SHAPES:
            say(f"gemv {fmt} shape p_in={p_in} p_out={p_out} nr={nr}")
            qd.set_launch_override(p_in, p_out, nr)
            for rep in range(2):   # the split-K counters must be reset for the next call
                y = qd.qgemv(fmt, Wd, xd).cpu().numpy()
                assert_bound(f"{fmt} {p_in}/{p_out}/{nr} rep{rep}", y, y64, S)
    finally:
        qd.set_launch_override(0, 0, 0)


# (p_in, p_out, nr, rows per lane group): groups walking several row slots,
# with K = 2560 (10 superunits) leaving dead units when p_in does not divide
# a slice, split-K across workgroups, and row counts that end mid-walk
WALKS = [(2, 1, 1, 2), (2, 1, 1, 8), (1, 1, 2, 3), (4, 1, 1, 5), (2, 3, 1, 4), (1, 4, 2, 2),
         (8, 2, 1, 3), (16, 1, 1, 2)]


@pytest.mark.parametrize("fmt", ["q4_k", "q6_k", "q8_0"])
@pytest.mark.parametrize("N,batch", [(300, 1), (1, 2), (1000, 8), (37, 1)])
def test_gemv_row_walk(qd, fmt, N, batch):
    """Lane groups that walk several rows (the register-streaming kernel's
    row walk) stay within the bound for every launch shape; a call repeated
    with the same shape is bitwise identical (split-K counters reset)."""
    K = 2560
    W = synth.quant_weights(fmt, N, K, SEED, tensor_id=57)
    x = synth.normal((batch, K), SEED, tensor_id=58)
    y64, S = oracle.gemv(fmt, W, x, N, K)
    Wd, xd = dev(W), dev(x)
    try:
        for p_in, p_out, nr, rpg in WALKS:
            say(f"gemv walk {fmt} N={N} batch={batch} p_in={p_in} p_out={p_out} nr={nr} rpg={rpg}")
            qd.set_launch_override(p_in, p_out, nr)
            qd.set_walk_override(rpg)
            y = qd.qgemv(fmt, Wd, xd).cpu().numpy()
            assert_bound(f"{fmt} walk {p_in}/{p_out}/{nr}/{rpg}", y, y64, S)
            again = qd.qgemv(fmt, Wd, xd).cpu().numpy()
            assert np.array_equal(y.view(np.uint32), again.view(np.uint32))
    finally:
        qd.set_launch_override(0, 0, 0)
        qd.set_walk_override(0)


@pytest.mark.parametrize("fmt,N,K", [("q4_k", 300, 2560), ("q8_0", 77, 1024), ("q6_k", 130, 2048)])
@pytest.mark.parametrize("batch", [1, 8])
def test_gate_up_row_walk(qd, fmt, N, K, batch):
    """The fused gate/up on the register-streaming kernel with walking lane
    groups: g, u each within the bound, h within the propagated bound."""
    Wg = synth.quant_weights(fmt, N, K, SEED, tensor_id=59)
    Wu = synth.quant_weights(fmt, N, K, SEED, tensor_id=60)
    x = synth.normal((batch, K), SEED, tensor_id=61)
    nw = synth.normal((K,), SEED, tensor_id=62, mean=1.0, std=0.1)
    xn = oracle.rmsnorm(x, nw, 1e-6).astype(np.float32)
    g64, Sg = oracle.gemv(fmt, Wg, xn, N, K)
    u64, Su = oracle.gemv(fmt, Wu, xn, N, K)
    href = oracle.act_vec(oracle.ACT_GELU_TANH, g64) * u64
    tol = h_tolerance(g64, u64, Sg, Su, oracle.ACT_GELU_TANH)
    try:
        for p_in, p_out, rpg in ((2, 1, 4), (1, 2, 3), (4, 1, 7)):
            say(f"gate/up walk {fmt} N={N} K={K} batch={batch} p_in={p_in} p_out={p_out} rpg={rpg}")
            qd.set_launch_override(p_in, p_out, 0)
            qd.set_walk_override(rpg)
            g = torch.empty((batch, N), device="cuda")
            u = torch.empty((batch, N), device="cuda")
            h = qd.qffn_gate_up_act(fmt, dev(Wg), dev(Wu), dev(x), dev(nw), 1e-6, "gelu_tanh",
                                    g_out=g, u_out=u).cpu().numpy()
            assert_bound("gate", g.cpu().numpy(), g64, Sg)
            assert_bound("up", u.cpu().numpy(), u64, Su)
            err = np.abs(h - href)
            assert (err <= tol).all(), f"h: worst {np.max(err / tol):.3f} of tolerance"
    finally:
        qd.set_launch_override(0, 0, 0)
        qd.set_walk_override(0)


@pytest.mark.parametrize("fmt,K", [("q4_k", 2560), ("q6_k", 2560), ("q8_0", 2560)])
def test_gemv_one_hot_and_zero_exact(qd, fmt, K):
    """x = e_k returns column k exactly; x = 0 returns 0."""
    N = 129
    say(f"gemv one-hot {fmt}")
    W = synth.quant_weights(fmt, N, K, SEED, tensor_id=27)
    wd = oracle.dequant(fmt, W, K)
    ks = [0, 1, 37, 255, 256, K - 1]
    x = np.zeros((len(ks), K), np.float32)
    for b, k in enumerate(ks):
        x[b, k] = 1.0
    y = qd.qgemv(fmt, dev(W), dev(x)).cpu().numpy()
    for b, k in enumerate(ks):
        assert np.array_equal(y[b], wd[:, k]), (fmt, k)
    z = qd.qgemv(fmt, dev(W), dev(np.zeros(K, np.float32))).cpu().numpy()
    assert not z.any()


def test_gemv_zero_weight_blocks(qd):
    """d = 0 blocks (all formats) and Q6_K quants at 32 give exact zeros."""
    say("gemv zero blocks")
    K, N = 512, 8
    x = synth.normal((K,), SEED, tensor_id=28)
    for fmt in ("q4_k", "q6_k", "q8_0"):
        W = synth.quant_weights(fmt, N, K, SEED, tensor_id=29)
        bb, qk = synth.BLOCK[fmt]
        Wz = W.reshape(-1, bb).copy()
        dcol = 208 if fmt == "q6_k" else 0
        Wz[:, dcol:dcol + 2] = 0
        if fmt == "q4_k":
            Wz[:, 2:4] = 0
        y = qd.qgemv(fmt, dev(Wz.ravel()), dev(x)).cpu().numpy()
        assert not y.any(), fmt
    W = synth.quant_weights("q6_k", N, K, SEED, tensor_id=30).reshape(-1, 210).copy()
    W[:, 0:128] = 0x00      # low bits 0
    W[:, 128:192] = 0xAA    # high bits 2 -> q = 32 everywhere
    y = qd.qgemv("q6_k", dev(W.ravel()), dev(x)).cpu().numpy()
    assert not y.any()


def test_gemv_deterministic_and_batch_columns(qd):
    """Repeated calls are bitwise identical; with the same launch shape every
    batch column is computed on its own: batch 2 equals batch 1 on each
    column (both on activation digits), batch 8 equals batch 3 on the columns
    they share (both fp32), bitwise.  (The automatic shape may split K
    differently for batch 8, whose staged x is 8 times larger; the shape is
    therefore forced here.)"""
    say("gemv determinism")
    fmt, N, K = "q4_k", 1024, 2560
    W = dev(synth.quant_weights(fmt, N, K, SEED, tensor_id=31))
    x = synth.normal((8, K), SEED, tensor_id=32)
    xd = dev(x)
    a = qd.qgemv(fmt, W, xd).cpu().numpy()
    b = qd.qgemv(fmt, W, xd).cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    try:
        qd.set_launch_override(2, 2, 1)
        y8 = qd.qgemv(fmt, W, xd).cpu().numpy()
        y2 = qd.qgemv(fmt, W, dev(x[:2])).cpu().numpy()
        for col in range(2):
            y1 = qd.qgemv(fmt, W, dev(x[col])).cpu().numpy()
            assert np.array_equal(y1.view(np.uint32), y2[col].view(np.uint32)), col
        for lo in (0, 3, 5):
            y3 = qd.qgemv(fmt, W, dev(x[lo:lo + 3])).cpu().numpy()
            assert np.array_equal(y3.view(np.uint32), y8[lo:lo + 3].view(np.uint32)), lo
    finally:
        qd.set_launch_override(0, 0, 0)


# ---------------------------------------------------------------- FFN ---

def check_ffn(qd, fmt_gu, hidden, ff, batch, act, tag, with_norm=True, down=True):
    Wg = synth.quant_weights(fmt_gu, ff, hidden, SEED, tensor_id=41)
    Wu = synth.quant_weights(fmt_gu, ff, hidden, SEED, tensor_id=42)
    x = synth.normal((batch, hidden), SEED, tensor_id=43)
    nw = synth.normal((hidden,), SEED, tensor_id=44, mean=1.0, std=0.1)
    say(f"ffn {tag} gate/up {fmt_gu} {ff}x{hidden} batch={batch} act={act}")
    g = torch.empty((batch, ff), device="cuda")
    u = torch.empty((batch, ff), device="cuda")
    h = qd.qffn_gate_up_act(fmt_gu, dev(Wg), dev(Wu), dev(x), dev(nw) if with_norm else None,
                            1e-6, act, g_out=g, u_out=u)
    h, g, u = (t.cpu().numpy() for t in (h, g, u))
    xn = oracle.rmsnorm(x, nw, 1e-6) if with_norm else x.astype(np.float64)
    # the oracle takes fp32 x: the normalised x rounded to fp32 (an ulp-level
    # difference from fp64, far inside the bound)
    xn32 = xn.astype(np.float32)
    th = oracle.host_threads()
    g64, Sg = oracle.gemv_threaded(fmt_gu, Wg, xn32, ff, hidden, th)
    u64, Su = oracle.gemv_threaded(fmt_gu, Wu, xn32, ff, hidden, th)
    assert_bound(f"{tag} gate", g, g64, Sg)
    assert_bound(f"{tag} up", u, u64, Su)
    aid = oracle.ACT_GELU_TANH if act == "gelu_tanh" else oracle.ACT_SILU
    href = oracle.act_vec(aid, g64) * u64
    tol = h_tolerance(g64, u64, Sg, Su, aid)
    err = np.abs(h - href)
    assert (err <= tol).all(), f"{tag} h: worst {np.max(err / tol):.3f} of tolerance"
    if down:
        Wd = synth.quant_weights("q6_k", hidden, ff, SEED, tensor_id=45)
        say(f"ffn {tag} down q6_k {hidden}x{ff} batch={batch}")
        y = qd.qgemv_q6k(dev(Wd), dev(h)).cpu().numpy()
        yref, Sy = oracle.gemv_threaded("q6_k", Wd, h, hidden, ff, th)
        assert_bound(f"{tag} down", y, yref, Sy)


@pytest.mark.parametrize("act", ["gelu_tanh", "silu"])
@pytest.mark.parametrize("batch", [1, 5])
def test_ffn_small(qd, act, batch):
    check_ffn(qd, "q4_k", 512, 1280, batch, act, "small")


def test_ffn_without_norm_q8_0(qd):
    check_ffn(qd, "q8_0", 2560, 512, 2, "silu", "q8 no-norm", with_norm=False, down=False)


# ------------------------------------------------- workload configurations ---

def test_config_q4k_512x512(qd):
    say("config: Q4_K 512x512 batch 1")
    W = synth.quant_weights("q4_k", 512, 512, SEED, tensor_id=1)
    x = synth.normal((512,), SEED, tensor_id=2)
    y = qd.qgemv_q4k(dev(W), dev(x)).cpu().numpy()
    y64, S = oracle.gemv("q4_k", W, x, 512, 512)
    assert_bound("c0", y, y64[0], S[0])


def test_config_q6k_down_2560x10240(qd):
    say("config: Q6_K 2560x10240 batch 1")
    W = synth.quant_weights("q6_k", 2560, 10240, SEED, tensor_id=3)
    x = synth.normal((10240,), SEED, tensor_id=4)
    y = qd.qgemv_q6k(dev(W), dev(x)).cpu().numpy()
    y64, S = oracle.gemv("q6_k", W, x, 2560, 10240)
    assert_bound("c1", y, y64[0], S[0])


def test_config_gemma3_ffn(qd):
    check_ffn(qd, "q4_k", 2560, 10240, 1, "gelu_tanh", "gemma3-4b")


@pytest.mark.parametrize("variant", ["kquant", "q8_0"])
def test_config_gemma3_qkv_lm_head(qd, variant):
    K = 2560
    x = synth.normal((K,), SEED, tensor_id=5)
    xd = dev(x)
    fm = {"kquant": ("q4_k", "q4_k", "q6_k", "q4_k"), "q8_0": ("q8_0",) * 4}[variant]
    for name, fmt, N, tid in (("q", fm[0], 2048, 6), ("k", fm[1], 1024, 7), ("v", fm[2], 1024, 8),
                              ("o", fm[0], 2560, 9)):
        KK = 2048 if name == "o" else K
        xx = x[:KK] if name == "o" else x
        say(f"config: {variant} {name} {fmt} {N}x{KK}")
        W = synth.quant_weights(fmt, N, KK, SEED, tensor_id=tid)
        y = qd.qgemv(fmt, dev(W), dev(xx)).cpu().numpy()
        y64, S = oracle.gemv(fmt, W, xx, N, KK)
        assert_bound(f"{variant} {name}", y, y64[0], S[0])
    N = 262144
    say(f"config: {variant} lm_head {fm[3]} {N}x{K}")
    W = synth.quant_weights(fm[3], N, K, SEED, tensor_id=10)
    y = qd.qgemv(fm[3], dev(W), xd).cpu().numpy()
    y64, S = oracle.gemv_threaded(fm[3], W, x[None], N, K, oracle.host_threads())
    assert_bound(f"{variant} lm_head", y, y64[0], S[0])


@pytest.mark.parametrize("batch", [1, 8])
def test_config_gemma4_31b_ffn(qd, batch):
    check_ffn(qd, "q4_k", 5376, 21504, batch, "gelu_tanh", f"gemma4-31b b{batch}")


# ------------------------------------------------- whole decode FFN (one call) ---
# Repetitions alternate two inputs, so an h left over from the previous call
# cannot pass.

def check_ffn_decode(qd, fg, fd, hidden, ff, batch, act, tag, with_h=True, reps=3):
    """qffn_decode against the oracle chain, every output checked."""
    _check_ffn_decode(qd, fg, fd, hidden, ff, batch, act, tag, with_h, reps)


def _check_ffn_decode(qd, fg, fd, hidden, ff, batch, act, tag, with_h, reps):
    Wg = synth.quant_weights(fg, ff, hidden, SEED, tensor_id=51)
    Wu = synth.quant_weights(fg, ff, hidden, SEED, tensor_id=52)
    Wd = synth.quant_weights(fd, hidden, ff, SEED, tensor_id=53)
    nw = synth.normal((hidden,), SEED, tensor_id=55, mean=1.0, std=0.1)
    xs = [synth.normal((batch, hidden), SEED, tensor_id=54), synth.normal((batch, hidden), SEED, tensor_id=56)]
    aid = oracle.ACT_GELU_TANH if act == "gelu_tanh" else oracle.ACT_SILU
    refs = []
    for x in xs:
        xn32 = oracle.rmsnorm(x, nw, 1e-6).astype(np.float32)
        g64, Sg = oracle.gemv_threaded(fg, Wg, xn32, ff, hidden, oracle.host_threads())
        u64, Su = oracle.gemv_threaded(fg, Wu, xn32, ff, hidden, oracle.host_threads())
        refs.append((oracle.act_vec(aid, g64) * u64, h_tolerance(g64, u64, Sg, Su, aid)))
    dW = [dev(a) for a in (Wg, Wu, Wd, nw)]
    dx = [dev(x) for x in xs]
    firsts = [None, None]
    wabs = None
    for rep in range(reps):
        i = rep % 2
        say(f"ffn_decode {tag} {fg}->{fd} hidden={hidden} ff={ff} batch={batch} rep={rep}")
        href, tol = refs[i]
        h = torch.empty((batch, ff), device="cuda") if with_h else None
        y = qd.qffn_decode(fg, dW[0], dW[1], fd, dW[2], dx[i], dW[3], 1e-6, act, h_out=h)
        y = y.cpu().numpy()
        if with_h:
            hh = h.cpu().numpy()
            err = np.abs(hh - href)
            assert (err <= tol).all(), f"{tag} h: worst {np.max(err / tol):.3f} of tolerance"
            yref, Sy = oracle.gemv_threaded(fd, Wd, hh, hidden, ff, oracle.host_threads())
            assert_bound(f"{tag} y", y, yref, Sy)
        else:
            # y against the all-oracle chain: the bound of the down GEMV on the
            # exact h, widened by the h tolerance carried through |Wd|
            yref, Sy = oracle.gemv(fd, Wd, href.astype(np.float32), hidden, ff)
            if wabs is None:
                wabs = np.abs(oracle.dequant(fd, Wd, ff)).astype(np.float64)
            slack = tol @ wabs.T
            err = np.abs(y - yref)
            assert (err <= 1e-4 * Sy + 1e-6 + slack).all(), f"{tag} y vs chain"
        if firsts[i] is None:
            firsts[i] = y.copy()
        else:
            assert np.array_equal(firsts[i].view(np.uint32), y.view(np.uint32)), "not deterministic"


@pytest.mark.parametrize("fg,fd,act,batch", [
    ("q4_k", "q6_k", "gelu_tanh", 1), ("q4_k", "q6_k", "silu", 3), ("q4_k", "q4_k", "silu", 1),
    ("q8_0", "q8_0", "gelu_tanh", 2), ("q8_0", "q8_0", "silu", 1), ("q6_k", "q6_k", "gelu_tanh", 1),
    ("q6_k", "q4_k", "silu", 1)])
def test_ffn_decode_small(qd, fg, fd, act, batch):
    check_ffn_decode(qd, fg, fd, 512, 1536, batch, act, "small")


def test_ffn_decode_without_h_out(qd):
    check_ffn_decode(qd, "q4_k", "q6_k", 512, 1024, 1, "gelu_tanh", "no-h", with_h=False)


def test_ffn_decode_gemma3(qd):
    check_ffn_decode(qd, "q4_k", "q6_k", 2560, 10240, 1, "gelu_tanh", "gemma3-4b", reps=4)


def test_ffn_decode_gemma4_31b_batch1(qd):
    """Gemma-4-31B FFN at batch 1 (one workgroup per CU, four copying waves,
    ring slots reused), every output row checked."""
    check_ffn_decode(qd, "q4_k", "q6_k", 5376, 21504, 1, "gelu_tanh", "gemma4-31b b1", reps=2)


def test_ffn_decode_gemma4_31b_batch8(qd):
    """batch 8 x K = 5376: the register-streaming kernels, every row checked."""
    check_ffn_decode(qd, "q4_k", "q6_k", 5376, 21504, 8, "gelu_tanh", "gemma4-31b b8", reps=1)
