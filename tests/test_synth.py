"""The seeded generator: determinism, chunk independence and the field
distributions of the workloads (checked through the oracle's decoder)."""
import hashlib

import numpy as np

import oracle
import synth


def test_deterministic_and_seed_sensitive():
    a = synth.quant_weights("q4_k", 64, 512, seed=1)
    b = synth.quant_weights("q4_k", 64, 512, seed=1)
    c = synth.quant_weights("q4_k", 64, 512, seed=2)
    assert hashlib.sha256(a).digest() == hashlib.sha256(b).digest()
    assert not np.array_equal(a, c)
    x1 = synth.normal((3, 100), seed=9)
    x2 = synth.normal((3, 100), seed=9)
    assert np.array_equal(x1, x2)


def test_chunking_does_not_change_bytes():
    for fmt in ("q4_k", "q6_k", "q8_0"):
        K = 512
        a = synth.quant_weights(fmt, 37, K, seed=4)
        b = synth.quant_weights(fmt, 37, K, seed=4, row_chunk=5)
        assert np.array_equal(a, b)
        # a prefix of rows is the same as generating fewer rows
        c = synth.quant_weights(fmt, 10, K, seed=4)
        assert np.array_equal(a[:c.size], c)


def test_sizes():
    assert synth.quant_weights("q4_k", 3, 512).size == 3 * 2 * 144
    assert synth.quant_weights("q6_k", 3, 512).size == 3 * 2 * 210
    assert synth.quant_weights("q8_0", 3, 96).size == 3 * 3 * 34


def test_q4k_field_distributions():
    N, K = 256, 2560
    W = synth.quant_weights("q4_k", N, K, seed=5).reshape(-1, 144)
    d = W[:, 0:2].copy().view(np.float16).astype(np.float64).ravel()
    dm = W[:, 2:4].copy().view(np.float16).astype(np.float64).ravel()
    for v in (d, dm):
        assert v.min() >= 1e-3 * (1 - 2 ** -11) and v.max() <= 1e-2 * (1 + 2 ** -11)
        assert abs(v.mean() - 5.5e-3) < 2e-4
    sc = np.zeros(64, int)
    mn = np.zeros(64, int)
    for blk in W[:400]:
        for j in range(8):
            s, m = oracle.q4k_scale_min(blk, j)
            sc[s] += 1
            mn[m] += 1
    # 3200 draws over 64 values: every value appears, none dominates
    assert (sc > 10).all() and (mn > 10).all()
    assert sc.max() < 110 and mn.max() < 110
    nib = np.concatenate([W[:, 16:] & 15, W[:, 16:] >> 4]).ravel()
    counts = np.bincount(nib, minlength=16)
    assert counts.min() > 0.9 * counts.mean() and counts.max() < 1.1 * counts.mean()


def test_q6k_and_q8_0_field_distributions():
    W6 = synth.quant_weights("q6_k", 128, 2560, seed=6).reshape(-1, 210)
    sc = W6[:, 192:208].copy().view(np.int8).ravel()
    assert sc.min() == -64 and sc.max() == 63
    d = W6[:, 208:210].copy().view(np.float16).astype(np.float64).ravel()
    assert d.min() >= 1e-4 * (1 - 2 ** -11) and d.max() <= 1e-3 * (1 + 2 ** -11)
    W8 = synth.quant_weights("q8_0", 128, 2560, seed=7).reshape(-1, 34)
    q = W8[:, 2:].copy().view(np.int8).ravel()
    assert q.min() == -127 and q.max() == 127
    d8 = W8[:, 0:2].copy().view(np.float16).astype(np.float64).ravel()
    assert d8.min() >= 1e-3 * (1 - 2 ** -11) and d8.max() <= 1e-2 * (1 + 2 ** -11)


def test_normal_moments_and_bf16():
    x = synth.normal((200000,), seed=8)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01
    w = synth.normal((100000,), seed=9, mean=1.0, std=0.1)
    assert abs(w.mean() - 1) < 0.002 and abs(w.std() - 0.1) < 0.002
    xb = synth.normal_bf16((1000,), seed=8)
    back = (xb.astype(np.uint32) << 16).view(np.float32)
    x32 = synth.normal((1000,), seed=8)
    assert np.all(np.abs(back - x32) <= np.abs(x32) * 2 ** -8)
