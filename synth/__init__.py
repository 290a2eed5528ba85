"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module draws random numbers and lays them into block bytes at the field
offsets of each format.  It holds none of the method's arithmetic: it never
decodes a block, never unpacks a scale and never forms a product, so it can
serve both the CPU oracle and the GPU library without tying them together.

Generator (counter-based, stateless): SplitMix64's output function
(Steele, Lea & Flood, "Fast splittable pseudorandom number generators",
OOPSLA 2014) applied to ``key + (i + 1) * 0x9E3779B97F4A7C15``, where ``i``
is the element counter and ``key`` mixes the base seed, a tensor id and a
field id.  So any element can be regenerated on its own, and every field of
every tensor is an independent stream.

Distributions (those of the workloads this library is measured on):
  Q4_K  d, dmin ~ U[1e-3, 1e-2] rounded to f16 (nearest-even);
        8 six-bit scales and 8 six-bit mins ~ U{0..63}; quants ~ U{0..15}.
  Q6_K  quants ~ U{0..63}; 16 int8 scales ~ U{-64..63};
        d ~ U[1e-4, 1e-3] rounded to f16.
  Q8_0  d ~ U[1e-3, 1e-2] rounded to f16; int8 quants ~ U{-127..127}.
  activations x ~ N(0, 1) as fp32; RMS-norm weight ~ N(1, 0.1) as fp32;
  prefill activations ~ N(0, 1) rounded to bf16 (nearest-even).

How fields become bytes without any packing code: the twelve Q4_K scale/min
bytes hold 16 six-bit fields in 96 bits, every bit belonging to exactly one
field, so drawing the 12 bytes uniformly is the same distribution as drawing
the 16 fields uniformly and packing them.  The same holds for the 4-bit
quants (128 bytes = 256 nibbles) and for the Q6_K low/high quant bits
(192 bytes = 256 six-bit values).  Those regions are therefore uniform random
bytes; only whole-byte fields (f16 scales, int8 scales and quants) are drawn
as values.
"""
from __future__ import annotations

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

DEFAULT_SEED = 0x5EED

# bytes per block and values per block, and where the random fields sit
BLOCK = {"q4_k": (144, 256), "q6_k": (210, 256), "q8_0": (34, 32)}
FORMAT_IDS = {"q4_k": 0, "q6_k": 1, "q8_0": 2}
FORMAT_NAMES = {v: k for k, v in FORMAT_IDS.items()}

# field ids
_F_D, _F_DMIN, _F_BYTES, _F_SCALES, _F_QUANTS, _F_NORMAL = 1, 2, 3, 4, 5, 6


def _fmt_name(fmt) -> str:
    return FORMAT_NAMES[fmt] if isinstance(fmt, (int, np.integer)) else str(fmt).lower()


def _mix64(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        return z ^ (z >> np.uint64(31))


def _key(seed: int, tensor_id: int, field: int) -> np.uint64:
    a = _mix64(np.array([(tensor_id * 0x100 + field) & 0xFFFFFFFFFFFFFFFF], dtype=np.uint64))[0]
    return _mix64(np.array([np.uint64(seed & 0xFFFFFFFFFFFFFFFF) ^ a], dtype=np.uint64))[0]


def stream_u64(seed: int, tensor_id: int, field: int, n: int, offset: int = 0) -> np.ndarray:
    """n raw 64-bit draws of one field stream, elements offset..offset+n-1."""
    k = _key(seed, tensor_id, field)
    ctr = np.arange(offset + 1, offset + n + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix64(k + ctr * GAMMA)


def uniform01(u: np.ndarray) -> np.ndarray:
    """[0, 1) doubles from the top 53 bits."""
    return (u >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def uniform_int(u: np.ndarray, lo: int, hi: int) -> np.ndarray:
    """Integers in [lo, hi] by the multiply-shift of the top 32 bits."""
    span = np.uint64(hi - lo + 1)
    return (((u >> np.uint64(32)) * span) >> np.uint64(32)).astype(np.int64) + lo


def f16_bits(v: np.ndarray) -> np.ndarray:
    """float64 -> IEEE binary16 bits, round to nearest even (numpy's cast)."""
    return np.asarray(v, dtype=np.float64).astype(np.float16).view(np.uint16)


def bf16_bits(v: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bits, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def _u16_into(out, col, vals):
    out[:, col] = (vals & 0xFF).astype(np.uint8)
    out[:, col + 1] = (vals >> 8).astype(np.uint8)


def quant_weights(fmt, N: int, K: int, seed: int = DEFAULT_SEED, tensor_id: int = 0,
                  row_chunk: int = 16384) -> np.ndarray:
    """Row-major N x K quantized matrix as uint8 [N * row_bytes]."""
    name = _fmt_name(fmt)
    bb, qk = BLOCK[name]
    if K <= 0 or K % qk:
        raise ValueError(f"K={K} is not a positive multiple of {qk}")
    nb = K // qk
    out = np.empty((N * nb, bb), dtype=np.uint8)
    # generate in row chunks to bound host memory; the counter is global, so
    # the bytes do not depend on the chunking
    step = max(1, row_chunk)
    for r0 in range(0, N, step):
        r1 = min(N, r0 + step)
        b0, b1 = r0 * nb, r1 * nb
        nblk = b1 - b0
        o = out[b0:b1]
        if name == "q4_k":
            d = 1e-3 + uniform01(stream_u64(seed, tensor_id, _F_D, nblk, b0)) * 9e-3
            dm = 1e-3 + uniform01(stream_u64(seed, tensor_id, _F_DMIN, nblk, b0)) * 9e-3
            _u16_into(o, 0, f16_bits(d))
            _u16_into(o, 2, f16_bits(dm))
            o[:, 4:144] = _random_bytes_at(seed, tensor_id, _F_BYTES, b0, nblk, 140)
        elif name == "q6_k":
            o[:, 0:192] = _random_bytes_at(seed, tensor_id, _F_BYTES, b0, nblk, 192)
            sc = uniform_int(stream_u64(seed, tensor_id, _F_SCALES, nblk * 16, b0 * 16), -64, 63)
            o[:, 192:208] = sc.astype(np.int8).view(np.uint8).reshape(nblk, 16)
            d = 1e-4 + uniform01(stream_u64(seed, tensor_id, _F_D, nblk, b0)) * 9e-4
            _u16_into(o, 208, f16_bits(d))
        else:  # q8_0
            d = 1e-3 + uniform01(stream_u64(seed, tensor_id, _F_D, nblk, b0)) * 9e-3
            _u16_into(o, 0, f16_bits(d))
            q = uniform_int(stream_u64(seed, tensor_id, _F_QUANTS, nblk * 32, b0 * 32), -127, 127)
            o[:, 2:34] = q.astype(np.int8).view(np.uint8).reshape(nblk, 32)
    return out.reshape(-1)


def _random_bytes_at(seed, tensor_id, field, blk0, nblk, nbytes):
    words = (nbytes + 7) // 8
    u = stream_u64(seed, tensor_id, field, nblk * words, blk0 * words)
    return u.view(np.uint8).reshape(nblk, words * 8)[:, :nbytes]


def normal(shape, seed: int = DEFAULT_SEED, tensor_id: int = 0, mean: float = 0.0,
           std: float = 1.0) -> np.ndarray:
    """fp32 normal draws (Box-Muller in fp64, then rounded to fp32)."""
    n = int(np.prod(shape))
    u = stream_u64(seed, tensor_id, _F_NORMAL, 2 * n)
    u1 = ((u[0::2] >> np.uint64(11)).astype(np.float64) + 1.0) * (2.0 ** -53)  # (0, 1]
    u2 = uniform01(u[1::2])
    z = np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)
    return (mean + std * z).astype(np.float32).reshape(shape)


def normal_bf16(shape, seed: int = DEFAULT_SEED, tensor_id: int = 0) -> np.ndarray:
    """bf16 bits (uint16) of N(0, 1) draws rounded to nearest even."""
    return bf16_bits(normal(shape, seed, tensor_id)).reshape(shape)


def row_bytes(fmt, K: int) -> int:
    bb, qk = BLOCK[_fmt_name(fmt)]
    return (K // qk) * bb


# ------------------------------------------------------------- workloads ---
# Shapes of the layers the library is measured on: Gemma 3 4B (hidden 2560,
# 8 query heads x 256, 4 KV heads, vocab 262144; FFN intermediate 10240) and
# Gemma 4 31B (hidden 5376, FFN intermediate 21504), from the larql page's
# Gemma 3 and Gemma 4 tables.
GEMMA3_HIDDEN, GEMMA3_FF, GEMMA3_VOCAB = 2560, 10240, 262144
GEMMA3_Q, GEMMA3_KV = 8 * 256, 4 * 256
GEMMA4_HIDDEN, GEMMA4_FF = 5376, 21504
