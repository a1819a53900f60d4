"""16-bit K/V storage: the value a stored word stands for (test infrastructure).

The pages define fp32 K/V pages only. Storing them as 16-bit words changes
the inputs, not the method: attention is then computed on the values the
words encode, so the oracle decodes each word exactly (every bfloat16 and
every IEEE binary16 value is a float32 value) and runs the fp32-input
oracle on the result.

* bfloat16: the word is the top half of an IEEE binary32 bit pattern
  (sign, 8 exponent bits, 7 fraction bits); the value is that binary32 with
  the low 16 bits zero.
* IEEE binary16: sign s, 5 exponent bits e (bias 15), 10 fraction bits f:
  e = 0 -> (-1)^s * 2^-14 * f / 1024 (zero and subnormals);
  0 < e < 31 -> (-1)^s * 2^(e - 15) * (1 + f / 1024);
  e = 31 -> +-inf (f = 0) or NaN.
"""
from __future__ import annotations

import numpy as np


def decode_bf16(bits) -> np.ndarray:
    """float32 values of bfloat16 words (any shape of uint16 / int16)."""
    w = np.asarray(bits).astype(np.uint16).astype(np.uint32)
    return (w << np.uint32(16)).view(np.float32)


def decode_fp16(bits) -> np.ndarray:
    """float32 values of IEEE binary16 words, from the field definition."""
    w = np.asarray(bits).astype(np.uint16).astype(np.int64)
    sign = np.where((w >> 15) & 1, -1.0, 1.0)
    e = (w >> 10) & 0x1F
    f = (w & 0x3FF).astype(np.float64)
    normal = sign * np.ldexp(1.0 + f / 1024.0, (e - 15).astype(np.int64))
    sub = sign * np.ldexp(f / 1024.0, -14)
    special = np.where(f == 0, sign * np.inf, np.nan)
    val = np.where(e == 0, sub, np.where(e == 31, special, normal))
    return val.astype(np.float32)


def decode_kv16(bits, fmt: str) -> np.ndarray:
    """Decode K/V words stored as ``fmt`` ("bf16" or "fp16") to float32."""
    if fmt == "bf16":
        return decode_bf16(bits)
    if fmt == "fp16":
        return decode_fp16(bits)
    raise ValueError(f"unknown 16-bit format {fmt!r}")
