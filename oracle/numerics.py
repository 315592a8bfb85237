"""Decoding of the stored number formats into float64 (oracle side; test infrastructure only).

The DSA pages say the lightning indexer runs in FP8 (page "A paper signed by Liang Wenfeng: The
most powerful open-source Agent model of DeepSeek has made a big splash" (36kr), section "02. Built
on the final version of DeepSeek-V3.1, DSA makes model computation smarter"; page "DeepSeek-V3.2:
Pushing the Frontier of Open Large Language Models" (paper digest), section "Key claims", paper
section 2.1). They do not name the format; the workloads fix OCP FP8 E4M3 (e4m3fn: no
infinities, 0x7F/0xFF are NaN, bias 7, largest finite 448).

Inputs are given already encoded; the oracle never quantises. Encodings:
  uint8   -> OCP FP8 e4m3fn code
  uint16  -> bfloat16 bit pattern (the upper half of an IEEE binary32)
  float32 / float64 -> IEEE value
"""
from __future__ import annotations

import numpy as np

_FP8_TABLE = None


def fp8_e4m3fn_table() -> np.ndarray:
    """Value of each of the 256 e4m3fn codes, built from the format's definition.

    code = s eeee mmm: normal (e > 0): (-1)^s * 2^(e-7) * (1 + m/8); subnormal (e == 0):
    (-1)^s * 2^(-6) * (m/8); e == 15 and m == 7 is NaN (no infinities in this format).
    """
    global _FP8_TABLE
    if _FP8_TABLE is None:
        t = np.empty(256, np.float64)
        for code in range(256):
            s = (code >> 7) & 1
            e = (code >> 3) & 0xF
            m = code & 0x7
            sign = -1.0 if s else 1.0
            if e == 0xF and m == 0x7:
                t[code] = np.nan
            elif e == 0:
                t[code] = sign * (2.0 ** -6) * (m / 8.0)
            else:
                t[code] = sign * (2.0 ** (e - 7)) * (1.0 + m / 8.0)
        _FP8_TABLE = t
    return _FP8_TABLE


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float64: the 16 bits are the high half of a binary32."""
    b = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def decode(x: np.ndarray) -> np.ndarray:
    """Stored tensor -> float64 by its numpy dtype (see the module docstring)."""
    x = np.asarray(x)
    if x.dtype == np.uint8:
        return fp8_e4m3fn_table()[x]
    if x.dtype == np.uint16:
        return bf16_bits_to_f64(x)
    if x.dtype in (np.float32, np.float64):
        return x.astype(np.float64)
    raise TypeError(f"unsupported stored dtype {x.dtype}")
