"""FP8 E4M3 storage for the KV cache (test infrastructure only).

Source: the Bitwise-consistent RL post, section 4.2 (FP8 KV cache: the cache keeps FP8
storage; one write path, and prefill, decode and the trainer's recompute all read it
through the same dequantization).  The post names FP8 storage but neither the exact
format nor its scaling; the readings here are:

  * format: the OCP 8-bit floating point E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits
    with bias 7, 3 mantissa bits; exponent field 0 holds the subnormals M * 2^-9; there
    are no infinities; S.1111.111 is NaN; the largest finite magnitude is 1.75 * 2^8 = 448;
  * scale: one power of two per tensor (K or V) of the model, 2^s with s an integer
    model constant (0 by default), so that the stored code is e4m3(x * 2^-s) and the
    value read back, code * 2^s, is exactly a bf16 value: dequantization adds no
    rounding of its own;
  * rounding: to nearest, ties to even; magnitudes beyond 448 saturate to 448 (the OCP
    "satfinite" conversion), infinities included; NaN stays NaN (sign kept).

Pinned by (tests/test_oracle_pins.py): codes fixed by the format's definition (448, 1,
-2, the subnormals, ties), torch's own float8_e4m3fn conversion on every bf16 value of
magnitude at most 464 (beyond which torch gives NaN instead of saturating), the decode of
all 256 codes against the field formula, round trips, and saturation cases.
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_encode(x) -> np.ndarray:
    """uint8 E4M3 codes of the float64 values x (round to nearest even, satfinite)."""
    x = np.asarray(x, dtype=np.float64)
    sign = np.signbit(x).astype(np.uint8) << 7
    nan = np.isnan(x)
    a = np.where(nan, 0.0, np.abs(x))
    # exponent of the leading bit, floored at the subnormal exponent -6; the spacing of
    # E4M3 values in [2^e, 2^(e+1)) is 2^(e-3)
    _, E = np.frexp(np.where(np.isinf(a), 1.0, a))
    e = np.maximum(E - 1, -6)
    q = np.ldexp(1.0, e - 3)
    v = np.rint(a / q) * q                    # np.rint: half to even
    v = np.where(np.isinf(a), np.inf, v)
    v = np.minimum(v, E4M3_MAX)               # satfinite
    # fields of the rounded magnitude v
    sub = v < 2.0 ** -6
    _, Ev = np.frexp(np.where(sub, 1.0, v))
    k = Ev - 1                                 # v = 2^k (1 + M/8) for normal v
    m_norm = np.rint((v / np.ldexp(1.0, k) - 1.0) * 8.0)
    m_sub = np.rint(v / 2.0 ** -9)
    ef = np.where(sub, 0, k + 7).astype(np.int64)
    mf = np.where(sub, m_sub, m_norm).astype(np.int64)
    code = (ef << 3) | mf
    code = np.where(nan, 0x7F, code)
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def e4m3_decode(codes) -> np.ndarray:
    """float64 values of uint8 E4M3 codes (NaN for S.1111.111)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    ef = (c >> 3) & 0xF
    mf = c & 7
    mag = np.where(ef == 0, mf * 2.0 ** -9, np.ldexp(1.0 + mf / 8.0, ef - 7))
    mag = np.where((ef == 15) & (mf == 7), np.nan, mag)
    return s * mag


def kv_fp8_store(x, scale_exp: int) -> np.ndarray:
    """The codes the FP8 cache holds for values x with scale 2^scale_exp."""
    return e4m3_encode(np.ldexp(np.asarray(x, dtype=np.float64), -int(scale_exp)))


def kv_fp8_load(codes, scale_exp: int) -> np.ndarray:
    """The values every phase reads back from those codes (exact in bf16)."""
    return np.ldexp(e4m3_decode(codes), int(scale_exp))


def kv_fp8_roundtrip(x, scale_exp: int = 0) -> np.ndarray:
    """x as it comes back from the FP8 cache: the K/V an FP8-cache model attends over."""
    return kv_fp8_load(kv_fp8_store(x, scale_exp), scale_exp)
