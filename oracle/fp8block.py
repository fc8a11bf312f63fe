"""Block-FP8 W8A8 GEMM for the lm-head (test infrastructure only).

Source: the Bitwise-consistent RL post, section 4.1 (dense GEMM: the deployment path is
W8A8 with block-FP8 weights; training quantizes the BF16 master weights to block FP8 by
the deployment rule and calls the same GEMM; one accumulation order for every M).  The
post names the scheme, not its constants; the readings here:

  * blocks: activations per row in groups of 128 consecutive K values (1 x 128),
    weights in 128 x 128 blocks (128 output columns x 128 K values);
  * scales: one power of two 2^e per group / block, e the smallest integer with
    amax <= 448 * 2^e (amax = the group's largest magnitude; e = 0 for an all-zero
    group), so x * 2^-e never exceeds the E4M3 range and scaling is exact.  The scale is
    an E8M0 value (the OCP microscaling scale format: a biased 8-bit exponent, 2^-127 to
    2^127, code 255 = NaN), so e is raised to -127 where it would fall below (groups whose
    largest magnitude is under 448 * 2^-128; bf16 values never need e > 120), and a group
    holding an infinity or NaN gets the NaN scale, which makes every product it enters NaN;
  * codes: e4m3(x * 2^-e), nearest even (oracle/fp8.py), of the bf16 values;
  * product: out[m, n] = sum over K of dequant(A)[m, k] * dequant(W)[n, k].  The GPU sums
    each 128-wide K block in one FP8 MFMA and adds the blocks in a fixed order per column;
    the oracle forms every scaled code product exactly in float64 (two 4-bit significands
    and a power of two) and adds them in float64.  That sum is exact while all partial
    sums fit 53 significant bits (the products' exponents spanning at most about 45
    binades, as for the operands here); beyond that it carries float64's rounding, some
    2^-53 relative per addition, far below the fp32 accumulation it is compared with.

Pinned by (tests/test_oracle_pins.py): the exponent rule against brute force (the clamp
and the NaN scale included), every code
inside the E4M3 range with the group maximum in its upper octave, the block structure
against an elementwise loop, and the GEMM of integer-valued operands against int64.
"""

from __future__ import annotations

import numpy as np

from .fp8 import e4m3_decode, e4m3_encode

GROUP = 128
E_MIN = -127        # the smallest E8M0 scale, 2^-127
E_NAN = 128         # the E8M0 NaN code (255) less the bias


def block_exponent(amax) -> np.ndarray:
    """Smallest integer e >= -127 with amax <= 448 * 2^e (0 where amax is 0, E_NAN where
    amax is not finite)."""
    a = np.asarray(amax, dtype=np.float64)
    fin = np.isfinite(a)
    m, E = np.frexp(np.where(fin, a, 1.0))   # a = m * 2^E, 0.5 <= m < 1
    e = E - 9 + (m > 0.875).astype(np.int64)  # 448 * 2^(E-9) = 0.875 * 2^E
    e = np.maximum(e, E_MIN)
    e = np.where(a > 0, e, 0)
    return np.where(fin, e, E_NAN).astype(np.int64)


def _scale(e):
    """2^e, NaN for the NaN scale."""
    e = np.asarray(e)
    return np.where(e == E_NAN, np.nan, np.ldexp(1.0, np.where(e == E_NAN, 0, e)))


def quantize_rows(x):
    """Per row, per 128-group along the last axis: (uint8 codes like x, int exponents
    [..., K/128])."""
    x = np.asarray(x, dtype=np.float64)
    K = x.shape[-1]
    assert K % GROUP == 0
    g = x.reshape(x.shape[:-1] + (K // GROUP, GROUP))
    e = block_exponent(np.max(np.abs(g), axis=-1))
    codes = e4m3_encode(np.ldexp(g, -np.where(e == E_NAN, 0, e)[..., None]))
    return codes.reshape(x.shape), e


def quantize_weight_blocks(w):
    """128 x 128 blocks of w [N, K]: (uint8 codes [N, K], int exponents [ceil(N/128), K/128])."""
    w = np.asarray(w, dtype=np.float64)
    N, K = w.shape
    assert K % GROUP == 0
    nb = -(-N // GROUP)
    pad = np.zeros((nb * GROUP, K))
    pad[:N] = w
    blocks = pad.reshape(nb, GROUP, K // GROUP, GROUP)
    e = block_exponent(np.max(np.abs(blocks), axis=(1, 3)))
    codes = e4m3_encode(np.ldexp(blocks, -np.where(e == E_NAN, 0, e)[:, None, :, None]))
    return codes.reshape(nb * GROUP, K)[:N], e


def dequant_rows(codes, e):
    c = np.asarray(codes)
    K = c.shape[-1]
    v = e4m3_decode(c).reshape(c.shape[:-1] + (K // GROUP, GROUP))
    return (v * _scale(e)[..., None]).reshape(c.shape)


def dequant_weight_blocks(codes, e):
    c = np.asarray(codes)
    N, K = c.shape
    v = e4m3_decode(c)
    rows = np.repeat(np.asarray(e), GROUP, axis=0)[:N]        # [N, K/128]
    return (v.reshape(N, K // GROUP, GROUP) * _scale(rows)[:, :, None]).reshape(N, K)


def w8a8_matmul(a, w) -> np.ndarray:
    """Product of the block-FP8 quantized a [M, K] and w [N, K] (float64 [M, N]): exact
    scaled code products summed in float64, exact while the partial sums fit 53 bits."""
    ca, ea = quantize_rows(a)
    cw, ew = quantize_weight_blocks(w)
    return dequant_rows(ca, ea) @ dequant_weight_blocks(cw, ew).T


def lm_head_logprob_w8a8(z, w_lm, target: int) -> float:
    """log_softmax of the W8A8 logits of one normalised row z at `target`."""
    logits = w8a8_matmul(np.asarray(z, dtype=np.float64)[None, :], w_lm)[0]
    mx = np.max(logits)
    return float(logits[target] - mx - np.log(np.sum(np.exp(logits - mx))))
