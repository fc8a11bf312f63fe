"""Block-FP8 W8A8 GEMM for the lm-head (test infrastructure only).

Source: the Bitwise-consistent RL post, section 4.1 (dense GEMM: the deployment path is
W8A8 with block-FP8 weights; training quantizes the BF16 master weights to block FP8 by
the deployment rule and calls the same GEMM; one accumulation order for every M).  The
post names the scheme, not its constants; the readings here:

  * blocks: activations per row in groups of 128 consecutive K values (1 x 128),
    weights in 128 x 128 blocks (128 output columns x 128 K values);
  * scales: one power of two 2^e per group / block, e the smallest integer with
    amax <= 448 * 2^e (amax = the group's largest magnitude; e = 0 for an all-zero
    group), so x * 2^-e never exceeds the E4M3 range and scaling is exact;
  * codes: e4m3(x * 2^-e), nearest even (oracle/fp8.py), of the bf16 values;
  * product: out[m, n] = sum over K of dequant(A)[m, k] * dequant(W)[n, k].  The GPU sums
    each 128-wide K block in one FP8 MFMA and adds the blocks in a fixed order per column;
    the oracle's value is the exact sum (float64 of exactly representable products).

Pinned by (tests/test_oracle_pins.py): the exponent rule against brute force, every code
inside the E4M3 range with the group maximum in its upper octave, the block structure
against an elementwise loop, and the GEMM of integer-valued operands against int64.
"""

from __future__ import annotations

import numpy as np

from .fp8 import e4m3_decode, e4m3_encode

GROUP = 128


def block_exponent(amax) -> np.ndarray:
    """Smallest integer e with amax <= 448 * 2^e (0 where amax is 0)."""
    a = np.asarray(amax, dtype=np.float64)
    m, E = np.frexp(a)                       # a = m * 2^E, 0.5 <= m < 1
    e = E - 9 + (m > 0.875).astype(np.int64)  # 448 * 2^(E-9) = 0.875 * 2^E
    return np.where(a > 0, e, 0).astype(np.int64)


def quantize_rows(x):
    """Per row, per 128-group along the last axis: (uint8 codes like x, int exponents
    [..., K/128])."""
    x = np.asarray(x, dtype=np.float64)
    K = x.shape[-1]
    assert K % GROUP == 0
    g = x.reshape(x.shape[:-1] + (K // GROUP, GROUP))
    e = block_exponent(np.max(np.abs(g), axis=-1))
    codes = e4m3_encode(np.ldexp(g, -e[..., None]))
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
    codes = e4m3_encode(np.ldexp(blocks, -e[:, None, :, None]))
    return codes.reshape(nb * GROUP, K)[:N], e


def dequant_rows(codes, e):
    c = np.asarray(codes)
    K = c.shape[-1]
    v = e4m3_decode(c).reshape(c.shape[:-1] + (K // GROUP, GROUP))
    return np.ldexp(v, np.asarray(e)[..., None]).reshape(c.shape)


def dequant_weight_blocks(codes, e):
    c = np.asarray(codes)
    N, K = c.shape
    v = e4m3_decode(c)
    rows = np.repeat(np.asarray(e), GROUP, axis=0)[:N]        # [N, K/128]
    return np.ldexp(v.reshape(N, K // GROUP, GROUP), rows[:, :, None]).reshape(N, K)


def w8a8_matmul(a, w) -> np.ndarray:
    """Exact product of the block-FP8 quantized a [M, K] and w [N, K] (float64 [M, N])."""
    ca, ea = quantize_rows(a)
    cw, ew = quantize_weight_blocks(w)
    return dequant_rows(ca, ea) @ dequant_weight_blocks(cw, ew).T


def lm_head_logprob_w8a8(z, w_lm, target: int) -> float:
    """log_softmax of the W8A8 logits of one normalised row z at `target`."""
    logits = w8a8_matmul(np.asarray(z, dtype=np.float64)[None, :], w_lm)[0]
    mx = np.max(logits)
    return float(logits[target] - mx - np.log(np.sum(np.exp(logits - mx))))
