"""Elementary fp64 definitions used by the oracle (test infrastructure only).

Each function is the textbook definition written out in float64.  See the
package docstring for the sources and the rules on who may import this.
"""

from __future__ import annotations

import numpy as np


def widen(t) -> np.ndarray:
    """Exact float64 copy of a bf16/fp32 torch tensor or array (values unchanged)."""
    try:
        import torch  # local: only to accept torch tensors from the tests

        if isinstance(t, torch.Tensor):
            return t.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(t, dtype=np.float64)


def bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value, ties to even.

    Rounding is done directly from float64 (no detour through float32).
    bfloat16 keeps 8 significant bits and float32's exponent range: in the
    binade [2^e, 2^(e+1)) its spacing is 2^(e-7); below 2^-126 (subnormals)
    the spacing is 2^-133.  Values that round to 2^128 or beyond become inf.
    The round-to-nearest rule is the one the Bitwise-consistent RL post
    (section 4.4, condition 1) settles on for every quantization point.

    Pinned by: torch's fp32->bf16 conversion on fp32-representable values,
    hand-built ties and subnormals.
    """
    x = np.asarray(x, dtype=np.float64)
    _, E = np.frexp(x)                      # |x| = m * 2^E with 0.5 <= m < 1
    e = np.maximum(E - 1, -126)             # exponent of the leading bit, floored
    q = np.ldexp(1.0, e - 7)                # bf16 spacing near x
    r = np.rint(x / q) * q                  # np.rint rounds half to even
    r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, x), r)
    return np.where(np.isfinite(x), r, x)


def rmsnorm(x, gain=None, eps: float = 1e-6) -> np.ndarray:
    """y = x / sqrt(mean(x^2) + eps) * gain over the last axis (float64, unrounded).

    RMSNorm is one of the small operators the Bitwise-consistent RL post
    lists among the model's modules (section 3.1).  Pinned by: the constant
    vector closed form c/sqrt(c^2 + eps) and torch.nn.functional.rms_norm.
    """
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    y = x / np.sqrt(ms + eps)
    if gain is not None:
        y = y * np.asarray(gain, dtype=np.float64)
    return y


def log_softmax_at(logits, target: int) -> float:
    """log softmax(logits)[target] = l_t - (max + log sum exp(l - max)).

    The compared quantity of the method: the logprob of the sampled token
    (Bitwise-consistent RL post, section 2: diff is taken on the per-token
    logprob).  Pinned by: W = 0 gives exactly -ln(V); scipy's log_softmax;
    probabilities summing to 1; lp <= 0.
    """
    l = np.asarray(logits, dtype=np.float64)
    m = np.max(l)
    lse = m + np.log(np.sum(np.exp(l - m)))
    return float(l[int(target)] - lse)


def lm_head_logprob(z, w_lm, target: int, chunk: int = 16384) -> float:
    """Logprob of ``target`` under logits = z . W_lm^T (float64 logits, never rounded).

    ``w_lm`` is [vocab, d] (nn.Linear layout); it is widened to float64 one
    vocabulary chunk at a time to bound memory.  Pinned as log_softmax_at.
    """
    z = np.asarray(z, dtype=np.float64)
    V = w_lm.shape[0]
    logits = np.empty(V, dtype=np.float64)
    for c0 in range(0, V, chunk):
        c1 = min(V, c0 + chunk)
        wc = widen(w_lm[c0:c1])
        logits[c0:c1] = wc @ z
    return log_softmax_at(logits, target)


def attention_row(q, K, V, scale: float) -> np.ndarray:
    """Softmax attention of one query row over the keys it may see.

    o = sum_j p_j v_j with p = softmax(scale * q . k_j); float64 throughout.
    ``K`` is [n, dk], ``V`` is [n, dv].  Pinned by: one key gives v_0; equal
    keys give mean(V); torch's scaled_dot_product_attention in float64; a
    per-element Python loop on tiny inputs.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    s = scale * (K @ q)
    s = s - np.max(s)
    p = np.exp(s)
    p = p / np.sum(p)
    return p @ V


def projection(a, W, residual=None) -> np.ndarray:
    """A projection GEMM with its storage points: bf16(a W^T), or with a residual
    bf16(residual + bf16(a W^T)).

    ``a`` is [M, K] (or one row [K]) and ``W`` is [N, K] in the nn.Linear layout, both
    holding bf16 values.  Every product of two bf16 values is exact in float64 and the
    float64 sum over K is exact for integer-valued operands (and carries at most K
    float64 roundings otherwise, far below one bf16 step), so the value rounded is the
    dense product (Bitwise-consistent RL post, section 4.1: one accumulation order for
    every M; the order does not change this exact value).  Pinned by: integer operands
    against the int64 product; the residual form against an explicit torch float64
    composition.
    """
    y = bf16(np.asarray(a, dtype=np.float64) @ np.asarray(W, dtype=np.float64).T)
    if residual is not None:
        y = bf16(np.asarray(residual, dtype=np.float64) + y)
    return y


def silu(x) -> np.ndarray:
    """SiLU (swish): x * sigmoid(x) = x / (1 + exp(-x)), float64.

    Pinned by: torch.nn.functional.silu in float64, silu(0) = 0, and the odd part
    silu(x) - silu(-x) = x.
    """
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def swiglu_rounded_once(gate, up) -> np.ndarray:
    """bf16(SiLU(gate) * up): the product is formed unrounded and rounded once.

    The Bitwise-consistent RL post (section 4.4, condition 3) computes SiLU(gate) x up
    between the two GEMMs in FP32 and rounds only the product to BF16: rounding SiLU to
    BF16 before the multiply can move the result by one ulp.  Here the product is formed
    in float64 and rounded once.  Pinned by: torch's float64 silu composition, and a
    planted round-before-multiply variant that a test shows differing.
    """
    return bf16(silu(gate) * np.asarray(up, dtype=np.float64))
