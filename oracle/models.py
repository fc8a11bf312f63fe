"""Per-sequence fp64 forwards of the workloads (test infrastructure only).

Every function computes one sequence or one decode row alone.  Inputs are
the exact bf16 values (float64 arrays or torch tensors, widened exactly).
``bf16()`` is applied only at the contract's storage points: the projections'
outputs, the attention output, the residual sum and the normalised
activations.  Logits are float64 and never rounded.  Readings of points the
pages leave open are stated where they are used.
"""

from __future__ import annotations

import ctypes
import math

import numpy as np

from .numerics import attention_row, bf16, lm_head_logprob, log_softmax_at, rmsnorm, swiglu_rounded_once, widen
from .fp8block import lm_head_logprob_w8a8, w8a8_matmul


# ---------------------------------------------------------------------------
# One-layer decoder with token input
# ---------------------------------------------------------------------------

def _tiny_params(p):
    return {k: widen(v) for k, v in p.items()}


def _matmul(a, W, proj_w8a8: bool):
    """a W^T: exact in fp64 from the bf16 values, or (proj_w8a8) the exact product of the
    block-FP8 quantized operands (fp8block.w8a8_matmul: rows in 1 x 128 groups, the weight
    in 128 x 128 blocks, the deployment rule of the Bitwise-consistent RL post, section
    4.1).  a is [M, K] or one row [K]."""
    if not proj_w8a8:
        return a @ W.T
    return w8a8_matmul(np.atleast_2d(a), W).reshape(a.shape[:-1] + (W.shape[0],))


def _mlp(P, y, eps, proj_w8a8=False):
    """The SwiGLU block after the attention residual, when the parameters have one
    (w_gate_up [2F, d]: gate rows then up rows; w_down [d, F]; norm_mlp [d]):
        h = bf16(rms(y) g3);  [g|u] = bf16(h Wgu^T);  a = bf16(silu(g) u)  (rounded once)
        y' = bf16(y + bf16(a Wdown^T))
    Reading (the pages name the rounding of the activation, post section 4.4 condition 3,
    not the block): pre-norm residual MLP of the same form as the attention block."""
    if "w_gate_up" not in P:
        return y
    F = P["w_down"].shape[1]
    h = bf16(rmsnorm(y, P["norm_mlp"], eps))
    gu = bf16(_matmul(h, P["w_gate_up"], proj_w8a8))
    a = swiglu_rounded_once(gu[..., :F], gu[..., F:])
    return bf16(y + bf16(_matmul(a, P["w_down"], proj_w8a8)))


def tiny_decoder_prefill(params, tokens, targets, n_q_heads, n_kv_heads, head_dim,
                         eps=1e-6, proj_w8a8=False):
    """Full-sequence (prefill / trainer recompute) logprobs of a 1-layer decoder.

    The trainer recomputes each sampled token's logprob over the whole prefix
    in one pass (Bitwise-consistent RL post, section 2 and section 3.1).
    Reading of the layer (the pages name none): pre-norm residual block with
    no positional encoding, then a final RMSNorm and the lm-head:
        x = E[t];  h = bf16(rms(x) g1);  [q|k|v] = bf16(h Wqkv^T)
        o_i = bf16(softmax_j<=i(q_i . k_j / sqrt(D)) v)    (q head h -> kv head h*Hkv/Hq)
        y = bf16(x + bf16(o Wo^T));  [y = the SwiGLU block of _mlp, when present]
        z = bf16(rms(y) g2);  l = z Wlm^T;  lp_i = log_softmax(l_i)[targets[i]]
    proj_w8a8: every projection (Wqkv, Wo and the MLP's) is the block-FP8 W8A8 product
    (``_matmul``), its output rounded to bf16 as above.
    Returns float64 [L].  Pinned by: agreement with ``tiny_decoder_decode``
    (coded separately) to 1e-12; closed forms with zeroed weights.
    """
    P = _tiny_params(params)
    t = np.asarray(tokens, dtype=np.int64)
    L = len(t)
    Hq, Hkv, D = n_q_heads, n_kv_heads, head_dim
    group = Hq // Hkv
    x = P["embed"][t]
    h = bf16(rmsnorm(x, P["norm_attn"], eps))
    qkv = bf16(_matmul(h, P["w_qkv"], proj_w8a8))
    q = qkv[:, : Hq * D].reshape(L, Hq, D)
    k = qkv[:, Hq * D:(Hq + Hkv) * D].reshape(L, Hkv, D)
    v = qkv[:, (Hq + Hkv) * D:].reshape(L, Hkv, D)
    scale = 1.0 / math.sqrt(D)
    o = np.zeros((L, Hq, D))
    for i in range(L):
        for hh in range(Hq):
            g = hh // group
            o[i, hh] = attention_row(q[i, hh], k[: i + 1, g], v[: i + 1, g], scale)
    o = bf16(o).reshape(L, Hq * D)
    y = bf16(x + bf16(_matmul(o, P["w_o"], proj_w8a8)))
    y = _mlp(P, y, eps, proj_w8a8)
    z = bf16(rmsnorm(y, P["norm_final"], eps))
    logits = z @ P["w_lm"].T
    return np.array([log_softmax_at(logits[i], targets[i]) for i in range(L)])


def tiny_decoder_decode(params, tokens, targets, n_prompt, n_q_heads, n_kv_heads, head_dim,
                        eps=1e-6, proj_w8a8=False):
    """Rollout-side logprobs: a prompt pass of ``n_prompt`` tokens, then one token per step.

    Coded separately from ``tiny_decoder_prefill`` on purpose: an explicit
    per-position K/V cache, per-head loops and no whole-sequence matrices, so
    the two oracles only agree if both follow the same definition.  This is
    the oracle side of "whole-input processing matches token-by-token"
    (Bitwise-consistent RL post, section 5, step 2).  Returns float64 [L].
    """
    P = _tiny_params(params)
    Hq, Hkv, D = n_q_heads, n_kv_heads, head_dim
    t = [int(a) for a in np.asarray(tokens)]
    L = len(t)
    scale = 1.0 / math.sqrt(D)
    cache_k = [[] for _ in range(Hkv)]   # cache_k[g][pos] -> [D]
    cache_v = [[] for _ in range(Hkv)]
    lps = []

    def step(pos):
        x = P["embed"][t[pos]]
        h = bf16(rmsnorm(x, P["norm_attn"], eps))
        qkv = bf16(_matmul(h, P["w_qkv"], proj_w8a8) if proj_w8a8 else P["w_qkv"] @ h)
        for g in range(Hkv):
            cache_k[g].append(qkv[(Hq + g) * D:(Hq + g + 1) * D])
            cache_v[g].append(qkv[(Hq + Hkv + g) * D:(Hq + Hkv + g + 1) * D])
        return x, qkv

    def finish(pos, x, qkv):
        heads = []
        for hh in range(Hq):
            g = (hh * Hkv) // Hq
            qh = qkv[hh * D:(hh + 1) * D]
            Kc = np.stack(cache_k[g][: pos + 1])
            Vc = np.stack(cache_v[g][: pos + 1])
            s = np.array([scale * float(np.dot(qh, kj)) for kj in Kc])
            w = np.exp(s - s.max())
            heads.append((w[:, None] * Vc).sum(axis=0) / w.sum())
        o = bf16(np.concatenate(heads))
        mv = (lambda W, a: _matmul(a, W, True)) if proj_w8a8 else (lambda W, a: W @ a)  # noqa: E731
        y = bf16(x + bf16(mv(P["w_o"], o)))
        if "w_gate_up" in P:  # the same block, written per row with matrix-vector products
            F = P["w_down"].shape[1]
            h = bf16(rmsnorm(y, P["norm_mlp"], eps))
            gu = bf16(mv(P["w_gate_up"], h))
            g, u = gu[:F], gu[F:]
            a = bf16(g / (1.0 + np.exp(-g)) * u)
            y = bf16(y + bf16(mv(P["w_down"], a)))
        z = bf16(rmsnorm(y, P["norm_final"], eps))
        return log_softmax_at(P["w_lm"] @ z, targets[pos])

    # prompt pass: write every prompt token's K/V first, then attend causally
    prompt = [step(pos) for pos in range(min(n_prompt, L))]
    for pos, (x, qkv) in enumerate(prompt):
        lps.append(finish(pos, x, qkv))
    for pos in range(len(prompt), L):
        x, qkv = step(pos)
        lps.append(finish(pos, x, qkv))
    return np.array(lps)


# ---------------------------------------------------------------------------
# Attention rows with q/K/V given
# ---------------------------------------------------------------------------

def gqa_row_attention(q, K, V, scale: float) -> np.ndarray:
    """Grouped-query attention of one query position over its whole context.

    q [Hq, D]; K, V [n, Hkv, D] (positions 0..n-1, all visible).  Reading
    (the pages do not say): contiguous grouping, q head h reads kv head
    floor(h * Hkv / Hq).  Returns float64 [Hq, D] (unrounded).  Pinned by:
    per-kv-head constant values identify the grouping; torch SDPA in float64.
    """
    q = widen(q)
    K = widen(K)
    V = widen(V)
    Hq, Hkv = q.shape[0], K.shape[1]
    out = np.empty((Hq, V.shape[2]))
    for h in range(Hq):
        g = (h * Hkv) // Hq
        out[h] = attention_row(q[h], K[:, g], V[:, g], scale)
    return out


def gqa_row_logprob(q, K, V, scale, w_lm, target, eps=1e-6, w_o=None, gain=None, lm_w8a8=False) -> float:
    """Logprob of ``target`` for one decode row whose q/K/V are given.

    Reading of the head (the pages name none for this case): the attention
    output is stored as bf16, flattened head-major, optionally projected by
    ``w_o`` (bf16 output), normalised by RMSNorm (gain 1 unless given, bf16
    output) and fed to the lm-head; logits stay float64.
    """
    return head_logprob(gqa_row_attention(q, K, V, scale), w_lm, target, eps, w_o, gain, lm_w8a8)


def head_logprob(o, w_lm, target, eps=1e-6, w_o=None, gain=None, lm_w8a8=False, proj_w8a8=False) -> float:
    """The head after attention: bf16 attention output, flattened head-major, an
    optional projection (bf16 output; proj_w8a8: the block-FP8 W8A8 product of
    ``_matmul``), bf16(RMSNorm), then the lm-head logprob, with bf16 weights or
    (lm_w8a8) the block-FP8 W8A8 product of fp8block.py."""
    o = bf16(np.asarray(o, dtype=np.float64)).reshape(-1)
    if w_o is not None:
        o = bf16(_matmul(o, widen(w_o), True)) if proj_w8a8 else bf16(widen(w_o) @ o)
    z = bf16(rmsnorm(o, gain, eps))
    if lm_w8a8:
        return lm_head_logprob_w8a8(z, widen(w_lm), target)
    return lm_head_logprob(z, w_lm, target)


def mla_row_attention(q, C, scale: float, dv: int) -> np.ndarray:
    """Absorbed multi-head latent attention of one query position.

    All heads share one cached latent row per position (latent + rope part);
    scores use the full row, values use its first ``dv`` entries
    (Bitwise-consistent RL post, section 3: MLA compresses KV before caching).
    q [H, dqk], C [n, dqk] -> float64 [H, dv].
    """
    q = widen(q)
    C = widen(C)
    out = np.empty((q.shape[0], dv))
    for h in range(q.shape[0]):
        out[h] = attention_row(q[h], C, C[:, :dv], scale)
    return out


def indexer_scores(q_idx, K_idx) -> np.ndarray:
    """Lightweight indexer: one score per visible history position.

    The pages say only that an indexer scores every history position
    (Bitwise-consistent RL post, sections 3 and 4.3).  Reading: I[s] =
    sum_h relu(q_h . k_s) with unit head weights.  q [Hi, Di], K [n, Di] ->
    float64 [n].
    """
    q = widen(q_idx)
    K = widen(K_idx)
    return np.maximum(K @ q.T, 0.0).sum(axis=1)


def indexer_scores_fp32(q_idx, K_idx) -> np.ndarray:
    """The indexer in the precision the selection is decided in: float32, one fused
    multiply-add per term, accumulated in a fixed order.

    A top-k selection is an integer decided by floating point, so both sides must
    decide it in the same arithmetic (a one-ulp difference can swap a selected
    position, Bitwise-consistent RL post section 4.3).  The order: for head h = 0..63,
    acc_h = fma(q_h,D-1, k_D-1, ... fma(q_h1, k_1, fma(q_h0, k_0, +0))) over d = 0..D-1,
    each step the exact q k + acc rounded once to float32; then
    I = (((0 + relu(acc_0)) + relu(acc_1)) + ...) over h, one rounding per add.
    relu(x) = x if x > 0 else +0.  The loops run in C (oracle/indexer.c, C99 fmaf).
    q [Hi, D], K [n, D] (float32 values) -> float32 [n].  Pinned by: an exact-rational
    loop with round-to-nearest-even to float32 written from the definition, on random
    inputs and on inputs where a fused and an unfused step differ; agreement with
    indexer_scores within the fp32 bound.
    """
    from . import cbuild
    q = np.ascontiguousarray(np.asarray(widen(q_idx), dtype=np.float32))
    kt = np.ascontiguousarray(np.asarray(widen(K_idx), dtype=np.float32).T)
    heads, dim = q.shape
    n = kt.shape[1]
    assert kt.shape[0] == dim
    out = np.empty(n, dtype=np.float32)
    acc = np.empty(n, dtype=np.float32)
    fp = ctypes.POINTER(ctypes.c_float)
    cbuild.lib().oracle_indexer_fma(q.ctypes.data_as(fp), heads, dim, kt.ctypes.data_as(fp), n,
                                    out.ctypes.data_as(fp), acc.ctypes.data_as(fp))
    return out


def sparse_mla_row_attention(q, C, selected, scale: float, dv: int) -> np.ndarray:
    """MLA attention of one query over the selected history positions only (the list
    may be padded with -1).  The set is what matters in float64; the order the kernel
    accumulates in is the list order (descending position)."""
    sel = np.asarray(selected)
    sel = sel[sel >= 0]
    C = widen(C)
    return mla_row_attention(q, C[sel], scale, dv)


def topk_select(scores, k: int, tie: str = "lowest") -> np.ndarray:
    """Stable top-k: the k best (score, position) keys, listed by descending position.

    Selection ranks by score, then breaks exact ties by position: "lowest"
    keeps the smaller position (the rule this build is graded on), "highest"
    the larger one (the rule of the Bitwise-consistent RL post, section 4.3).
    The selected positions are then sorted by descending position and padded
    with -1 up to k (section 4.3: invalid entries last).  Returns int64 [k].
    Pinned by: the post's two-way tie example; brute-force ranking.
    """
    s = np.asarray(scores, dtype=np.float64)
    n = s.shape[0]
    pos = np.arange(n)
    if tie == "lowest":
        order = np.lexsort((pos, -s))
    elif tie == "highest":
        order = np.lexsort((-pos, -s))
    else:
        raise ValueError(tie)
    chosen = np.sort(order[: min(k, n)])[::-1]
    out = np.full(k, -1, dtype=np.int64)
    out[: chosen.shape[0]] = chosen
    return out
