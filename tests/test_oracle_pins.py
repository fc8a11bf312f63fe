"""Pins for the fp64 oracle: checks against what the pages and the mathematics fix.

Every check here is independent of the oracle's own code: closed forms,
library routines (torch's RNE conversion, scaled_dot_product_attention,
rms_norm, scipy's log_softmax), brute force on tiny inputs, invariants, and
the one worked example the pages print (the top-k tie caption).  The
``test_planted_*`` cases plant a plausible mistake into a copy of an oracle
function and assert that the matching pin rejects it.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

import oracle
from oracle import models as om
from oracle import numerics as on
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(12345)


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# pin checks (take the implementation under test as an argument)
# ---------------------------------------------------------------------------

def check_bf16(fn):
    """fn must equal torch's fp32 -> bf16 round-to-nearest-even on fp32 inputs."""
    x32 = np.concatenate([
        RNG.standard_normal(20000).astype(np.float32) * np.float32(10.0) ** RNG.integers(-30, 30, 20000).astype(np.float32),
        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 1.0 + 2 ** -8 + 2 ** -20,
                  2 ** -130, 3 * 2 ** -134, 2 ** -149, 0.0, -0.0, 65504.0, 3.3895314e38],
                 dtype=np.float32),
    ])
    ref = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    got = fn(x32.astype(np.float64))
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    return bool(np.all(same) and np.array_equal(np.signbit(got), np.signbit(ref)))


def check_rmsnorm(fn):
    g = _golden("closed_forms.json")["rmsnorm_constant"]
    y = fn(np.full(g["d"], g["c"]), None, g["eps"])
    if not np.allclose(y, g["expected"], rtol=0, atol=1e-15):
        return False
    x = RNG.standard_normal((5, 96))
    gain = RNG.standard_normal(96)
    ref = F.rms_norm(torch.from_numpy(x), (96,), torch.from_numpy(gain), eps=1e-6).numpy()
    return bool(np.allclose(fn(x, gain, 1e-6), ref, rtol=1e-13, atol=1e-13))


def check_log_softmax(fn):
    cf = _golden("closed_forms.json")["uniform_logprob"]
    if fn(np.zeros(2048), 7) != cf["vocab_2048"]:
        return False
    if abs(fn(np.zeros(129280), 129279) - cf["vocab_129280"]) > 1e-15:
        return False
    l = RNG.standard_normal(3000) * 4
    ref = scipy.special.log_softmax(l)
    got = np.array([fn(l, t) for t in range(0, 3000, 7)])
    if not np.allclose(got, ref[::7], rtol=0, atol=1e-12):
        return False
    full = np.array([fn(l, t) for t in range(3000)])
    return bool(abs(np.exp(full).sum() - 1.0) < 1e-12 and np.all(full <= 0))


def check_attention(fn):
    # one key -> its value exactly
    v0 = RNG.standard_normal((1, 8))
    if not np.array_equal(fn(RNG.standard_normal(8), RNG.standard_normal((1, 8)), v0, 0.3), v0[0]):
        return False
    # equal keys -> mean of values
    k = np.tile(RNG.standard_normal(8), (6, 1))
    V = RNG.standard_normal((6, 8))
    if not np.allclose(fn(RNG.standard_normal(8), k, V, 0.5), V.mean(0), atol=1e-14):
        return False
    # library routine: torch SDPA in float64 (scale passed explicitly)
    for n, dk, dv, sc in [(7, 16, 16, 0.25), (33, 64, 48, 1 / math.sqrt(64)), (5, 576, 512, 1 / math.sqrt(192))]:
        q = RNG.standard_normal(dk)
        K = RNG.standard_normal((n, dk))
        V = RNG.standard_normal((n, dv))
        ref = F.scaled_dot_product_attention(torch.from_numpy(q)[None, None, None],
                                             torch.from_numpy(K)[None, None],
                                             torch.from_numpy(V)[None, None], scale=sc)[0, 0, 0].numpy()
        if not np.allclose(fn(q, K, V, sc), ref, rtol=1e-12, atol=1e-12):
            return False
    # brute force: per-element Python loops
    q = RNG.standard_normal(3)
    K = RNG.standard_normal((4, 3))
    V = RNG.standard_normal((4, 2))
    s = [0.7 * sum(q[d] * K[j][d] for d in range(3)) for j in range(4)]
    e = [math.exp(x) for x in s]
    bf = [sum(e[j] * V[j][c] for j in range(4)) / sum(e) for c in range(2)]
    return bool(np.allclose(fn(q, K, V, 0.7), bf, rtol=1e-13, atol=1e-14))


def check_gqa_grouping(fn):
    """Each kv head holds a constant distinct value; q head h must read kv head h*Hkv//Hq."""
    Hq, Hkv, D, n = 8, 2, 4, 5
    K = RNG.standard_normal((n, Hkv, D))
    V = np.zeros((n, Hkv, D))
    for g in range(Hkv):
        V[:, g, :] = 10.0 * (g + 1)
    o = fn(RNG.standard_normal((Hq, D)), K, V, 0.5)
    want = np.array([[10.0 * (h * Hkv // Hq + 1)] * D for h in range(Hq)])
    return bool(np.allclose(o, want, atol=1e-12))


def check_topk(fn):
    g = _golden("topk_tie_example.json")
    s = np.full(g["n"], g["default_score"])
    for pos, val in g["scores"].items():
        s[int(pos)] = val
    if list(fn(s, g["k"], tie="highest")) != g["expected_larger_position_rule"]:
        return False
    if list(fn(s, g["k"], tie="lowest")) != g["expected_lowest_index_rule"]:
        return False
    p = g["k4_with_padding_n3"]
    if list(fn(np.array(p["scores"]), p["k"], tie="lowest")) != p["expected_lowest_index_rule"]:
        return False
    # brute force on small integer-valued scores (many ties)
    for n, k in [(40, 7), (100, 33), (16, 16), (9, 12)]:
        s = RNG.integers(0, 5, n).astype(np.float64)
        ranked = sorted(range(n), key=lambda j: (-s[j], j))[:k]
        want = sorted(ranked, reverse=True) + [-1] * (k - min(k, n))
        if list(fn(s, k, tie="lowest")) != want:
            return False
    return True


def check_tiny_prefill_vs_decode(prefill, decode):
    """Brute-force tiny decoders: prefill and token-by-token decode agree to 1e-12."""
    for (L, d, Hq, Hkv, D, V, n_prompt, seed) in [(9, 16, 2, 1, 8, 11, 3, 1), (12, 32, 4, 2, 8, 29, 1, 2),
                                                 (7, 16, 2, 2, 8, 13, 7, 3)]:
        r = np.random.default_rng(seed)
        p = {
            "embed": on.bf16(r.standard_normal((V, d)) * 0.5),
            "w_qkv": on.bf16(r.standard_normal(((Hq + 2 * Hkv) * D, d)) * 0.3),
            "w_o": on.bf16(r.standard_normal((d, Hq * D)) * 0.3),
            "norm_attn": np.ones(d), "norm_final": on.bf16(1 + 0.1 * r.standard_normal(d)),
            "w_lm": on.bf16(r.standard_normal((V, d)) * 0.3),
        }
        tok = r.integers(0, V, L)
        tgt = r.integers(0, V, L)
        a = prefill(p, tok, tgt, Hq, Hkv, D)
        b = decode(p, tok, tgt, n_prompt, Hq, Hkv, D)
        if a.shape != (L,) or not np.allclose(a, b, rtol=0, atol=1e-12):
            return False
    return True


# ---------------------------------------------------------------------------
# pins on the real oracle
# ---------------------------------------------------------------------------

def test_bf16_matches_torch_rne():
    assert check_bf16(oracle.bf16)


def test_bf16_direct_from_float64_ties():
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even -> 1; a hair above rounds up.
    assert oracle.bf16(1.0 + 2 ** -8) == 1.0
    assert oracle.bf16(1.0 + 2 ** -8 + 2 ** -40) == 1.0 + 2 ** -7
    assert oracle.bf16(1.0 + 3 * 2 ** -8) == 1.0 + 2 ** -6
    assert oracle.bf16(2.0 ** 200) == np.inf


def test_rmsnorm_pins():
    assert check_rmsnorm(oracle.rmsnorm)


def test_log_softmax_pins():
    assert check_log_softmax(oracle.log_softmax_at)


def test_lm_head_uniform_when_weights_zero():
    cf = _golden("closed_forms.json")["uniform_logprob"]
    z = oracle.bf16(RNG.standard_normal(256))
    assert oracle.lm_head_logprob(z, np.zeros((2048, 256), np.float32), 5, chunk=300) == cf["vocab_2048"]


def test_lm_head_integer_inputs_exact():
    # integer-valued logits: the float64 sum is exact, so lm_head_logprob equals the
    # closed form computed from an exact integer matmul.
    W = RNG.integers(-2, 3, (50, 64)).astype(np.float32)
    z = RNG.integers(-2, 3, 64).astype(np.float64)
    logits = (W.astype(np.int64) @ z.astype(np.int64)).astype(np.float64)
    want = float(logits[3] - scipy.special.logsumexp(logits))
    assert abs(oracle.lm_head_logprob(z, W, 3, chunk=7) - want) < 1e-12


def test_attention_pins():
    assert check_attention(oracle.attention_row)


def test_gqa_grouping_pin():
    assert check_gqa_grouping(oracle.gqa_row_attention)


def test_gqa_row_logprob_matches_sdpa_composition():
    # Attention via torch SDPA (enable_gqa) in float64, the rest as the contract says.
    Hq, Hkv, D, n, V = 8, 2, 16, 37, 300
    q = oracle.bf16(RNG.standard_normal((Hq, D)))
    K = oracle.bf16(RNG.standard_normal((n, Hkv, D)))
    Vv = oracle.bf16(RNG.standard_normal((n, Hkv, D)))
    W = oracle.bf16(RNG.standard_normal((V, Hq * D)) * 0.05)
    o = F.scaled_dot_product_attention(torch.from_numpy(q)[None, :, None],
                                       torch.from_numpy(K).permute(1, 0, 2)[None],
                                       torch.from_numpy(Vv).permute(1, 0, 2)[None],
                                       scale=0.25, enable_gqa=True)[0, :, 0].numpy()
    z = oracle.bf16(F.rms_norm(torch.from_numpy(oracle.bf16(o).reshape(-1)), (Hq * D,), eps=1e-6).numpy())
    want = float(torch.log_softmax(torch.from_numpy(W @ z), 0)[17])
    assert abs(oracle.gqa_row_logprob(q, K, Vv, 0.25, W, 17) - want) < 1e-12


def test_gqa_row_with_output_projection_zero():
    # W_o = 0 -> the normalised input is 0 -> uniform logprob.
    q = oracle.bf16(RNG.standard_normal((4, 8)))
    K = oracle.bf16(RNG.standard_normal((3, 2, 8)))
    lp = oracle.gqa_row_logprob(q, K, K, 0.3, RNG.standard_normal((2048, 16)), 9,
                                w_o=np.zeros((16, 32)))
    assert abs(lp - _golden("closed_forms.json")["uniform_logprob"]["vocab_2048"]) < 1e-12


def check_head_with_projection(fn):
    """fn(o, w_lm, target, eps, w_o) must equal the head composed from torch float64
    operations with the contract's bf16 points: bf16(o) flattened, bf16(W_o o),
    bf16(rms_norm(.)), log_softmax(W_lm z)[target]."""
    Hq, D, dh, V = 4, 16, 48, 333
    o = RNG.standard_normal((Hq, D))
    w_o = oracle.bf16(RNG.standard_normal((dh, Hq * D)) * 0.1)
    w_lm = oracle.bf16(RNG.standard_normal((V, dh)) * 0.3)
    ob = torch.from_numpy(oracle.bf16(o).reshape(-1))
    y = torch.from_numpy(oracle.bf16((torch.from_numpy(w_o) @ ob).numpy()))
    z = torch.from_numpy(oracle.bf16(F.rms_norm(y, (dh,), eps=1e-6).numpy()))
    for t in (0, 5, 332):
        want = float(torch.log_softmax(torch.from_numpy(w_lm) @ z, 0)[t])
        if abs(fn(o, w_lm, t, 1e-6, w_o) - want) > 1e-12:
            return False
    return True


def test_head_with_output_projection_matches_torch_composition():
    assert check_head_with_projection(lambda o, w, t, eps, w_o: oracle.head_logprob(o, w, t, eps, w_o=w_o))


def test_planted_projection_output_unrounded_is_caught():
    def bad(o, w_lm, t, eps, w_o):
        ob = oracle.bf16(np.asarray(o)).reshape(-1)
        z = oracle.bf16(on.rmsnorm(oracle.widen(w_o) @ ob, None, eps))  # bf16() after W_o dropped
        return on.lm_head_logprob(z, w_lm, t)
    assert not check_head_with_projection(bad)


def check_projection(fn):
    """fn(a, W, residual) on integer-valued bf16 operands must equal the int64 product
    rounded by torch's fp32 -> bf16 conversion (every value involved is an integer below
    2^24, so fp32 holds it exactly), with the residual added after that rounding and the
    sum rounded again; checked for K spanning several tile widths."""
    for M, N, K in ((3, 5, 32), (17, 40, 96), (9, 7, 1024)):
        # integers up to 40 in magnitude are bf16 values; products up to 1600 and sums up
        # to 1600 K < 2^24 stay exact in fp32, and most sums need the bf16 rounding
        a = RNG.integers(-40, 41, (M, K))
        W = RNG.integers(-40, 41, (N, K))
        R = RNG.integers(-3000, 3001, (M, N)) // 16 * 16  # bf16 values (8 significant bits)
        p = a.astype(np.int64) @ W.astype(np.int64).T
        pb = torch.from_numpy(p.astype(np.float32)).to(torch.bfloat16).to(torch.float32)
        want = pb.to(torch.float64).numpy()
        want_r = (torch.from_numpy(R.astype(np.float32)) + pb).to(torch.bfloat16).to(torch.float64).numpy()
        got, got_r = fn(a.astype(np.float64), W.astype(np.float64), None), fn(a, W, R)
        if not (np.array_equal(got, want) and np.array_equal(got_r, want_r)):
            return False
    return True


def test_projection_integer_operands_exact():
    assert check_projection(on.projection)


def test_planted_projection_rounded_once_with_residual_is_caught():
    def bad(a, W, R):
        y = np.asarray(a, dtype=np.float64) @ np.asarray(W, dtype=np.float64).T
        return oracle.bf16(y if R is None else y + R)  # the inner bf16 before the residual dropped
    assert not check_projection(bad)


def test_planted_projection_transposed_weight_is_caught():
    def bad(a, W, R):
        W = np.asarray(W, dtype=np.float64)
        return on.projection(a, W.reshape(W.shape[1], W.shape[0]).T, R)  # a wrong index map
    assert not check_projection(bad)


def test_mla_matches_sdpa():
    H, dqk, dv, n = 3, 576, 512, 19
    q = oracle.bf16(RNG.standard_normal((H, dqk)))
    C = oracle.bf16(RNG.standard_normal((n, dqk)))
    sc = 1 / math.sqrt(192)
    ref = F.scaled_dot_product_attention(torch.from_numpy(q)[:, None], torch.from_numpy(C)[None].expand(H, n, dqk),
                                         torch.from_numpy(C[:, :dv])[None].expand(H, n, dv), scale=sc)[:, 0].numpy()
    assert np.allclose(oracle.mla_row_attention(q, C, sc, dv), ref, rtol=1e-12, atol=1e-12)


def test_indexer_brute_force():
    q = RNG.standard_normal((3, 4))
    K = RNG.standard_normal((6, 4))
    want = [sum(max(0.0, sum(q[h][d] * K[s][d] for d in range(4))) for h in range(3)) for s in range(6)]
    assert np.allclose(oracle.indexer_scores(q, K), want, rtol=1e-14, atol=1e-14)


def _round_f32(x: Fraction) -> float:
    """x rounded to the nearest binary32 value, ties to the even significand, written from
    the format's definition (24-bit significands, exponents down to -126, subnormals on a
    2^-149 grid); the inputs here stay far from overflow."""
    if x == 0:
        return 0.0
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1  # now 2^e <= a < 2^(e+1)
    quantum = Fraction(2) ** (max(e, -126) - 23)
    m = a / quantum
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    v = float(fl * quantum)
    return v if x > 0 else -v


def _indexer_exact_rational(q, K):
    """The indexer's float32 chain with every step's exact value taken as a rational:
    acc <- round(q k + acc) per term, total <- round(total + relu(acc)) per head."""
    out = []
    for s in range(K.shape[0]):
        tot = 0.0
        for h in range(q.shape[0]):
            acc = 0.0
            for d in range(q.shape[1]):
                acc = _round_f32(Fraction(float(q[h, d])) * Fraction(float(K[s, d])) + Fraction(acc))
            tot = _round_f32(Fraction(tot) + Fraction(acc if acc > 0 else 0.0))
        out.append(tot)
    return np.array(out, dtype=np.float32)


def test_round_f32_agrees_with_numpy_conversion():
    # the rounding helper itself: on doubles, numpy's float64 -> float32 conversion is RNE
    x = np.concatenate([RNG.standard_normal(2000), RNG.standard_normal(200) * 1e-40,
                        np.array([1 + 2.0 ** -24, 1 + 3 * 2.0 ** -24, -(1 + 2.0 ** -24), 2.0 ** -150, 3 * 2.0 ** -150])])
    want = x.astype(np.float32)
    got = np.array([_round_f32(Fraction(float(v))) for v in x], dtype=np.float32)
    assert np.array_equal(got, want)


def test_indexer_fp32_brute_force_exact_rational():
    q = RNG.standard_normal((3, 9)).astype(np.float32)
    K = RNG.standard_normal((11, 9)).astype(np.float32)
    got = oracle.indexer_scores_fp32(q, K)
    assert got.dtype == np.float32 and np.array_equal(got, _indexer_exact_rational(q, K))


def _fused_differs_case():
    # d = 0: acc = -1; d = 1: (1 + 2^-12)^2 - 1 = 2^-11 + 2^-24 exactly (representable);
    # an unfused step first rounds the product 1 + 2^-11 + 2^-24 (a tie) to 1 + 2^-11
    a = np.float32(1 + 2.0 ** -12)
    q = np.array([[1.0, a], [0.5, 0.25]], dtype=np.float32)
    K = np.array([[-1.0, a], [2.0, 4.0]], dtype=np.float32)
    return q, K


def test_indexer_fp32_steps_are_fused():
    q, K = _fused_differs_case()
    got = oracle.indexer_scores_fp32(q, K)
    assert got[0] == np.float32(2.0 ** -11 + 2.0 ** -24)  # head 1 scores -0.25 + 2^-14: relu 0
    assert np.array_equal(got, _indexer_exact_rational(q, K))


def test_planted_indexer_unfused_steps_are_caught():
    # a plausible slip: multiply, round, then add (two roundings per term)
    def unfused(q, K):
        tot = np.zeros(K.shape[0], dtype=np.float32)
        for h in range(q.shape[0]):
            acc = np.zeros(K.shape[0], dtype=np.float32)
            for d in range(q.shape[1]):
                acc = acc + q[h, d] * K[:, d]
            tot = tot + np.where(acc > 0, acc, np.float32(0))
        return tot
    q, K = _fused_differs_case()
    assert not np.array_equal(unfused(q, K), _indexer_exact_rational(q, K))


def test_indexer_fp32_within_error_bound_of_fp64():
    # |fl32 - exact| <= gamma_n * sum_h sum_d |q_hd k_d| with n = D + H (sequential sums)
    q = RNG.standard_normal((64, 128)).astype(np.float32)
    K = RNG.standard_normal((300, 128)).astype(np.float32)
    exact = oracle.indexer_scores(q, K)
    got = oracle.indexer_scores_fp32(q, K).astype(np.float64)
    u = 2.0 ** -24
    n = 128 + 64
    bound = (n * u / (1 - n * u)) * (np.abs(K.astype(np.float64)) @ np.abs(q.astype(np.float64)).T).sum(1)
    assert np.all(np.abs(got - exact) <= bound)


def test_sparse_mla_equals_dense_over_selection():
    q = oracle.bf16(RNG.standard_normal((2, 576)))
    C = oracle.bf16(RNG.standard_normal((40, 576)))
    sel = np.array([31, 17, 5, 2, -1, -1])
    sc = 1 / math.sqrt(192)
    got = oracle.sparse_mla_row_attention(q, C, sel, sc, 512)
    want = oracle.mla_row_attention(q, C[[31, 17, 5, 2]], sc, 512)
    assert np.allclose(got, want, rtol=0, atol=1e-15)
    # all positions selected == dense attention
    assert np.allclose(oracle.sparse_mla_row_attention(q, C, np.arange(40)[::-1], sc, 512),
                       oracle.mla_row_attention(q, C, sc, 512), rtol=1e-13, atol=1e-14)


def test_topk_pins():
    assert check_topk(oracle.topk_select)


def test_tiny_decoder_prefill_equals_decode():
    assert check_tiny_prefill_vs_decode(oracle.tiny_decoder_prefill, oracle.tiny_decoder_decode)


def test_tiny_decoder_zero_projection_closed_form():
    # Wq = Wk = 0 -> uniform attention; W_o = 0 -> y = x; then z = bf16(rms(E[t])) and the
    # logprob is the plain log-softmax of z . W_lm, checked with scipy.
    w = wl.TinyDecoder(d_model=32, n_q_heads=2, n_kv_heads=2, head_dim=8, vocab=40, lengths=(6,))
    p = {k: oracle.widen(v) for k, v in wl.tiny_weights(w).items()}
    p["w_o"] = np.zeros_like(p["w_o"])
    tok = np.array([3, 1, 4, 1, 5, 9])
    tgt = np.array([1, 4, 1, 5, 9, 2])
    lp = oracle.tiny_decoder_prefill(p, tok, tgt, 2, 2, 8)
    z = oracle.bf16(oracle.bf16(p["embed"][tok]) / np.sqrt(np.mean(p["embed"][tok] ** 2, 1, keepdims=True) + 1e-6))
    ref = scipy.special.log_softmax(z @ p["w_lm"].T, axis=1)[np.arange(6), tgt]
    assert np.allclose(lp, ref, rtol=0, atol=1e-12)


def test_metrics_closed_forms():
    cf = _golden("closed_forms.json")["k3"]
    a = RNG.standard_normal(100)
    s = oracle.diff_stats(a, a)
    assert s["max"] == s["mean"] == s["std"] == s["p_max"] == 0.0
    assert oracle.k3_mean(a, a) == 0.0
    assert abs(oracle.k3_mean(np.array([math.log(2.0)]), np.array([0.0])) - cf["delta_ln2"]) < 1e-15
    d = oracle.diff_stats(np.array([0.0, -1.0]), np.array([-0.5, -1.0]))
    assert d["max"] == 0.5 and d["mean"] == 0.25 and d["std"] == 0.25


# ---------------------------------------------------------------------------
# planted mistakes: each pin must reject a plausible bug
# ---------------------------------------------------------------------------

def test_planted_bf16_truncation_is_caught():
    def trunc(x):
        x = np.asarray(x, np.float64)
        _, E = np.frexp(x)
        q = np.ldexp(1.0, np.maximum(E - 1, -126) - 7)
        return np.trunc(x / q) * q
    assert not check_bf16(trunc)


def test_planted_bf16_via_float16_is_caught():
    with np.errstate(over='ignore'):
        assert not check_bf16(lambda x: np.asarray(x, np.float16).astype(np.float64))


def test_planted_rmsnorm_without_eps_is_caught():
    def bad(x, gain=None, eps=1e-6):
        return on.rmsnorm(x, gain, 0.0)
    assert not check_rmsnorm(bad)


def test_planted_rmsnorm_mean_abs_is_caught():
    def bad(x, gain=None, eps=1e-6):
        x = np.asarray(x, np.float64)
        y = x / (np.mean(np.abs(x), -1, keepdims=True) + eps)
        return y if gain is None else y * gain
    assert not check_rmsnorm(bad)


def test_planted_log_softmax_missing_max_shift_sign_is_caught():
    def bad(l, t):
        l = np.asarray(l, np.float64)
        m = l.max()
        return float(l[t] - m - np.log(np.sum(np.exp(l + m))))
    assert not check_log_softmax(bad)


def test_planted_attention_wrong_scale_is_caught():
    assert not check_attention(lambda q, K, V, sc: on.attention_row(q, K, V, sc * sc))


def test_planted_attention_values_from_keys_is_caught():
    def bad(q, K, V, sc):
        K = np.asarray(K, np.float64)
        return on.attention_row(q, K, K[:, : np.shape(V)[1]], sc)
    assert not check_attention(bad)


def test_planted_attention_softmax_without_normalisation_is_caught():
    def bad(q, K, V, sc):
        s = sc * (np.asarray(K) @ np.asarray(q))
        return np.exp(s - s.max()) @ np.asarray(V)
    assert not check_attention(bad)


def test_planted_interleaved_grouping_is_caught():
    def bad(q, K, V, sc):
        q, K, V = map(np.asarray, (q, K, V))
        return np.stack([on.attention_row(q[h], K[:, h % K.shape[1]], V[:, h % K.shape[1]], sc)
                         for h in range(q.shape[0])])
    assert not check_gqa_grouping(bad)


def test_planted_topk_reversed_tie_is_caught():
    def bad(s, k, tie="lowest"):
        return om.topk_select(s, k, tie={"lowest": "highest", "highest": "lowest"}[tie])
    assert not check_topk(bad)


def test_planted_topk_ascending_order_is_caught():
    def bad(s, k, tie="lowest"):
        out = om.topk_select(s, k, tie)
        v = np.sort(out[out >= 0])
        return np.concatenate([v, out[out < 0]])
    assert not check_topk(bad)


def test_planted_causal_off_by_one_is_caught():
    def bad_prefill(params, tokens, targets, Hq, Hkv, D, eps=1e-6):
        # attends to one position fewer than allowed (excludes itself)
        real = on.attention_row

        def shifted(q, K, V, sc):
            return real(q, K[:-1], V[:-1], sc) if K.shape[0] > 1 else real(q, K, V, sc)
        om.attention_row = shifted
        try:
            return om.tiny_decoder_prefill(params, tokens, targets, Hq, Hkv, D, eps)
        finally:
            om.attention_row = real
    assert not check_tiny_prefill_vs_decode(bad_prefill, oracle.tiny_decoder_decode)


def test_planted_residual_dropped_is_caught():
    def bad_decode(params, tokens, targets, n_prompt, Hq, Hkv, D, eps=1e-6):
        p = dict(params)
        p["w_o"] = np.asarray(params["w_o"]) * 0.0
        return om.tiny_decoder_decode(p, tokens, targets, n_prompt, Hq, Hkv, D, eps)
    assert not check_tiny_prefill_vs_decode(oracle.tiny_decoder_prefill, bad_decode)


# ---------------------------------------------------------------------------
# FP8 E4M3 storage of the KV cache (oracle/fp8.py)
# ---------------------------------------------------------------------------

from oracle import fp8 as of8  # noqa: E402


def _all_bf16_values():
    bits = torch.arange(0, 1 << 16, dtype=torch.int32).to(torch.int16)
    return bits.view(torch.bfloat16).to(torch.float64).numpy()


def test_e4m3_codes_fixed_by_the_format():
    cases = [(1.0, 0x38), (448.0, 0x7E), (-2.0, 0xC0), (0.5, 0x30), (3.0, 0x44), (2.0 ** -6, 0x08),
             (2.0 ** -9, 0x01), (7 * 2.0 ** -9, 0x07), (2.0 ** -4, 0x18), (240.0, 0x77), (-448.0, 0xFE),
             (0.0, 0x00), (-0.0, 0x80),
             (1.0625, 0x38),            # tie between 1 (M=0) and 1.125 (M=1): even
             (1.1875, 0x3A),            # tie between 1.125 (M=1) and 1.25 (M=2): even
             (2.0 ** -10, 0x00),        # tie between 0 and 2^-9: even (0)
             (3 * 2.0 ** -10, 0x02),    # tie between 2^-9 and 2^-8: even
             (1.0625 + 2.0 ** -20, 0x39),
             (464.0, 0x7E), (465.0, 0x7E), (1e30, 0x7E), (np.inf, 0x7E), (-np.inf, 0xFE)]  # satfinite
    got = of8.e4m3_encode(np.array([v for v, _ in cases]))
    assert [int(c) for c in got] == [c for _, c in cases]
    assert int(of8.e4m3_encode(np.array([np.nan]))[0]) & 0x7F == 0x7F


def test_e4m3_decode_all_codes_by_field_formula():
    vals = of8.e4m3_decode(np.arange(256, dtype=np.uint8))
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            assert np.isnan(vals[c])
            continue
        mag = m * 2.0 ** -9 if e == 0 else 2.0 ** (e - 7) * (1 + m / 8)
        assert vals[c] == (-mag if s else mag), c
    pos = vals[:127]
    assert np.all(np.diff(pos) > 0) and pos[-1] == 448.0


def test_e4m3_roundtrip_of_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert np.array_equal(of8.e4m3_encode(of8.e4m3_decode(codes)), codes)


def test_e4m3_matches_torch_on_every_bf16_value_within_range():
    x = _all_bf16_values()
    keep = np.isfinite(x) & (np.abs(x) <= 464.0)
    ref = torch.from_numpy(x[keep]).to(torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(of8.e4m3_encode(x[keep]), ref)


def test_e4m3_is_nearest_with_even_ties():
    pos = of8.e4m3_decode(np.arange(127, dtype=np.uint8))  # 0 .. 448
    mids = (pos[:-1] + pos[1:]) / 2
    lo_even = (np.arange(126) % 2) == 0                    # code parity = mantissa parity
    want = np.where(lo_even, np.arange(126), np.arange(1, 127))
    assert np.array_equal(of8.e4m3_encode(mids), want)
    eps = np.minimum(np.diff(pos), 1.0) * 1e-3
    assert np.array_equal(of8.e4m3_encode(mids - eps), np.arange(126))
    assert np.array_equal(of8.e4m3_encode(mids + eps), np.arange(1, 127))


def test_kv_fp8_scale_is_exact_power_of_two():
    x = _all_bf16_values()
    x = x[np.isfinite(x) & (np.abs(x) < 1e3)]
    for s in (-3, 0, 2):
        assert np.array_equal(of8.kv_fp8_store(x, s), of8.e4m3_encode(x * 2.0 ** -s))
        back = of8.kv_fp8_roundtrip(x, s)
        assert np.array_equal(back, of8.e4m3_decode(of8.e4m3_encode(x * 2.0 ** -s)) * 2.0 ** s)
        assert np.array_equal(on.bf16(back[np.isfinite(back)]), back[np.isfinite(back)])  # bf16-exact


def test_planted_e4m3_truncation_is_caught():
    # a planted mistake: truncating instead of rounding must break a pin
    x = np.array([1.0625 + 2.0 ** -20, 1.1875])
    trunc = np.floor(x * 8) / 8
    assert not np.array_equal(of8.e4m3_encode(trunc), of8.e4m3_encode(x))


# ---------------------------------------------------------------------------
# SwiGLU MLP block, activation rounded once (oracle/numerics.py, oracle/models.py)
# ---------------------------------------------------------------------------

def test_silu_pins():
    x = np.linspace(-30, 30, 2001)
    ref = F.silu(torch.from_numpy(x)).numpy()
    assert np.allclose(on.silu(x), ref, rtol=1e-15, atol=1e-300)
    assert on.silu(0.0) == 0.0
    assert np.allclose(on.silu(x) - on.silu(-x), x, rtol=0, atol=1e-12)


def test_swiglu_rounds_once_and_round_before_multiply_differs():
    rng = np.random.default_rng(3)
    g = on.bf16(rng.normal(size=20000))
    u = on.bf16(rng.normal(size=20000))
    once = on.swiglu_rounded_once(g, u)
    assert np.array_equal(once, on.bf16(F.silu(torch.from_numpy(g)).numpy() * u))
    twice = on.bf16(on.bf16(on.silu(g)) * u)   # the pitfall the pages name
    assert np.any(once != twice)


def test_tiny_decoder_with_mlp_prefill_equals_decode():
    W = wl.TINY_MLP
    wts = wl.tiny_weights(W)
    t = wl.tiny_tokens(0, W).numpy()[:40]
    tg = np.roll(t, -1)
    a = oracle.tiny_decoder_prefill(wts, t, tg, W.n_q_heads, W.n_kv_heads, W.head_dim, W.rms_eps)
    b = oracle.tiny_decoder_decode(wts, t, tg, W.prompt_tokens, W.n_q_heads, W.n_kv_heads, W.head_dim,
                                   W.rms_eps)
    assert np.max(np.abs(a - b)) <= 1e-12


def test_tiny_decoder_mlp_with_zero_down_projection_is_the_plain_decoder():
    W = wl.TINY_MLP
    wts = wl.tiny_weights(W)
    t = wl.tiny_tokens(1, W).numpy()[:24]
    tg = np.roll(t, -1)
    z = dict(wts, w_down=torch.zeros_like(wts["w_down"]))
    plain = {k: v for k, v in wts.items() if k not in ("w_gate_up", "w_down", "norm_mlp")}
    a = oracle.tiny_decoder_prefill(z, t, tg, W.n_q_heads, W.n_kv_heads, W.head_dim, W.rms_eps)
    b = oracle.tiny_decoder_prefill(plain, t, tg, W.n_q_heads, W.n_kv_heads, W.head_dim, W.rms_eps)
    assert np.array_equal(a, b)
    full = oracle.tiny_decoder_prefill(wts, t, tg, W.n_q_heads, W.n_kv_heads, W.head_dim, W.rms_eps)
    assert not np.array_equal(full, b)  # the block does act when its weights are there


def test_tiny_decoder_w8a8_projections_prefill_equals_decode():
    """Block-FP8 projections in both oracles (the whole-sequence matrices and the per-row
    matrix-vector form) agree to 1e-12, and they do change the result."""
    W = wl.TINY_MLP
    wts = wl.tiny_weights(W)
    t = wl.tiny_tokens(2, W).numpy()[:24]
    tg = np.roll(t, -1)
    a = oracle.tiny_decoder_prefill(wts, t, tg, W.n_q_heads, W.n_kv_heads, W.head_dim, W.rms_eps, proj_w8a8=True)
    b = oracle.tiny_decoder_decode(wts, t, tg, W.prompt_tokens, W.n_q_heads, W.n_kv_heads, W.head_dim,
                                   W.rms_eps, proj_w8a8=True)
    assert np.max(np.abs(a - b)) <= 1e-12
    plain = oracle.tiny_decoder_prefill(wts, t, tg, W.n_q_heads, W.n_kv_heads, W.head_dim, W.rms_eps)
    assert not np.array_equal(a, plain)
    assert np.max(np.abs(a - plain)) < 0.5  # a perturbation of the same model, not another one


def test_w8a8_matmul_of_one_row_equals_the_rows_form():
    """The per-row form the decode oracle uses is the same product as the matrix form."""
    r = np.random.default_rng(21)
    a = on.bf16(r.standard_normal((5, 256)))
    w = on.bf16(r.standard_normal((300, 256)) * 0.1)
    full = oracle.w8a8_matmul(a, w)
    for i in range(5):
        assert np.array_equal(oracle.w8a8_matmul(a[i][None], w)[0], full[i])


# ---------------------------------------------------------------------------
# Block-FP8 W8A8 GEMM for the lm-head (oracle/fp8block.py)
# ---------------------------------------------------------------------------

from oracle import fp8block as ofb  # noqa: E402


def _exponent_brute(a):
    if not np.isfinite(a):
        return 128                       # the E8M0 NaN code less the bias
    if a == 0:
        return 0
    return max(-127, min(e for e in range(-300, 300) if a <= 448.0 * 2.0 ** e))


def check_block_exponent(fn):
    vals = [0.0, 448.0, 448.0 * 2 ** -7, 448.0 * 2 ** 5, 449.0, 447.0, 224.0, 224.0 + 2 ** -8, 1.0,
            2 ** -133, 3.3895314e38, 0.0078125, 57.0, 448.0 * 2 ** -127, 448.0 * 2 ** -127 * 1.01,
            448.0 * 2 ** -128, 2 ** -126, np.inf, np.nan]
    vals += list(np.abs(RNG.standard_normal(300)) * 10.0 ** RNG.integers(-45, 30, 300))
    vals += list(_all_bf16_values()[1:0x7F80:97])
    got = fn(np.array(vals))
    return all(int(g) == _exponent_brute(v) for g, v in zip(got, vals))


def test_block_exponent_matches_brute_force():
    assert check_block_exponent(ofb.block_exponent)


def test_non_finite_group_gives_nan_products_only_where_it_enters():
    a = on.bf16(RNG.standard_normal((3, 256)))
    w = on.bf16(RNG.standard_normal((5, 256)) * 0.02)
    a[1, 200] = np.inf                   # row 1, second group
    out = ofb.w8a8_matmul(a, w)
    assert np.all(np.isnan(out[1])) and np.all(np.isfinite(out[[0, 2]]))
    w[4, 3] = np.nan                     # column block 0, first K block: every column of it
    out = ofb.w8a8_matmul(a, w)
    assert np.all(np.isnan(out))


def test_tiny_group_uses_the_smallest_scale():
    x = np.zeros((1, 128))
    x[0, :3] = [2.0 ** -125, -(2.0 ** -126), 3 * 2.0 ** -127]
    codes, e = ofb.quantize_rows(x)
    assert e[0, 0] == -127
    assert np.array_equal(ofb.dequant_rows(codes, e)[0, :3], x[0, :3])  # 4, 2, 1.5 at 2^-127: exact


def test_row_groups_in_range_with_max_in_upper_octave():
    x = on.bf16(RNG.standard_normal((5, 512)) * np.array([1e-3, 1.0, 30.0, 1e4])[RNG.integers(0, 4, (5, 1))])
    x[2, 128:256] = 0.0                                       # an all-zero group
    codes, e = ofb.quantize_rows(x)
    assert codes.shape == x.shape and codes.dtype == np.uint8 and e.shape == (5, 4)
    vals = of8.e4m3_decode(codes)
    assert np.all(np.isfinite(vals)) and np.all(np.abs(vals) <= 448.0)
    gmax = np.max(np.abs(vals.reshape(5, 4, 128)), axis=-1)
    nz = np.max(np.abs(x.reshape(5, 4, 128)), axis=-1) > 0
    assert np.all((gmax[nz] >= 224.0) & (gmax[nz] <= 448.0))   # the scale is the tightest power of two
    assert e[2, 1] == 0 and np.all(codes[2, 128:256] == 0)
    # each value within half a spacing (relative 2^-4, or 2^-10 * 2^e for subnormals) of x
    back = ofb.dequant_rows(codes, e)
    ee = np.repeat(e, 128, axis=-1)
    assert np.all(np.abs(back - x) <= np.maximum(np.abs(x) * 2.0 ** -4, np.ldexp(1.0, ee - 10)))


def test_weight_blocks_match_elementwise_loop():
    w = on.bf16(RNG.standard_normal((130, 256)) * 0.02)
    w[129, :] *= 50.0                       # the ragged last block has its own scale
    codes, e = ofb.quantize_weight_blocks(w)
    assert e.shape == (2, 2) and codes.shape == w.shape
    for n in range(0, 130, 3):
        for k in range(0, 256, 5):
            blk = w[(n // 128) * 128:(n // 128 + 1) * 128, (k // 128) * 128:(k // 128 + 1) * 128]
            s = _exponent_brute(float(np.max(np.abs(blk))))
            assert e[n // 128, k // 128] == s
            assert codes[n, k] == of8.e4m3_encode(np.array([w[n, k] * 2.0 ** -s]))[0]
    back = ofb.dequant_weight_blocks(codes, e)
    assert np.array_equal(back[129], of8.e4m3_decode(codes[129]) * 2.0 ** np.repeat(e[1], 128))


def test_w8a8_matmul_of_fp8_exact_integers_is_the_integer_product():
    # integers of magnitude <= 16 have at most 4 significant bits, so every block scaling
    # and E4M3 code is exact and the product must be the int64 one
    a = RNG.integers(-16, 17, (7, 384))
    w = RNG.integers(-16, 17, (200, 384))
    a[:, 0] = 16                                               # the scales are then 2^-4
    w[:, 0] = 16
    ref = a.astype(np.int64) @ w.T.astype(np.int64)
    assert np.array_equal(ofb.w8a8_matmul(a.astype(np.float64), w.astype(np.float64)), ref.astype(np.float64))
    tg = 17
    lp = ofb.lm_head_logprob_w8a8(a[3].astype(np.float64), w.astype(np.float64), tg)
    assert abs(lp - scipy.special.log_softmax(ref[3].astype(np.float64))[tg]) < 1e-12


def test_w8a8_matmul_within_quantization_bound_of_exact():
    a = on.bf16(RNG.standard_normal((4, 256)))
    w = on.bf16(RNG.standard_normal((64, 256)) * 0.02)
    got = ofb.w8a8_matmul(a, w)
    exact = a @ w.T
    # |qa qw - a w| <= |a||w| (2 * 2^-4 + 2^-8) plus the subnormal terms (tiny at these scales)
    bound = np.abs(a) @ np.abs(w).T * (2 * 2.0 ** -4 + 2.0 ** -8) + 1e-6
    assert np.all(np.abs(got - exact) <= bound)
    assert np.any(got != exact)


def test_planted_floor_exponent_is_caught():
    # a plausible mistake: e rounded down (amax > 448 * 2^e) saturates the group's largest values
    def floor_exp(amax):
        a = np.asarray(amax, dtype=np.float64)
        ok = np.isfinite(a) & (a > 0)
        e = np.maximum(np.floor(np.log2(np.where(ok, a, 1.0) / 448.0)), -127)
        return np.where(ok, e, np.where(np.isfinite(a), 0, 128)).astype(np.int64)
    assert not check_block_exponent(floor_exp)


def test_planted_transposed_weight_blocks_are_caught():
    # a plausible mistake: the weight block exponents indexed [k-block, n-block]
    w = on.bf16(RNG.standard_normal((256, 256)) * 0.02)
    w[:128, 128:] *= 100.0
    codes, e = ofb.quantize_weight_blocks(w)
    assert not np.array_equal(ofb.dequant_weight_blocks(codes, e.T), ofb.dequant_weight_blocks(codes, e))


# ---------------------------------------------------------------------------
# Mamba-2 SSD mixer (oracle/ssd.py)
# ---------------------------------------------------------------------------

def _ssd_inputs(T=9, H=4, P=3, G=2, N=5, seed=0):
    r = np.random.default_rng(seed)
    x = r.standard_normal((T, H, P))
    B = r.standard_normal((T, G, N))
    C = r.standard_normal((T, G, N))
    dt = np.log1p(np.exp(r.standard_normal((T, H)) - 1.0))   # softplus: positive
    A = -np.exp(r.uniform(0.0, 1.5, H))
    D = r.standard_normal(H)
    return x, B, C, dt, A, D


def _ssd_quadratic(x, B, C, dt, A, D):
    """The same layer as one masked matrix product per head (the state-space / attention
    duality): y_h = (L_h o (C_g B_g^T)) (dt_h x_h) + D_h x_h, L_h[t, s] the product of the
    decays a_r over s < r <= t (0 above the diagonal), written out as explicit products."""
    T, H, P = x.shape
    G = B.shape[1]
    y = np.empty((T, H, P))
    for h in range(H):
        g = h // (H // G)
        a = np.exp(dt[:, h] * A[h])
        L = np.zeros((T, T))
        for t in range(T):
            for s in range(t + 1):
                L[t, s] = np.prod(a[s + 1:t + 1])
        M = L * (C[:, g, :] @ B[:, g, :].T)
        y[:, h, :] = M @ (dt[:, h, None] * x[:, h, :]) + D[h] * x[:, h, :]
    return y


def check_ssd(fn):
    x, B, C, dt, A, D = _ssd_inputs()
    y = fn(x, B, C, dt, A, D)[0]
    assert np.allclose(y, _ssd_quadratic(x, B, C, dt, A, D), rtol=1e-12, atol=1e-12)
    # one position: y_0 = dt_0 (C_0 . B_0) x_0 + D x_0 per head
    y0 = fn(x[:1], B[:1], C[:1], dt[:1], A, D)[0][0]
    H, G = x.shape[1], B.shape[1]
    for h in range(H):
        g = h // (H // G)
        want = dt[0, h] * (C[0, g] @ B[0, g]) * x[0, h] + D[h] * x[0, h]
        assert np.allclose(y0[h], want, rtol=1e-13, atol=1e-14)
    # an infinitely fast decay forgets everything but the current position
    yf = fn(x, B, C, dt, np.full_like(A, -1e6), D)[0]
    for t in range(x.shape[0]):
        for h in range(H):
            g = h // (H // G)
            want = dt[t, h] * (C[t, g] @ B[t, g]) * x[t, h] + D[h] * x[t, h]
            assert np.allclose(yf[t, h], want, rtol=1e-12, atol=1e-13)


def test_ssd_matches_quadratic_form_and_closed_forms():
    check_ssd(oracle.ssd_scan)


def test_ssd_state_by_brute_force_and_without_decay():
    x, B, C, dt, A, D = _ssd_inputs(T=6, H=2, P=2, G=1, N=3, seed=4)
    T, H, P = x.shape
    y, S_last = oracle.ssd_scan(x, B, C, dt, A, D)
    for t in range(T):   # the state as an explicit sum over past positions
        for h in range(H):
            S = np.zeros((3, P))
            for s in range(t + 1):
                w = dt[s, h] * math.prod(math.exp(dt[r, h] * A[h]) for r in range(s + 1, t + 1))
                S += w * np.outer(B[s, 0], x[s, h])
            assert np.allclose(y[t, h], C[t, 0] @ S + D[h] * x[t, h], rtol=1e-12, atol=1e-13)
            if t == T - 1:
                assert np.allclose(S_last[h], S, rtol=1e-12, atol=1e-13)
    # A = 0: no decay, the state is a running sum
    y0 = oracle.ssd_scan(x, B, C, dt, np.zeros(H), np.zeros(H))[0]
    run = np.cumsum(dt[:, :, None, None] * B[:, 0][:, None, :, None] * x[:, :, None, :], axis=0)
    assert np.allclose(y0, np.einsum("tn,thnp->thp", C[:, 0], run), rtol=1e-12, atol=1e-13)


def test_ssd_state_carry_equals_one_pass():
    x, B, C, dt, A, D = _ssd_inputs(T=13, seed=9)
    y, S = oracle.ssd_scan(x, B, C, dt, A, D)
    y1, S1 = oracle.ssd_scan(x[:5], B[:5], C[:5], dt[:5], A, D)
    y2, S2 = oracle.ssd_scan(x[5:], B[5:], C[5:], dt[5:], A, D, state=S1)
    assert np.allclose(np.concatenate([y1, y2]), y, rtol=1e-13, atol=1e-14)
    assert np.allclose(S2, S, rtol=1e-13, atol=1e-14)
    assert np.array_equal(oracle.ssd_outputs(x, B, C, dt, A, D), oracle.bf16(y))


def _ssd_planted(kind):
    def fn(x, B, C, dt, A, D, state=None):
        T, H, P = x.shape
        G, N = B.shape[1], B.shape[2]
        grp = np.arange(H) % G if kind == "group" else np.arange(H) // (H // G)
        S = np.zeros((H, N, P))
        y = np.empty((T, H, P))
        for t in range(T):
            ta = max(t - 1, 0) if kind == "shift" else t
            a = np.exp(dt[ta] * A)
            Bt, Ct = (C[t][grp], B[t][grp]) if kind == "swap" else (B[t][grp], C[t][grp])
            w = np.ones_like(dt[t]) if kind == "no_dt" else dt[t]
            S = a[:, None, None] * S + (w[:, None, None] * Bt[:, :, None]) * x[t][:, None, :]
            y[t] = np.einsum("hn,hnp->hp", Ct, S) + (0.0 if kind == "no_d" else D[:, None] * x[t])
        return y, S
    return fn


@pytest.mark.parametrize("kind", ["no_dt", "shift", "swap", "no_d", "group"])
def test_planted_ssd_mistakes_are_caught(kind):
    with pytest.raises(AssertionError):
        check_ssd(_ssd_planted(kind))
