"""GPU tests of the token-input decoder with a SwiGLU MLP block (activation rounded once,
Bitwise-consistent RL post, section 4.4 condition 3): parity with the fp64 oracle's two
forms, decode bitwise equal to prefill across batch orderings, and chunk-size invariance."""

import itertools
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from test_gpu_tiny_decoder import _bits, _prefill, _prompt_then_decode, _targets

pytestmark = pytest.mark.gpu

TOL = 2e-2
W = wl.TINY_MLP


@pytest.fixture(scope="module")
def tiny_mlp():
    from invariant_rl_logprob_amd import RIL_INPUT_TOKENS
    from invariant_rl_logprob_amd.session import Session
    wts = wl.tiny_weights(W, device="cuda")
    toks = [wl.tiny_tokens(i, W, device="cuda") for i in range(len(W.lengths))]
    s = Session(n_q_heads=W.n_q_heads, n_kv_heads=W.n_kv_heads, head_dim=W.head_dim, vocab=W.vocab,
                d_head=W.d_model, d_model=W.d_model, w_lm=wts["w_lm"], embed=wts["embed"],
                w_qkv=wts["w_qkv"], w_o=wts["w_o"], norm_attn=wts["norm_attn"],
                norm_final=wts["norm_final"], max_rows=8, max_tokens=512, max_ctx=max(W.lengths),
                pool_pages=4096, softmax_scale=1.0 / math.sqrt(W.head_dim), rms_eps=W.rms_eps,
                shuffle_seed=17, input_mode=RIL_INPUT_TOKENS, d_ff=W.d_ff, w_gate_up=wts["w_gate_up"],
                w_down=wts["w_down"], norm_mlp=wts["norm_mlp"])
    return s, wts, toks


def test_tiny_mlp_prefill_matches_oracle(tiny_mlp):
    s, wts, toks = tiny_mlp
    lp = _prefill(s, "full", [0, 1, 2, 3], toks)
    for i in range(4):
        t = toks[i].cpu().numpy()
        tg = _targets(toks[i]).cpu().numpy()
        want = oracle.tiny_decoder_prefill(wts, t, tg, W.n_q_heads, W.n_kv_heads, W.head_dim, W.rms_eps)
        got = lp[i].cpu().numpy()
        assert np.max(np.abs(got[:-1] - want[:-1])) <= TOL, (i, np.max(np.abs(got[:-1] - want[:-1])))
    # the decode-form oracle on one sequence as well
    t = toks[0].cpu().numpy()
    want_d = oracle.tiny_decoder_decode(wts, t, _targets(toks[0]).cpu().numpy(), W.prompt_tokens, W.n_q_heads,
                                        W.n_kv_heads, W.head_dim, W.rms_eps)
    assert np.max(np.abs(lp[0].cpu().numpy()[:-1] - want_d[:-1])) <= TOL


def test_tiny_mlp_decode_bitwise_equals_prefill(tiny_mlp):
    s, wts, toks = tiny_mlp
    full = _prefill(s, "ref", [0, 1, 2, 3], toks)
    ref = {i: _bits(full[i][:-1]) for i in range(4)}
    orders = [[i] for i in range(4)] + [[2, 0], [3, 1]] + [list(p) for p in itertools.permutations(range(4))][::5]
    for n, order in enumerate(orders):
        got = _prompt_then_decode(s, ("o", n), order, toks, W.prompt_tokens)
        for i in order:
            assert np.array_equal(_bits(got[i]), ref[i]), (order, i)
        for i in order:
            s.release((("o", n), i))


def test_tiny_mlp_prefill_chunk_sizes(tiny_mlp):
    s, wts, toks = tiny_mlp
    ref = _prefill(s, "c0", [0, 1, 2, 3], toks)
    for ch in (1, 33):
        got = _prefill(s, ("c", ch), [3, 1, 0, 2], toks, chunk=ch)
        for i in range(4):
            assert np.array_equal(_bits(got[i][:-1]), _bits(ref[i][:-1])), (ch, i)
