"""GPU tests of the captured decode step (ril_decode_graph_create / ril_graph_launch).

A replay runs the same kernels with the same arguments as the uncaptured call, so its
logprobs must equal that call's bitwise on the same inputs: over successive steps whose
inputs are rewritten in place, with eager work between replays (each eager call and a
second replay follow every replay), after the lm-head weights are rewritten in place,
and for the token-input one-layer decoder (embedding, QKV and O projections inside the
step).  The eager calls also use a smaller grid bound than the graph, so the test checks
that the bits do not depend on the grid either."""

import math

import numpy as np
import pytest
import torch

import workloads as wl

pytestmark = pytest.mark.gpu

SMALL = wl.scaled(wl.GQA_DECODE_B64, rows=6, vocab=2100, recompute_tokens=16)
CTX = [17, 64, 65, 600, 1100]
ROWS = [1, 2, 3, 4, 5]
STEPS = 12


def _bits(t):
    return t.detach().cpu().contiguous().view(torch.int32).numpy()


def _case():
    from gqa_case import GQACase
    return GQACase(SMALL, ROWS, ctx=CTX, copies=4)


def test_graph_replays_equal_eager_over_steps():
    c = _case()
    seqs = [("g", r) for r in ROWS]
    c.write_history("g", ROWS, STEPS)
    q, k, v, t, ctx = c.step_inputs(ROWS, STEPS)
    bound = max(c.ctx(r) for r in ROWS)  # the model's max_ctx; above every other row's context
    g = c.sess.decode_graph(seqs, bound, ctx=ctx, targets=t, q=q, k=k, v=v)
    try:
        for back in range(STEPS, 0, -1):
            q, k, v, t, ctx = c.step_inputs(ROWS, back)
            lg = g.run(ctx, targets=t, q=q, k=k, v=v).clone()
            le = c.sess.decode(seqs, ctx, targets=t, q=q, k=k, v=v)  # grid bound max(ctx)
            assert bool(torch.isfinite(le).all())
            assert np.array_equal(_bits(lg), _bits(le)), back
            g.replay()  # the same inputs again, after the eager call
            torch.cuda.synchronize()
            assert np.array_equal(_bits(g.out), _bits(le)), back
    finally:
        g.close()


def test_graph_sees_weights_rewritten_in_place():
    from invariant_rl_logprob_amd import ril_pack_lm_head
    c = _case()
    seqs = [("w", r) for r in ROWS]
    c.write_history("w", ROWS, 1)
    q, k, v, t, ctx = c.step_inputs(ROWS, 1)
    g = c.sess.decode_graph(seqs, max(ctx), ctx=ctx, targets=t, q=q, k=k, v=v)
    try:
        before = g.run(ctx, targets=t, q=q, k=k, v=v).clone()
        w2 = c.head["w_lm"].flip(0).contiguous()  # another head, same shape
        ril_pack_lm_head(w2, c.sess.w_lm_packed)  # into the captured buffer
        after = g.run(ctx, targets=t, q=q, k=k, v=v).clone()
        eager = c.sess.decode(seqs, ctx, targets=t, q=q, k=k, v=v)
        assert np.array_equal(_bits(after), _bits(eager))
        assert not np.array_equal(_bits(after), _bits(before))
    finally:
        g.close()


def test_graph_rejects_contexts_past_its_bound():
    c = _case()
    seqs = [("b", r) for r in ROWS]
    c.write_history("b", ROWS, 2)
    q, k, v, t, ctx = c.step_inputs(ROWS, 2)
    g = c.sess.decode_graph(seqs, max(ctx), ctx=ctx, targets=t, q=q, k=k, v=v)
    try:
        with pytest.raises(ValueError):
            g.run([x + 1 for x in ctx], targets=t, q=q, k=k, v=v)
    finally:
        g.close()


def test_graph_tiny_decoder_token_input():
    from invariant_rl_logprob_amd import RIL_INPUT_TOKENS
    from invariant_rl_logprob_amd.session import Session
    W = wl.TINY
    wts = wl.tiny_weights(W, device="cuda")
    toks = [wl.tiny_tokens(i, W, device="cuda") for i in range(len(W.lengths))]
    s = Session(n_q_heads=W.n_q_heads, n_kv_heads=W.n_kv_heads, head_dim=W.head_dim, vocab=W.vocab,
                d_head=W.d_model, d_model=W.d_model, w_lm=wts["w_lm"], embed=wts["embed"],
                w_qkv=wts["w_qkv"], w_o=wts["w_o"], norm_attn=wts["norm_attn"],
                norm_final=wts["norm_final"], max_rows=8, max_tokens=512, max_ctx=max(W.lengths),
                pool_pages=4096, softmax_scale=1.0 / math.sqrt(W.head_dim), rms_eps=W.rms_eps,
                shuffle_seed=7, input_mode=RIL_INPUT_TOKENS)
    P = W.prompt_tokens
    ids = list(range(len(W.lengths)))
    seqs = [("t", i) for i in ids]
    tgt = lambda i, p: toks[i][p + 1] if p + 1 < toks[i].shape[0] else toks[i][0]  # noqa: E731
    s.prefill(seqs, [0] * len(ids), targets=[toks[i][1:P + 1] for i in ids], tokens=[toks[i][:P] for i in ids])
    steps = min(W.lengths) - P - 1  # every sequence still has a next token
    first = torch.stack([toks[i][P] for i in ids]).to(torch.int32)
    g = s.decode_graph(seqs, max(W.lengths), ctx=[P + 1] * len(ids),
                       targets=torch.stack([tgt(i, P) for i in ids]).to(torch.int32), tokens=first)
    try:
        for j in range(steps):
            p = P + j
            tok = torch.stack([toks[i][p] for i in ids]).to(torch.int32)
            tg = torch.stack([tgt(i, p) for i in ids]).to(torch.int32)
            lg = g.run([p + 1] * len(ids), targets=tg, tokens=tok).clone()
            le = s.decode(seqs, [p + 1] * len(ids), targets=tg, tokens=tok)
            assert np.array_equal(_bits(lg), _bits(le)), j
    finally:
        g.close()
