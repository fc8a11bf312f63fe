"""GPU tests of ril_decode_step_logprobs_noalloc, the decode step on the library's static
device scratch (for callers that cannot allocate): its logprobs equal those of
ril_decode_step_logprobs with a caller workspace bit for bit, on two calls in a row, the
second with fewer rows, for the q/k/v-input GQA model and the token-input decoder (whose
projections use more of the workspace)."""

import math

import numpy as np
import pytest
import torch

import workloads as wl

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.detach().cpu().contiguous().view(torch.int32).numpy()


def _noalloc(sess, seqs, ctx, **kw):
    import invariant_rl_logprob_amd as ril
    b, keep = sess._decode_batch(seqs, ctx, kw.pop("targets"), kw.pop("q", None), kw.pop("k", None),
                                 kw.pop("v", None), kw.pop("tokens", None), None, None, None, None)
    out = torch.full((len(seqs),), float("nan"), dtype=torch.float32, device="cuda")
    ril.ril_decode_step_logprobs_noalloc(sess.model, sess.kv, b, out)
    torch.cuda.synchronize()
    return out


def test_noalloc_decode_equals_workspace_decode_gqa():
    import invariant_rl_logprob_amd as ril
    from gqa_case import GQACase
    w = wl.scaled(wl.GQA_DECODE_B64, rows=6, vocab=2100, recompute_tokens=4)
    c = GQACase(w, list(range(6)), ctx=[1, 17, 520, 1024, 1100, 2050])
    assert ril.ril_workspace_bytes(c.sess.model) <= ril.RIL_NOALLOC_SCRATCH_BYTES
    for rows in (list(range(6)), [4, 1, 5]):  # the second call with fewer rows, reordered
        tag = f"r{len(rows)}"
        c.write_history(tag, rows, 1)
        q, k, v, t, ctx = c.step_inputs(rows, 1)
        seqs = [(tag, r) for r in rows]
        ref = c.sess.decode(seqs, ctx, targets=t, q=q, k=k, v=v)
        got = _noalloc(c.sess, seqs, ctx, targets=t, q=q, k=k, v=v)
        assert bool(torch.isfinite(got).all())
        assert np.array_equal(_bits(got), _bits(ref)), rows


def test_noalloc_decode_equals_workspace_decode_token_input():
    import invariant_rl_logprob_amd as ril
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
                shuffle_seed=9, input_mode=RIL_INPUT_TOKENS)
    assert ril.ril_workspace_bytes(s.model) <= ril.RIL_NOALLOC_SCRATCH_BYTES
    P = W.prompt_tokens
    for ids in ([0, 1, 2, 3], [2, 0]):  # the second call with fewer rows
        tag = f"t{len(ids)}"
        seqs = [(tag, i) for i in ids]
        s.prefill(seqs, [0] * len(ids), targets=[toks[i][1:P + 1] for i in ids], tokens=[toks[i][:P] for i in ids])
        tok = torch.stack([toks[i][P] for i in ids]).to(torch.int32)
        tgt = torch.stack([toks[i][P + 1] for i in ids]).to(torch.int32)
        ref = s.decode(seqs, [P + 1] * len(ids), targets=tgt, tokens=tok)
        got = _noalloc(s, seqs, [P + 1] * len(ids), targets=tgt, tokens=tok)
        assert bool(torch.isfinite(got).all())
        assert np.array_equal(_bits(got), _bits(ref)), ids


def test_noalloc_rejects_a_workspace_above_the_scratch():
    import invariant_rl_logprob_amd as ril
    from gqa_case import GQACase
    w = wl.scaled(wl.GQA_DECODE_B64, rows=2, vocab=2100, recompute_tokens=4)
    c = GQACase(w, [0, 1], ctx=[40, 60], max_tokens=40000)  # a prefill-sized workspace
    assert ril.ril_workspace_bytes(c.sess.model) > ril.RIL_NOALLOC_SCRATCH_BYTES
    q, k, v, t, ctx = c.step_inputs([0, 1], 1)
    c.write_history("x", [0, 1], 1)
    with pytest.raises(ril.RilError) as e:
        _noalloc(c.sess, [("x", 0), ("x", 1)], ctx, targets=t, q=q, k=k, v=v)
    assert e.value.status == ril.RIL_ERANGE
