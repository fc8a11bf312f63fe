"""GPU tests of the one-layer decoder with token input (embedding, RMSNorm, QKV GEMM,
paged attention, O GEMM + residual, final RMSNorm, lm-head): full prefill vs a
16-token prefill followed by token-by-token decode, across batch orderings of the
four sequences, bitwise; and parity with the fp64 oracle."""

import itertools
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as wl

pytestmark = pytest.mark.gpu

TOL = 2e-2
W = wl.TINY


@pytest.fixture(scope="module")
def tiny():
    from invariant_rl_logprob_amd import RIL_INPUT_TOKENS
    from invariant_rl_logprob_amd.session import Session
    wts = wl.tiny_weights(W, device="cuda")
    toks = [wl.tiny_tokens(i, W, device="cuda") for i in range(len(W.lengths))]
    s = Session(n_q_heads=W.n_q_heads, n_kv_heads=W.n_kv_heads, head_dim=W.head_dim, vocab=W.vocab,
                d_head=W.d_model, d_model=W.d_model, w_lm=wts["w_lm"], embed=wts["embed"],
                w_qkv=wts["w_qkv"], w_o=wts["w_o"], norm_attn=wts["norm_attn"],
                norm_final=wts["norm_final"], max_rows=8, max_tokens=512, max_ctx=max(W.lengths),
                pool_pages=4096, softmax_scale=1.0 / math.sqrt(W.head_dim), rms_eps=W.rms_eps,
                shuffle_seed=99, input_mode=RIL_INPUT_TOKENS)
    return s, wts, toks


def _targets(t):
    # next token; the last position has none (0 is a placeholder, never compared)
    return torch.cat([t[1:], torch.zeros(1, dtype=t.dtype, device=t.device)])


def _prefill(s, tag, seqs, toks, chunk=None):
    """Prefill each listed sequence entirely (in chunks of `chunk` tokens); lp per seq."""
    L = {i: toks[i].shape[0] for i in seqs}
    out = {i: [] for i in seqs}
    done = 0
    step = chunk or max(L.values())
    while any(done < L[i] for i in seqs):
        live = [i for i in seqs if done < L[i]]
        lens = [min(step, L[i] - done) for i in live]
        lp = s.prefill([(tag, i) for i in live], [done] * len(live),
                       targets=[_targets(toks[i])[done:done + n] for i, n in zip(live, lens)],
                       tokens=[toks[i][done:done + n] for i, n in zip(live, lens)])
        o = 0
        for i, n in zip(live, lens):
            out[i].append(lp[o:o + n])
            o += n
        done += step
    return {i: torch.cat(v) for i, v in out.items()}


def _prompt_then_decode(s, tag, seqs, toks, n_prompt):
    """Prefill n_prompt tokens of the listed sequences together, then decode them in
    lockstep (the batch shrinks as sequences end).  lp per seq for positions 0..L-2."""
    pre = s.prefill([(tag, i) for i in seqs], [0] * len(seqs),
                    targets=[_targets(toks[i])[:n_prompt] for i in seqs],
                    tokens=[toks[i][:n_prompt] for i in seqs])
    out = {i: [pre[k * n_prompt:(k + 1) * n_prompt]] for k, i in enumerate(seqs)}
    pos = n_prompt
    while True:
        live = [i for i in seqs if pos < toks[i].shape[0] - 1]
        if not live:
            break
        tg = torch.stack([_targets(toks[i])[pos] for i in live])
        tk = torch.stack([toks[i][pos] for i in live]).to(torch.int32)
        lp = s.decode([(tag, i) for i in live], [pos + 1] * len(live), targets=tg, tokens=tk)
        for k, i in enumerate(live):
            out[i].append(lp[k:k + 1])
        pos += 1
    return {i: torch.cat(v) for i, v in out.items()}


def _bits(t):
    return t.detach().cpu().view(torch.int32).numpy()


def test_tiny_prefill_matches_oracle(tiny):
    s, wts, toks = tiny
    lp = _prefill(s, "full", [0, 1, 2, 3], toks)
    for i in range(4):
        t = toks[i].cpu().numpy()
        want = oracle.tiny_decoder_prefill(wts, t, _targets(toks[i]).cpu().numpy(), W.n_q_heads,
                                           W.n_kv_heads, W.head_dim, W.rms_eps)
        got = lp[i].cpu().numpy()
        assert np.max(np.abs(got[:-1] - want[:-1])) <= TOL, (i, np.max(np.abs(got[:-1] - want[:-1])))


def test_tiny_decode_bitwise_equals_prefill_across_orderings(tiny):
    s, wts, toks = tiny
    full = _prefill(s, "ref", [0, 1, 2, 3], toks)
    ref = {i: _bits(full[i][:-1]) for i in range(4)}
    orders = [[i] for i in range(4)]
    orders += [[0, 1], [2, 3], [3, 1], [2, 0], [1, 2]]
    orders += [list(p) for p in itertools.permutations(range(4))]
    for n, order in enumerate(orders):
        got = _prompt_then_decode(s, ("o", n), order, toks, W.prompt_tokens)
        for i in order:
            assert np.array_equal(_bits(got[i]), ref[i]), (order, i)
        for i in order:
            s.release((("o", n), i))


def test_tiny_prefill_chunk_sizes(tiny):
    s, wts, toks = tiny
    ref = _prefill(s, "c0", [0, 1, 2, 3], toks)
    for ch in (1, 16, 33, 64):
        got = _prefill(s, ("c", ch), [3, 1, 0, 2], toks, chunk=ch)
        for i in range(4):
            assert np.array_equal(_bits(got[i][:-1]), _bits(ref[i][:-1])), (ch, i)
