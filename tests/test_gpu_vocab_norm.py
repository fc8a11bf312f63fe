"""The head's normalisation over the whole vocabulary (Defeating Nondeterminism in LLM
Inference, the sampled-token logprob as log-softmax over the vocabulary; the
Bitwise-consistent RL post, section 4: the trainer and the sampler read the same
logprob), checked through ril_lm_head_logprobs by exporting every vocabulary entry's
logprob for a few rows: each row's probabilities must sum to 1 within 1e-5 (fp32).

A vocabulary tile dropped from the log-sum-exp, a ragged last tile padded with zeros
instead of being masked, or a merge that rescales one partial sum twice moves the sum by
far more than that (one 256-entry tile of a 129280-word vocabulary carries about 0.2% of
the mass of a flat row).  The bf16 and the W8A8 head both, at the full 129280 x 4096
head, with 4096-row calls (row tiles back to back per vocabulary tile), and at a ragged
2100-entry vocabulary with the 16-row decode shape.
"""

import numpy as np
import pytest
import torch

import workloads as wl

pytestmark = pytest.mark.gpu

W8A8 = 1


def _rows(d_head, seed):
    g = torch.Generator().manual_seed(seed)
    z = torch.randn(3, d_head, generator=g)
    z[1] *= 8.0          # peaked: logits of standard deviation about 10
    z[2] = 0.0           # uniform
    return z.to(torch.bfloat16)


def _session(w, V, lm_dtype, max_tokens):
    from invariant_rl_logprob_amd.session import Session
    return Session(n_q_heads=32, n_kv_heads=8, head_dim=128, vocab=V, d_head=w.shape[1], w_lm=w, max_rows=16,
                   max_tokens=max_tokens, max_ctx=64, pool_pages=8, softmax_scale=0.088388, lm_dtype=lm_dtype)


def _every_logprob(s, z, V, call_rows):
    """fp32 [V] logprobs of every vocabulary entry for one normalised row z."""
    out = []
    for lo in range(0, V, call_rows):
        n = min(call_rows, V - lo)
        t = torch.arange(lo, lo + n, dtype=torch.int32, device="cuda")
        out.append(s.lm_head(z.expand(n, -1).contiguous(), t))
    return torch.cat(out).cpu().numpy().astype(np.float64)


def _check(lp, V, what):
    assert lp.shape == (V,) and np.all(np.isfinite(lp)) and np.all(lp <= 0.0), what
    total = np.exp(lp).sum()
    print("%s: |sum exp(lp) - 1| = %.3g" % (what, abs(total - 1.0)))
    assert abs(total - 1.0) <= 1e-5, (what, total)


@pytest.mark.parametrize("lm_dtype", [0, W8A8])
def test_every_vocab_logprob_sums_to_one_full_head(lm_dtype):
    w = wl.gqa_head_weights(wl.GQA_DECODE_B64)["w_lm"].cuda()
    V = w.shape[0]
    s = _session(w, V, lm_dtype, 4096)
    z = _rows(w.shape[1], 21).cuda()
    for i in range(3):
        lp = _every_logprob(s, z[i:i + 1], V, 4096)
        _check(lp, V, ("full", lm_dtype, i))
        if i == 2:
            assert np.all(lp == lp[0]) and abs(lp[0] + np.log(V)) < 4e-6


@pytest.mark.parametrize("lm_dtype", [0, W8A8])
def test_every_vocab_logprob_sums_to_one_ragged_vocab_decode_shape(lm_dtype):
    V = 2100
    w = wl.gqa_head_weights(wl.scaled(wl.GQA_DECODE_B64, vocab=V))["w_lm"].cuda()
    s = _session(w, V, lm_dtype, 256)
    z = _rows(w.shape[1], 22).cuda()
    for i in range(2):
        _check(_every_logprob(s, z[i:i + 1], V, 16), V, ("ragged", lm_dtype, i))
