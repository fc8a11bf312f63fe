"""GPU tests of absorbed MLA decode through the C ABI: attention output and logprob
parity with the fp64 oracle, bitwise prefill recompute == decode, and batch invariance."""

import numpy as np
import pytest
import torch

import workloads as wl

pytestmark = pytest.mark.gpu

# 64 heads (one head group), a small vocabulary and head; contexts span tiles, splits
# (2048 tokens) and ragged tails.
SMALL = wl.scaled(wl.MLA_DECODE_B128, rows=5, n_heads=64, vocab=1000, d_head=256, recompute_tokens=16)
SMALL_CTX = [1, 65, 700, 2100, 4200]
MULTI = [1, 2, 3, 4]


def _case(**kw):
    from mla_case import MLACase
    return MLACase(SMALL, list(range(5)), ctx=SMALL_CTX, **kw)


def _bits(t):
    return t.detach().cpu().contiguous().view(torch.int32).numpy()


def test_mla_decode_matches_oracle():
    c = _case()
    rows = list(range(5))
    c.write_history("d", rows, 1)
    lp = c.decode_back("d", rows, 1).cpu().numpy()
    att = c.attn_out(len(rows)).float().cpu().numpy()
    for i, r in enumerate(rows):
        lp_o, o_o = c.oracle_row(r)
        err = np.max(np.abs(att[i] - o_o))
        assert err < 2e-2, (r, err)
        assert abs(lp[i] - lp_o) <= 2e-2, (r, lp[i], lp_o)


def test_mla_prefill_equals_decode_bitwise():
    c = _case()
    rows = MULTI
    n = 16
    c.write_history("d", rows, n)
    dec, att_dec = [], []
    for back in range(n, 0, -1):
        dec.append(c.decode_back("d", rows, back))
        att_dec.append(c.attn_out(len(rows)).clone())
    dec = torch.stack(dec, dim=1)
    c.write_history("p", rows, n)
    pre = c.prefill_last("p", rows, n)
    assert np.array_equal(_bits(dec), _bits(pre))
    # attention outputs too: prefill row (i, j) is token i*n + j
    att_pre = c.attn_out(len(rows) * n).view(len(rows), n, SMALL.n_heads, SMALL.kv_rank)
    for j in range(n):
        assert torch.equal(att_dec[j].view(torch.int16), att_pre[:, j].contiguous().view(torch.int16)), j


def test_mla_batch_invariance():
    c = _case()
    rows = list(range(5))
    c.write_history("d", rows, 1)
    ref = _bits(c.decode_back("d", rows, 1))
    rng = np.random.default_rng(3)
    for size in (1, 2, 3, 5):
        pick = [int(x) for x in rng.permutation(5)[:size]]
        assert np.array_equal(_bits(c.decode_back("d", pick, 1)), ref[pick]), pick


def test_mla_128_heads_two_groups():
    from mla_case import MLACase
    w = wl.scaled(wl.MLA_DECODE_B128, rows=2, n_heads=128, vocab=600, d_head=128, recompute_tokens=4)
    c = MLACase(w, [0, 1], ctx=[300, 2500])
    c.write_history("d", [0, 1], 4)
    dec = torch.stack([c.decode_back("d", [0, 1], b) for b in (4, 3, 2, 1)], dim=1)
    att = c.attn_out(2).float().cpu().numpy()
    for i in range(2):
        lp_o, o_o = c.oracle_row(i)
        assert np.max(np.abs(att[i] - o_o)) < 2e-2
        assert abs(float(dec[i, -1]) - lp_o) <= 2e-2
    c.write_history("p", [0, 1], 4)
    assert np.array_equal(_bits(dec), _bits(c.prefill_last("p", [0, 1], 4)))
