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


def test_mla_split_multiple_contexts():
    # contexts at and across multiples of the 2048-token MLA split (and of the 64-token
    # tile): full last splits in decode, and the prefill chain's split boundary
    from mla_case import MLACase
    c = MLACase(SMALL, [0, 1, 2], ctx=[2048, 2056, 4096])
    rows = [0, 1, 2]
    n = 16
    c.write_history("d", rows, n)
    dec = torch.stack([c.decode_back("d", rows, back) for back in range(n, 0, -1)], dim=1)
    att_last = c.attn_out(3).float().cpu().numpy()
    c.write_history("p", rows, n)
    pre = c.prefill_last("p", rows, n)
    assert np.array_equal(_bits(dec), _bits(pre))
    dn = dec.cpu().numpy()
    for i, r in enumerate(rows):
        lp_o, o_o = c.oracle_row(r)
        assert np.max(np.abs(att_last[i] - o_o)) < 2e-2, r
        assert abs(dn[i, -1] - lp_o) <= 2e-2, r
    # the row whose window crosses 2048: the step at context exactly 2048 (back = 9)
    lp_o, _ = c.oracle_row(1, back=9)
    assert abs(dn[1, n - 9] - lp_o) <= 2e-2


def test_mla_graph_replays_equal_eager():
    # the captured MLA decode step: contexts cross the 2048-token split between replays
    from mla_case import MLACase
    c = MLACase(SMALL, [0, 1], ctx=[2050, 700], copies=3)
    rows = [0, 1]
    steps = 8
    c.write_history("g", rows, steps)
    seqs = [("g", r) for r in rows]

    def inputs(back):
        q, cc, t, ctx = [], [], [], []
        for r in rows:
            d = c.data[r]
            R = d["q"].shape[0]
            p = d["ctx"] - back
            q.append(d["q"][R - back])
            cc.append(d["c"][p])
            t.append(d["target"][R - back])
            ctx.append(p + 1)
        return dict(q=torch.stack(q), k=torch.stack(cc), targets=torch.stack(t).to(torch.int32)), ctx

    kw, ctx = inputs(steps)
    g = c.sess.decode_graph(seqs, max(c.ctx(r) for r in rows), ctx=ctx, **kw)
    try:
        for back in range(steps, 0, -1):
            kw, ctx = inputs(back)
            lg = g.run(ctx, **kw).clone()
            le = c.sess.decode(seqs, ctx, **kw)
            assert np.array_equal(_bits(lg), _bits(le)), (back, ctx)
            g.replay()
            torch.cuda.synchronize()
            assert np.array_equal(_bits(g.out), _bits(le)), back
    finally:
        g.close()
