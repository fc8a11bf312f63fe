"""GPU tests of the GQA path through the C ABI: parity with the fp64 oracle and
bitwise invariance (prefill vs decode, batch composition, row order, chunking,
page placement)."""

import math

import numpy as np
import pytest
import torch

import oracle
import workloads as wl

pytestmark = pytest.mark.gpu

TOL = 2e-2  # nats per token, GPU vs fp64 oracle

# A workload of the decode shape with short contexts spanning tile, split and page
# boundaries and a vocabulary with a partial last tile.
SMALL = wl.scaled(wl.GQA_DECODE_B64, rows=6, vocab=2100, recompute_tokens=16)
SMALL_CTX = [1, 17, 64, 65, 600, 1100]
MULTI = [1, 2, 3, 4, 5]  # rows with at least 16 positions, for multi-position checks


def _case(**kw):
    from gqa_case import GQACase
    return GQACase(SMALL, list(range(6)), ctx=SMALL_CTX, **kw)


def _bits(t):
    return t.detach().cpu().view(torch.int32).numpy()


def test_uniform_logprob_with_zero_lm_head():
    from gqa_case import GQACase
    w = wl.scaled(wl.GQA_DECODE_B64, rows=2, recompute_tokens=1)
    head = {"w_lm": torch.zeros(w.vocab, w.d_head, dtype=torch.bfloat16, device="cuda")}
    c = GQACase(w, [0, 1], ctx=[5, 700], head=head)
    c.write_history("d", [0, 1], 1)
    lp = c.decode_back("d", [0, 1], 1).cpu().numpy()
    assert np.all(np.abs(lp + math.log(w.vocab)) < 1e-5), lp


def test_decode_matches_oracle():
    c = _case()
    rows = list(range(6))
    c.write_history("d", rows, 1)
    lp = c.decode_back("d", rows, 1).cpu().numpy()
    att = c.sess.attn_out(len(rows)).float().cpu().numpy()
    for i, r in enumerate(rows):
        lp_o, o_o = c.oracle_row(r)
        assert abs(lp[i] - lp_o) <= TOL, (r, lp[i], lp_o)
        # attention output: bf16 of a value within fp32/bf16-P error of the fp64 one
        assert np.max(np.abs(att[i] - o_o)) < 2e-2, (r, np.max(np.abs(att[i] - o_o)))
        assert np.max(np.abs(att[i] - o_o)) / (np.max(np.abs(o_o)) + 1e-30) < 1e-2


def test_prefill_matches_oracle():
    c = _case()
    rows = MULTI
    c.write_history("p", rows, 16)
    lps = c.prefill_last("p", rows, 16).cpu().numpy()
    for i, r in enumerate(rows):
        for back in (1, 9, 16):
            if c.ctx(r) - back < 0:
                continue
            lp_o, _ = c.oracle_row(r, back)
            assert abs(lps[i, 16 - back] - lp_o) <= TOL, (r, back)


def test_decode_bitwise_equals_prefill_and_chunking():
    c = _case()
    rows = MULTI
    n = 16
    c.write_history("d", rows, n)
    dec = torch.stack([c.decode_back("d", rows, back) for back in range(n, 0, -1)], dim=1)
    c.write_history("p", rows, n)
    pre = c.prefill_last("p", rows, n)
    assert np.array_equal(_bits(dec), _bits(pre)), "prefill != decode"
    s = oracle.diff_stats(dec.double().cpu().numpy().ravel(), pre.double().cpu().numpy().ravel())
    assert s["max"] == s["mean"] == s["std"] == 0.0
    assert oracle.k3_mean(pre.double().cpu().numpy(), dec.double().cpu().numpy()) == 0.0
    # the same tokens prefilled in uneven chunks (rewrites identical K/V: idempotent)
    pre2 = c.prefill_last("p", rows, n, chunks=[5, 1, 10])
    assert np.array_equal(_bits(pre), _bits(pre2)), "chunking changed bits"


def test_batch_composition_and_order_invariance():
    c = _case()
    rows = list(range(6))
    c.write_history("d", rows, 1)
    ref = _bits(c.decode_back("d", rows, 1))
    ref_att = c.sess.attn_out(6).clone()
    rng = np.random.default_rng(7)
    for size in (1, 2, 3, 5, 6):
        for _ in range(3):
            pick = list(rng.permutation(6)[:size])
            got = _bits(c.decode_back("d", pick, 1))
            assert np.array_equal(got, ref[pick]), (pick, got, ref[pick])
            att = c.sess.attn_out(size)
            assert torch.equal(att.view(torch.int16), ref_att.view(torch.int16)[pick])


def test_page_placement_invariance():
    c = _case(copies=3)
    rows = list(range(6))
    c.write_history("a", rows, 1)
    c.write_history("b", rows, 1)  # different pages from a shuffled pool
    a = _bits(c.decode_back("a", rows, 1))
    b = _bits(c.decode_back("b", rows, 1))
    assert c.sess.pages[("a", 5)] != c.sess.pages[("b", 5)]
    assert np.array_equal(a, b)


@pytest.mark.parametrize("kv_dtype", [0, 1], ids=["bf16", "fp8"])
def test_checkpoint_restore_into_a_new_pool_continues_bitwise(kv_dtype):
    """The first steps after a restore equal the run that never stopped (Bitwise-consistent
    RL post, section 2 on a correct backward and restore, and section 5's check of the
    first step after a checkpoint load).  Mid-decode the cache is checkpointed as the
    pool's bytes on the host plus each sequence's page list; a second session (its own
    pool at other addresses, another page shuffle) takes every sequence's pages back
    under new page ids; both sessions then decode the same next steps."""
    from gqa_case import GQACase
    kw = dict(ctx=SMALL_CTX, kv_dtype=kv_dtype, k_scale_exp=1 if kv_dtype else 0)
    a = GQACase(SMALL, list(range(6)), shuffle_seed=11, **kw)
    rows = MULTI
    a.write_history("s", rows, 4)
    for back in (4, 3):
        a.decode_back("s", rows, back)
    torch.cuda.synchronize()
    host = a.sess.pool.cpu()
    lists = {seq: list(ids) for seq, ids in a.sess.pages.items()}

    b = GQACase(SMALL, list(range(6)), shuffle_seed=977, **kw)
    pb = a.sess.page_bytes
    assert b.sess.page_bytes == pb and b.sess.pool.data_ptr() != a.sess.pool.data_ptr()
    for seq, ids in lists.items():
        b.sess.ensure(seq, len(ids) * 16)
        for old, new in zip(ids, b.sess.pages[seq]):
            b.sess.pool[new * pb:(new + 1) * pb].copy_(host[old * pb:(old + 1) * pb])
    assert any(b.sess.pages[seq] != ids for seq, ids in lists.items())
    for back in (2, 1):
        x = _bits(a.decode_back("s", rows, back))
        y = _bits(b.decode_back("s", rows, back))
        assert np.array_equal(x, y), back


def test_mixed_batch_prefill_with_decode_rows():
    """Decode rows inside a prefill call (one-token sequences) equal the decode path."""
    c = _case()
    rows = list(range(6))
    c.write_history("d", rows, 1)
    dec = _bits(c.decode_back("d", rows, 1))
    c.write_history("m", rows, 1)
    mix = _bits(c.prefill_last("m", rows, 1)[:, 0])
    assert np.array_equal(dec, mix)


def test_run_to_run_determinism():
    c = _case()
    rows = list(range(6))
    c.write_history("d", rows, 1)
    outs = [_bits(c.decode_back("d", rows, 1)) for _ in range(5)]
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


# Contexts at and across exact multiples of the 512-token split (and of the 64-token
# tile): the last split of a row is then full, and the decode grid has no partial split
# for it (the branch a row with a ragged tail never takes).
EDGE_CTX = [512, 520, 1024, 1030, 1536, 2048]


def test_split_multiple_contexts_decode_equals_prefill_and_oracle():
    from gqa_case import GQACase
    c = GQACase(SMALL, list(range(6)), ctx=EDGE_CTX)
    rows = list(range(6))
    n = 16
    c.write_history("d", rows, n)
    dec = torch.stack([c.decode_back("d", rows, back) for back in range(n, 0, -1)], dim=1)
    c.write_history("p", rows, n)
    pre = c.prefill_last("p", rows, n)
    assert np.array_equal(_bits(dec), _bits(pre)), "prefill != decode at split multiples"
    dn = dec.cpu().numpy()
    for i, r in enumerate(rows):
        for back in range(1, n + 1):
            ctx = c.ctx(r) - back + 1
            if ctx % 512 == 0 or back == 1:
                lp_o, _ = c.oracle_row(r, back)
                assert abs(dn[i, n - back] - lp_o) <= TOL, (r, ctx, dn[i, n - back], lp_o)


@pytest.mark.parametrize("kv_dtype", [0, 1])
def test_rejected_rows_give_nan_and_leave_batch_mates_unchanged(kv_dtype):
    """Rows the device-side checks reject come back NaN (ril.h: a context below 1 or past the
    batch's bound, a page id outside the pool, a target outside [0, V)); the other rows of
    the same batch keep their bits (batch invariance holds for broken batch-mates too)."""
    c = _case(kv_dtype=kv_dtype)
    rows = list(range(6))
    seqs = [("d", r) for r in rows]
    c.write_history("d", rows, 1)
    q, k, v, t, ctx = c.step_inputs(rows, 1)
    ref = _bits(c.sess.decode(seqs, ctx, targets=t, q=q, k=k, v=v))
    launch, out = c.sess.prepare_decode(seqs, ctx, targets=t, q=q, k=k, v=v)
    keep = launch.keep
    bound = max(ctx)
    stride = keep["pt"].shape[1]
    assert stride == math.ceil(bound / 16)
    keep["ctx"][1] = 0                      # no position
    keep["ctx"][2] = 16 * stride + 1        # past the bound; its new token's page is past the table
    keep["pt"][3, 1] = c.sess.pool.numel() // c.sess.page_bytes + 5  # outside the pool, inside row 3's context
    keep["tgt"][4] = SMALL.vocab            # a target outside the vocabulary
    launch()
    torch.cuda.synchronize()
    got = out.cpu()
    assert bool(torch.isnan(got[1:5]).all()), got
    assert np.array_equal(_bits(out)[[0, 5]], ref[[0, 5]])


def test_wide_rows_take_the_separate_merge_and_norm_and_stay_invariant():
    """Rows wider than the merge + RMSNorm kernel stages in LDS (256 q heads x 128 =
    32768 values) take the separate merge and RMSNorm launches: decode still equals the
    prefill recompute bit for bit and matches the oracle."""
    from gqa_case import GQACase
    w = wl.scaled(wl.GQA_DECODE_B64, rows=4, n_q_heads=256, n_kv_heads=16, vocab=512, d_head=256 * 128,
                  recompute_tokens=16)
    c = GQACase(w, list(range(4)), ctx=[17, 40, 530, 100])
    rows = list(range(4))
    n = 16
    c.write_history("d", rows, n)
    dec = torch.stack([c.decode_back("d", rows, back) for back in range(n, 0, -1)], dim=1)
    c.write_history("p", rows, n)
    pre = c.prefill_last("p", rows, n)
    assert np.array_equal(_bits(dec), _bits(pre))
    dn = dec.cpu().numpy()
    for i, r in enumerate(rows):
        lp, _ = c.oracle_row(r, 1)
        assert abs(dn[i, -1] - lp) <= TOL, (r, dn[i, -1], lp)


@pytest.mark.parametrize("model", ["g4", "g8", "g4_d64"])
def test_prefill_segment_lengths_across_column_blocks(model):
    """A prefill segment of n tokens fills a workgroup's two column blocks per wave in
    every pattern (block 1 empty, partial, full; a second workgroup): n tokens of one
    call equal n decode steps bitwise, for n around the blocks' sizes (16/G tokens per
    wave block, 8 waves); head_dim 128 and 64."""
    from gqa_case import GQACase
    base = {"g4": wl.GQA_DECODE_B64, "g8": wl.LONG_MIX.decode,
            "g4_d64": wl.scaled(wl.GQA_DECODE_B64, head_dim=64, d_head=32 * 64)}[model]
    n_max = 80
    w = wl.scaled(base, rows=3, vocab=2100, recompute_tokens=n_max)
    c = GQACase(w, [0, 1, 2], ctx=[n_max, 700, 1500])
    rows = [0, 1, 2]
    c.write_history("d", rows, n_max)
    dec = torch.stack([c.decode_back("d", rows, back) for back in range(n_max, 0, -1)], dim=1)
    c.write_history("p", rows, n_max)
    for n in (80, 65, 64, 63, 40, 33, 32, 31, 17, 16, 15, 5, 1):
        pre = c.prefill_last("p", rows, n)
        assert np.array_equal(_bits(pre), _bits(dec[:, n_max - n:])), n
    lp_o, _ = c.oracle_row(1, 33)
    assert abs(float(dec[1, n_max - 33]) - lp_o) <= TOL
