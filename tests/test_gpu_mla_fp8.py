"""GPU tests of the FP8 (OCP E4M3) latent cache of MLA, dense and sparse (Bitwise-consistent
RL post, section 4.2: FP8 storage, one write path, one dequantizing read shared by every
phase; the zero-mismatch-rl README lists FlashMLA sparse attention over an FP8 KV cache).

* The codes the write path stores: every bf16 value as a latent, at three scale
  exponents, byte for byte against the oracle's E4M3 encoder (integer work: bit-exact);
  the sparse kind's fp32 indexer keys beside them, bit for bit.
* Parity: decode and prefill logprobs and attention outputs against the fp64 oracle run
  over the latents the cache gives back (the oracle's round trip of them); the sparse
  selection equals the oracle's exactly (the indexer keys stay fp32).
* Invariance: decode steps equal the prefill recompute bitwise, across the 2048-token
  split and at the top-k boundary, and a row's bits do not depend on its batch-mates."""

import numpy as np
import pytest
import torch

import oracle
import workloads as wl

pytestmark = pytest.mark.gpu

TOL = 2e-2
FP8 = 1
MLA_SMALL = wl.scaled(wl.MLA_DECODE_B128, rows=5, n_heads=64, vocab=1000, d_head=256, recompute_tokens=16)
MLA_CTX = [1, 65, 700, 2056, 4200]
SP_SMALL = wl.scaled(wl.SPARSE_MLA_B32, rows=4, n_heads=64, vocab=1000, d_head=256, topk=256,
                     recompute_tokens=16)
SP_CTX = [1, 256, 257, 2100]


def _bits(t):
    return t.detach().cpu().contiguous().view(torch.int32).numpy()


def _mla(ctx=MLA_CTX, scale_exp=1, **kw):
    from mla_case import MLACase
    return MLACase(MLA_SMALL, list(range(len(ctx))), ctx=ctx, kv_dtype=FP8, scale_exp=scale_exp, **kw)


def _sparse(ctx=SP_CTX, scale_exp=-2, **kw):
    from sparse_case import SparseCase
    return SparseCase(SP_SMALL, list(range(len(ctx))), ctx=ctx, split_entries=64, kv_dtype=FP8,
                      scale_exp=scale_exp, **kw)


@pytest.mark.parametrize("scale_exp", [0, 3, -5])
@pytest.mark.parametrize("sparse", [False, True], ids=["dense", "sparse"])
def test_latent_codes_of_every_bf16_value(scale_exp, sparse):
    from invariant_rl_logprob_amd import RIL_ATTN_MLA, RIL_ATTN_MLA_SPARSE
    from invariant_rl_logprob_amd.session import Session
    D = 576
    T = -(-(1 << 16) // D)  # 114 tokens: every bf16 bit pattern at least once
    vals = torch.arange(0, T * D, dtype=torch.int32).remainder(1 << 16).to(torch.int16).view(torch.bfloat16)
    c = vals.view(T, D).cuda()
    keys = torch.randn(T, 128, generator=torch.Generator().manual_seed(5)).cuda() if sparse else None
    extra = dict(index_heads=64, index_dim=128, topk=256) if sparse else {}
    s = Session(n_q_heads=64, n_kv_heads=1, head_dim=512, rope_dim=64, vocab=64, d_head=64 * 512,
                w_lm=torch.zeros(64, 64 * 512, dtype=torch.bfloat16, device="cuda"), max_rows=1, max_tokens=1,
                max_ctx=T, pool_pages=T // 16 + 4, softmax_scale=1.0, shuffle_seed=5,
                attn_kind=RIL_ATTN_MLA_SPARSE if sparse else RIL_ATTN_MLA, kv_dtype=FP8, k_scale_exp=scale_exp,
                v_scale_exp=scale_exp, **extra)
    assert s.page_bytes == 16 * D + (16 * 128 * 4 if sparse else 0)
    s.write_kv(["x"], [0], [c], None, k_index=[keys] if sparse else None)
    torch.cuda.synchronize()
    pool = s.pool.cpu().numpy()
    pages = np.array(s.pages["x"])
    t = np.arange(T)
    base = pages[t // 16] * s.page_bytes + (t % 16) * D
    got = pool[base[:, None] + np.arange(D)[None, :]]
    want = oracle.fp8.kv_fp8_store(c.cpu().to(torch.float64).numpy(), scale_exp)
    assert np.array_equal(got, want), np.argwhere(got != want)[:5]
    if sparse:
        kb = pages[t // 16] * s.page_bytes + 16 * D + (t % 16) * 512
        kgot = pool[kb[:, None] + np.arange(512)[None, :]]
        assert np.array_equal(kgot, keys.cpu().numpy().view(np.uint8).reshape(T, 512))
    s.close()


def test_mla_fp8_decode_matches_oracle():
    c = _mla()
    rows = list(range(5))
    c.write_history("d", rows, 1)
    lp = c.decode_back("d", rows, 1).cpu().numpy()
    att = c.attn_out(len(rows)).float().cpu().numpy()
    for i, r in enumerate(rows):
        lp_o, o_o = c.oracle_row(r)
        assert np.max(np.abs(att[i] - o_o)) < 2e-2, (r, np.max(np.abs(att[i] - o_o)))
        assert abs(lp[i] - lp_o) <= TOL, (r, lp[i], lp_o)


def test_mla_fp8_prefill_equals_decode_bitwise_across_the_split():
    c = _mla(ctx=[2048, 2056, 4096, 700], scale_exp=-3)
    rows = [0, 1, 2, 3]
    n = 16
    c.write_history("d", rows, n)
    dec = torch.stack([c.decode_back("d", rows, back) for back in range(n, 0, -1)], dim=1)
    c.write_history("p", rows, n)
    pre = c.prefill_last("p", rows, n)
    assert np.array_equal(_bits(dec), _bits(pre))
    dn = dec.cpu().numpy()
    for i, r in enumerate(rows):
        for back in (1, 9, 16):
            lp_o, _ = c.oracle_row(r, back)
            assert abs(dn[i, n - back] - lp_o) <= TOL, (r, back, dn[i, n - back], lp_o)


def test_mla_fp8_batch_invariance_and_differs_from_bf16():
    from mla_case import MLACase
    c = _mla()
    rows = list(range(5))
    c.write_history("d", rows, 1)
    ref = _bits(c.decode_back("d", rows, 1))
    rng = np.random.default_rng(7)
    for size in (1, 2, 3, 5):
        pick = [int(x) for x in rng.permutation(5)[:size]]
        assert np.array_equal(_bits(c.decode_back("d", pick, 1)), ref[pick]), pick
    b = MLACase(MLA_SMALL, rows, ctx=MLA_CTX)
    b.write_history("d", rows, 1)
    assert not np.array_equal(_bits(b.decode_back("d", rows, 1)), ref)


def test_mla_fp8_128_heads_two_groups():
    from mla_case import MLACase
    w = wl.scaled(wl.MLA_DECODE_B128, rows=2, n_heads=128, vocab=600, d_head=128, recompute_tokens=4)
    c = MLACase(w, [0, 1], ctx=[300, 2500], kv_dtype=FP8, scale_exp=2)
    c.write_history("d", [0, 1], 4)
    dec = torch.stack([c.decode_back("d", [0, 1], b) for b in (4, 3, 2, 1)], dim=1)
    att = c.attn_out(2).float().cpu().numpy()
    for i in range(2):
        lp_o, o_o = c.oracle_row(i)
        assert np.max(np.abs(att[i] - o_o)) < 2e-2
        assert abs(float(dec[i, -1]) - lp_o) <= TOL
    c.write_history("p", [0, 1], 4)
    assert np.array_equal(_bits(dec), _bits(c.prefill_last("p", [0, 1], 4)))


def test_sparse_fp8_decode_selection_and_parity():
    c = _sparse()
    rows = list(range(4))
    c.write_history("d", rows, 1)
    sel = torch.full((4, SP_SMALL.topk), -7, dtype=torch.int32, device="cuda")
    lp = c.decode_back("d", rows, 1, selected_out=sel).cpu().numpy()
    att = c.attn_out(4).float().cpu().numpy()
    sel = sel.cpu().numpy()
    for i, r in enumerate(rows):
        lp_o, o_o, _, sel_o = c.oracle_row(r)
        assert np.array_equal(sel[i], sel_o), r
        assert np.max(np.abs(att[i] - o_o)) < 2e-2, r
        assert abs(lp[i] - lp_o) <= TOL, (r, lp[i], lp_o)


def test_sparse_fp8_prefill_equals_decode_bitwise():
    c = _sparse(ctx=[256, 257, 300, 2100])
    rows = [0, 1, 2, 3]
    n = 12
    c.write_history("d", rows, n)
    sd = torch.empty((len(rows), SP_SMALL.topk), dtype=torch.int32, device="cuda")
    dec, sels = [], []
    for back in range(n, 0, -1):
        dec.append(c.decode_back("d", rows, back, selected_out=sd))
        sels.append(sd.clone())
    dec = torch.stack(dec, dim=1)
    c.write_history("p", rows, n)
    sp = torch.empty((len(rows) * n, SP_SMALL.topk), dtype=torch.int32, device="cuda")
    pre = c.prefill_last("p", rows, n, selected_out=sp)
    assert np.array_equal(_bits(dec), _bits(pre))
    sp = sp.view(len(rows), n, -1)
    for j in range(n):
        assert torch.equal(sels[j], sp[:, j]), j
