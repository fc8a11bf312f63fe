"""GPU tests of the FP8 (OCP E4M3) KV cache, GQA (Bitwise-consistent RL post, section 4.2:
FP8 storage, one write path, one dequantizing read shared by every phase).

* The codes the write path stores: every bf16 value, as K and as V, at three scale
  exponents, byte for byte against the oracle's E4M3 encoder (integer work: bit-exact).
* Parity: decode and prefill logprobs and attention outputs against the fp64 oracle run
  over the K/V the cache gives back (its decode of those codes).
* Invariance: decode steps equal the prefill recompute bitwise, in chunks too, and a
  row's bits do not depend on its batch-mates or their order."""

import math

import numpy as np
import pytest
import torch

import oracle
import workloads as wl

pytestmark = pytest.mark.gpu

TOL = 2e-2
SMALL = wl.scaled(wl.GQA_DECODE_B64, rows=6, vocab=2100, recompute_tokens=16)
SMALL_CTX = [1, 17, 64, 65, 600, 1100]
MULTI = [1, 2, 3, 4, 5]
FP8 = 1


def _bits(t):
    return t.detach().cpu().contiguous().view(torch.int32).numpy()


def _case(k_exp=0, v_exp=0, **kw):
    from gqa_case import GQACase
    return GQACase(SMALL, list(range(6)), ctx=SMALL_CTX, kv_dtype=FP8, k_scale_exp=k_exp, v_scale_exp=v_exp,
                   **kw)


def _k_off(t, d):   # byte of K (t, d) in an FP8 page block (the layout ril.h points to)
    return 2 * ((d >> 6) * 512 + ((d & 31) >> 3) * 128 + ((t & 7) >> 2) * 64 + (t >> 3) * 32 + (t & 3) * 8) + \
        ((d >> 5) & 1) * 8 + (d & 7)


def _v_off(t, d, D):
    return 16 * D + (t >> 3) * 8 * D + ((d >> 5) * 16 + (d & 15)) * 16 + ((d >> 4) & 1) * 8 + (t & 7)


@pytest.mark.parametrize("k_exp,v_exp", [(0, 0), (3, -2), (-5, 1)])
def test_fp8_codes_of_every_bf16_value(k_exp, v_exp):
    from invariant_rl_logprob_amd.session import Session
    D, Hkv, T = 128, 1, 512            # 512 tokens x 128 dims = every bf16 bit pattern once
    vals = torch.arange(0, 1 << 16, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    k = vals.view(T, Hkv * D).cuda()
    v = vals.roll(12345).view(T, Hkv * D).cuda()     # a different value at each V position
    w_lm = torch.zeros(64, 4 * D, dtype=torch.bfloat16, device="cuda")
    s = Session(n_q_heads=4, n_kv_heads=Hkv, head_dim=D, vocab=64, d_head=4 * D, w_lm=w_lm, max_rows=1,
                max_tokens=1, max_ctx=T, pool_pages=T // 16 + 4, softmax_scale=1.0, shuffle_seed=5,
                kv_dtype=FP8, k_scale_exp=k_exp, v_scale_exp=v_exp)
    s.write_kv(["x"], [0], [k.view(T, Hkv, D)], [v.view(T, Hkv, D)])
    torch.cuda.synchronize()
    pool = s.pool.cpu().numpy()
    pages = s.pages["x"]
    t_idx = np.arange(T)
    d_idx = np.arange(D)
    base = (np.array(pages)[t_idx // 16] * s.page_bytes)[:, None]
    tt = (t_idx % 16)[:, None]
    dd = d_idx[None, :]
    kbytes = pool[base + np.vectorize(_k_off)(tt, dd)]
    vbytes = pool[base + np.vectorize(lambda a, b: _v_off(a, b, D))(tt, dd)]
    xk = k.cpu().to(torch.float64).numpy()
    xv = v.cpu().to(torch.float64).numpy()
    want_k = oracle.fp8.kv_fp8_store(xk, k_exp)
    want_v = oracle.fp8.kv_fp8_store(xv, v_exp)
    assert np.array_equal(kbytes, want_k), np.argwhere(kbytes != want_k)[:5]
    assert np.array_equal(vbytes, want_v), np.argwhere(vbytes != want_v)[:5]


def test_fp8_decode_matches_oracle():
    c = _case()
    rows = list(range(6))
    c.write_history("d", rows, 1)
    lp = c.decode_back("d", rows, 1).cpu().numpy()
    att = c.sess.attn_out(len(rows)).float().cpu().numpy()
    for i, r in enumerate(rows):
        lp_o, o_o = c.oracle_row(r)
        assert abs(lp[i] - lp_o) <= TOL, (r, lp[i], lp_o)
        assert np.max(np.abs(att[i] - o_o)) < 2e-2, (r, np.max(np.abs(att[i] - o_o)))


def test_fp8_scaled_prefill_matches_oracle():
    c = _case(k_exp=-1, v_exp=2)
    rows = MULTI
    c.write_history("p", rows, 16)
    lps = c.prefill_last("p", rows, 16).cpu().numpy()
    for i, r in enumerate(rows):
        for back in (1, 9, 16):
            lp_o, _ = c.oracle_row(r, back)
            assert abs(lps[i, 16 - back] - lp_o) <= TOL, (r, back, lps[i, 16 - back], lp_o)


def test_fp8_decode_bitwise_equals_prefill_and_chunking():
    c = _case()
    rows = MULTI
    n = 16
    c.write_history("d", rows, n)
    dec = torch.stack([c.decode_back("d", rows, back) for back in range(n, 0, -1)], dim=1)
    c.write_history("p", rows, n)
    pre = c.prefill_last("p", rows, n)
    assert np.array_equal(_bits(dec), _bits(pre)), "prefill != decode"
    pre2 = c.prefill_last("p", rows, n, chunks=[5, 1, 10])
    assert np.array_equal(_bits(pre), _bits(pre2)), "chunking changed bits"
    s = oracle.diff_stats(dec.double().cpu().numpy().ravel(), pre.double().cpu().numpy().ravel())
    assert s["max"] == s["mean"] == s["std"] == 0.0


def test_fp8_batch_composition_and_order_invariance():
    c = _case()
    rows = list(range(6))
    c.write_history("d", rows, 1)
    ref = _bits(c.decode_back("d", rows, 1))
    rng = np.random.default_rng(11)
    for size in (1, 2, 4, 6):
        for _ in range(2):
            pick = list(rng.permutation(6)[:size])
            assert np.array_equal(_bits(c.decode_back("d", pick, 1)), ref[pick]), pick


def test_fp8_differs_from_bf16_cache():
    """The FP8 cache is a different model numerically: same inputs, different logprobs
    (so the tests above are not passing on a bf16 read)."""
    from gqa_case import GQACase
    a = _case()
    b = GQACase(SMALL, list(range(6)), ctx=SMALL_CTX)
    rows = [4, 5]
    a.write_history("d", rows, 1)
    b.write_history("d", rows, 1)
    assert not np.array_equal(_bits(a.decode_back("d", rows, 1)), _bits(b.decode_back("d", rows, 1)))


def test_fp8_split_multiple_contexts_decode_equals_prefill_and_oracle():
    # contexts at and across multiples of the 512-token split with the FP8 cache
    from gqa_case import GQACase
    c = GQACase(SMALL, list(range(4)), ctx=[512, 1030, 1536, 2048], kv_dtype=FP8, k_scale_exp=1, v_scale_exp=-1)
    rows = list(range(4))
    n = 16
    c.write_history("d", rows, n)
    dec = torch.stack([c.decode_back("d", rows, back) for back in range(n, 0, -1)], dim=1)
    c.write_history("p", rows, n)
    pre = c.prefill_last("p", rows, n)
    assert np.array_equal(_bits(dec), _bits(pre))
    dn = dec.cpu().numpy()
    for i, r in enumerate(rows):
        for back in range(1, n + 1):
            if (c.ctx(r) - back + 1) % 512 == 0 or back == 1:
                lp_o, _ = c.oracle_row(r, back)
                assert abs(dn[i, n - back] - lp_o) <= TOL, (r, back)


@pytest.mark.parametrize("v_exp", [0, -4])
def test_fp8_read_path_returns_every_code_exactly(v_exp):
    """Every E4M3 code read back through the attention, decode and prefill: with one
    position of context and q = 0, each output element is that position's V value
    exactly (softmax weight 1, the other MFMA entries zeroed), so the attention output
    must equal the oracle's decode of the stored codes exactly -- subnormal codes, the
    largest magnitudes -- and be NaN for both NaN codes.  (Zero compares by value: the
    MFMA adds the other, zeroed entries, and -0 + 0 is +0.)"""
    from invariant_rl_logprob_amd.session import Session
    D, Hkv = 128, 8
    codes = (np.arange(Hkv * D) % 256).astype(np.uint8)    # every code four times
    vals = oracle.fp8.kv_fp8_load(codes, v_exp)             # exact in bf16; NaN for S.1111.111
    nan = np.isnan(vals)
    want = torch.from_numpy(vals).to(torch.bfloat16)
    v = want.view(1, Hkv * D).cuda()
    zeros = torch.zeros(1, Hkv * D, dtype=torch.bfloat16, device="cuda")
    w_lm = torch.zeros(64, Hkv * D, dtype=torch.bfloat16, device="cuda")
    s = Session(n_q_heads=Hkv, n_kv_heads=Hkv, head_dim=D, vocab=64, d_head=Hkv * D, w_lm=w_lm, max_rows=1,
                max_tokens=1, max_ctx=16, pool_pages=8, softmax_scale=1.0, shuffle_seed=3, kv_dtype=FP8,
                v_scale_exp=v_exp)
    t0 = torch.zeros(1, dtype=torch.int32, device="cuda")
    s.decode(["d"], [1], targets=t0, q=zeros, k=zeros, v=v)
    dec = s.attn_out(1).reshape(-1).cpu()
    s.prefill(["p"], [0], targets=[t0], qs=[zeros], ks=[zeros], vs=[v])
    pre = s.attn_out(1).reshape(-1).cpu()
    torch.cuda.synchronize()
    keep = ~torch.from_numpy(nan)
    for got in (dec, pre):
        assert np.array_equal(torch.isnan(got).numpy(), nan)
        g, w = got[keep].double().numpy(), want[keep].double().numpy()
        assert np.array_equal(g, w), (np.flatnonzero(g != w)[:8], codes[keep.numpy()][g != w][:8])
