"""GPU tests of the W8A8 block-FP8 projections (proj_dtype = RIL_PROJ_W8A8_FP8: the
deployment GEMMs of the Bitwise-consistent RL post, section 4.1, with one accumulation
order for every M).

* The weight quantization writes exactly the oracle's codes and block exponents.
* The projection GEMM matches the exact product of the quantized operands (oracle
  fp8block.w8a8_matmul) to the output's bf16 rounding plus fp32 accumulation error, and
  its rows keep their bits whatever the number of rows (the three launch shapes).
* The token-input decoder (with and without its SwiGLU block) with every projection in
  W8A8: decode bitwise equal to prefill across batch orders and chunk sizes, and the
  logprobs within the end-to-end bar of the oracle with the same projections.

End-to-end bar: as for the W8A8 lm-head, an activation that sits within an ulp of an
E4M3 rounding boundary can take the other code when the GPU's bf16 input differs from
the oracle's by one ulp (fp32 against fp64 normalisation), which moves a logprob by a few
thousandths of a nat; the bar is 5e-2 per token with the median under 1e-2."""

import itertools
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from oracle import fp8block
from test_gpu_tiny_decoder import _bits, _prefill, _prompt_then_decode, _targets

pytestmark = pytest.mark.gpu

TOL_E2E = 5e-2


def _rand_bf16(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(torch.bfloat16)


@pytest.mark.parametrize("N,K", [(300, 256), (128, 128), (1000, 512), (64, 384)])
def test_quantize_weight_matches_oracle(N, K):
    import invariant_rl_logprob_amd as ril
    w = _rand_bf16((N, K), N + K, 0.05)
    w[3, 7] = float("nan")
    dst = torch.zeros(ril.ril_proj_fp8_bytes(N, K), dtype=torch.uint8, device="cuda")
    ril.ril_quantize_weight_fp8(w.cuda(), dst)
    torch.cuda.synchronize()
    got = dst.cpu().numpy()
    codes, e = oracle.quantize_weight_blocks(w.float().numpy())
    assert np.array_equal(got[:N * K].reshape(N, K), codes)
    ew = got[N * K:].view(np.int32).reshape(-(-N // 128), K // 128)
    assert np.array_equal(ew, np.where(e == fp8block.E_NAN, 255, e + 127))
    assert ew[0, 0] == 255  # the block holding the NaN


def _quant_rows(x):
    import invariant_rl_logprob_amd as ril
    rows, K = x.shape
    codes = torch.empty((rows, K), dtype=torch.uint8, device="cuda")
    exps = torch.empty((rows, K // 128), dtype=torch.int32, device="cuda")
    ril.ril_quantize_rows_fp8(x, codes, exps)
    return codes, exps


@pytest.mark.parametrize("M,N,K", [(1, 300, 256), (17, 128, 128), (100, 520, 512), (300, 256, 384)])
def test_proj_matches_exact_product(M, N, K):
    import invariant_rl_logprob_amd as ril
    x = _rand_bf16((M, K), 7 * M + N)
    w = _rand_bf16((N, K), 11 * N + K, 0.05)
    w8 = torch.empty(ril.ril_proj_fp8_bytes(N, K), dtype=torch.uint8, device="cuda")
    ril.ril_quantize_weight_fp8(w.cuda(), w8)
    codes, exps = _quant_rows(x.cuda())
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ril.ril_proj_w8a8(codes, exps, w8, N, out)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    xa, wa = x.float().numpy(), w.float().numpy()
    ref = oracle.w8a8_matmul(xa, wa)
    ca, ea = fp8block.quantize_rows(xa)
    cw, ew = fp8block.quantize_weight_blocks(wa)
    mag = np.abs(fp8block.dequant_rows(ca, ea)) @ np.abs(fp8block.dequant_weight_blocks(cw, ew)).T
    # one bf16 rounding of the output (half an ulp, 2^-9 relative) on top of the fp32 sums'
    # rounding (each of the K/128 accumulations and the products within a step: K * 2^-24)
    bound = 2.0 ** -8 * np.abs(ref) + K * 2.0 ** -23 * mag
    assert np.all(np.abs(got - ref) <= bound), float(np.max(np.abs(got - ref) / np.maximum(bound, 1e-30)))


def test_proj_rows_keep_their_bits_at_every_row_count():
    import invariant_rl_logprob_amd as ril
    N, K = 384, 512
    x = _rand_bf16((300, K), 5).cuda()
    w = _rand_bf16((N, K), 6, 0.05).cuda()
    w8 = torch.empty(ril.ril_proj_fp8_bytes(N, K), dtype=torch.uint8, device="cuda")
    ril.ril_quantize_weight_fp8(w, w8)
    got = {}
    # launch shapes: up to 16 rows one 16-row block per workgroup, up to 256 rows four
    # 16-row blocks per workgroup, past 256 rows the 256 x 256 tiles of the wide kernel
    # (its second 128-row group from row 128)
    for M in (1, 16, 17, 256, 257, 300):
        codes, exps = _quant_rows(x[:M])
        out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        ril.ril_proj_w8a8(codes, exps, w8, N, out)
        torch.cuda.synchronize()
        got[M] = out.view(torch.int16).cpu().numpy()
    for (M1, b1), (M2, b2) in itertools.combinations(got.items(), 2):
        n = min(M1, M2)
        assert np.array_equal(b1[:n], b2[:n]), (M1, M2)


def _session(W, wts, proj_dtype):
    from invariant_rl_logprob_amd import RIL_INPUT_TOKENS
    from invariant_rl_logprob_amd.session import Session
    mlp = {"d_ff": W.d_ff, "w_gate_up": wts["w_gate_up"], "w_down": wts["w_down"], "norm_mlp": wts["norm_mlp"]} \
        if W.d_ff else {}
    return Session(n_q_heads=W.n_q_heads, n_kv_heads=W.n_kv_heads, head_dim=W.head_dim, vocab=W.vocab,
                   d_head=W.d_model, d_model=W.d_model, w_lm=wts["w_lm"], embed=wts["embed"],
                   w_qkv=wts["w_qkv"], w_o=wts["w_o"], norm_attn=wts["norm_attn"],
                   norm_final=wts["norm_final"], max_rows=8, max_tokens=512, max_ctx=max(W.lengths),
                   pool_pages=4096, softmax_scale=1.0 / math.sqrt(W.head_dim), rms_eps=W.rms_eps,
                   shuffle_seed=23, input_mode=RIL_INPUT_TOKENS, proj_dtype=proj_dtype, **mlp)


@pytest.fixture(scope="module", params=["tiny", "tiny_mlp"])
def w8_model(request):
    W = wl.TINY if request.param == "tiny" else wl.TINY_MLP
    wts = wl.tiny_weights(W, device="cuda")
    toks = [wl.tiny_tokens(i, W, device="cuda") for i in range(len(W.lengths))]
    return W, _session(W, wts, 1), wts, toks


def test_w8a8_proj_decoder_matches_oracle(w8_model):
    W, s, wts, toks = w8_model
    lp = _prefill(s, "full", [0, 1, 2, 3], toks)
    errs = []
    for i in range(4):
        t = toks[i].cpu().numpy()
        tg = _targets(toks[i]).cpu().numpy()
        want = oracle.tiny_decoder_prefill(wts, t, tg, W.n_q_heads, W.n_kv_heads, W.head_dim, W.rms_eps,
                                           proj_w8a8=True)
        errs.append(np.abs(lp[i].cpu().numpy()[:-1] - want[:-1]))
    errs = np.concatenate(errs)
    print("W8A8 projections, |gpu - oracle|: max %.4g median %.4g" % (errs.max(), np.median(errs)))
    assert errs.max() <= TOL_E2E and np.median(errs) <= 1e-2, errs


def test_w8a8_proj_decode_bitwise_equals_prefill(w8_model):
    W, s, wts, toks = w8_model
    full = _prefill(s, "ref", [0, 1, 2, 3], toks)
    ref = {i: _bits(full[i][:-1]) for i in range(4)}
    orders = [[i] for i in range(4)] + [[2, 0], [3, 1]] + [list(p) for p in itertools.permutations(range(4))][::7]
    for n, order in enumerate(orders):
        got = _prompt_then_decode(s, ("o", n), order, toks, W.prompt_tokens)
        for i in order:
            assert np.array_equal(_bits(got[i]), ref[i]), (order, i)
        for i in order:
            s.release((("o", n), i))
    for ch in (1, 33):
        got = _prefill(s, ("c", ch), [3, 1, 0, 2], toks, chunk=ch)
        for i in range(4):
            assert np.array_equal(_bits(got[i][:-1]), ref[i]), (ch, i)


def test_w8a8_proj_differs_from_bf16(w8_model):
    W, s, wts, toks = w8_model
    b = _session(W, wts, 0)  # the same weights with bf16 projections
    got8 = _prefill(s, "d8", [0], toks)[0].cpu().numpy()
    got16 = _prefill(b, "d16", [0], toks)[0].cpu().numpy()
    assert not np.array_equal(got8, got16)
    assert np.max(np.abs(got8[:-1] - got16[:-1])) < 0.5


def test_w8a8_o_projection_with_mla():
    """Absorbed MLA (64 heads x latent 512: the o-projection's K is 32768) with a W8A8
    o-projection: 16 decode steps equal the prefill recompute bitwise, and the last
    position's logprob is within the end-to-end bar of the oracle with the same
    projection."""
    from mla_case import MLACase
    W = wl.scaled(wl.MLA_DECODE_B128, rows=4, n_heads=64, vocab=1000, d_head=256, recompute_tokens=16)
    c = MLACase(W, [0, 1, 2, 3], ctx=[70, 700, 2100, 33], proj_dtype=1)
    rows, n = [0, 1, 2, 3], 16
    c.write_history("d", rows, n)
    dec = torch.stack([c.decode_back("d", rows, back) for back in range(n, 0, -1)], dim=1)
    c.write_history("p", rows, n)
    pre = c.prefill_last("p", rows, n)
    assert np.array_equal(_bits(dec), _bits(pre))
    errs = [abs(float(dec[i, -1]) - c.oracle_row(r)[0]) for i, r in enumerate(rows)]
    print("MLA with a W8A8 o-projection, |gpu - oracle|:", errs)
    assert max(errs) <= TOL_E2E
