"""GPU tests of the bf16 projection GEMM (S4) at its own boundary, ril_proj_bf16: the
kernel every QKV, O and MLP projection of the model runs.

The contract (Bitwise-consistent RL post, section 4.1: one accumulation order for every
M, no split-K) is checked element by element against the oracle's projection:
* integer-valued operands in {-2..2}: every fp32 partial sum is exact (|sum| <= 4K <=
  2^18), so the output equals bf16 of the int64 product bit for bit, and with an
  integer residual bf16(R + bf16(product)) bit for bit;
* random bf16 operands: the output is bf16(exact) or its neighbour (the fp32 sum's
  rounding can move it across a rounding boundary), within the fp32 accumulation bound,
  and in practice equal for almost every element; the residual epilogue equals the fp32
  sum of the residual and the rounded product, rounded to bf16, bit for bit;
* a row's bits do not depend on how many rows share the call, across every kernel the
  row count and K select (16- and 64-row tiles, the few-row long-K kernel with 1, 2 and 4
  row blocks, the 256 x 256 tiled kernel past 256 rows).
"""

import itertools

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

ROWS = (1, 16, 17, 64, 65, 256, 257, 300)
N = 300  # ragged for the 64-, 128- and 256-column tiles


def _run(a, w, residual=None):
    import invariant_rl_logprob_amd as ril
    out = torch.empty((a.shape[0], w.shape[0]), dtype=torch.bfloat16, device="cuda")
    ril.ril_proj_bf16(a, w, out, residual=residual)
    torch.cuda.synchronize()
    return out


def _bits(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy()


def _bf16_of_f32(x):
    """torch's round-to-nearest-even fp32 -> bf16, as float64."""
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


@pytest.mark.parametrize("K", [256, 8192, 65536])
def test_integer_operands_bit_exact(K):
    g = torch.Generator().manual_seed(K)
    a = torch.randint(-2, 3, (max(ROWS), K), generator=g)
    w = torch.randint(-2, 3, (N, K), generator=g)
    r = torch.randint(-50, 51, (max(ROWS), N), generator=g)
    p = (a.to(torch.int64) @ w.to(torch.int64).T).numpy()
    want = _bf16_of_f32(p)
    want_r = _bf16_of_f32(r.numpy().astype(np.float32) + want.astype(np.float32))
    ad, wd, rd = (t.to(torch.bfloat16).cuda() for t in (a, w, r))
    for M in ROWS:
        got = _run(ad[:M], wd).double().cpu().numpy()
        assert np.array_equal(got, want[:M]), (K, M, int(np.sum(got != want[:M])))
        got_r = _run(ad[:M], wd, rd[:M]).double().cpu().numpy()
        assert np.array_equal(got_r, want_r[:M]), (K, M)
    # the oracle's projection reproduces the integer product too (both sides pinned)
    assert np.array_equal(oracle.projection(a.numpy(), w.numpy(), r.numpy())[:5], want_r[:5])


@pytest.mark.parametrize("K", [256, 8192, 65536])
def test_random_operands_match_oracle_and_keep_bits_at_every_row_count(K):
    g = torch.Generator().manual_seed(1000 + K)
    a = torch.randn((max(ROWS), K), generator=g).to(torch.bfloat16)
    w = (torch.randn((N, K), generator=g) * 0.02).to(torch.bfloat16)
    r = torch.randn((max(ROWS), N), generator=g).to(torch.bfloat16)
    an, wn = a.double().numpy(), w.double().numpy()
    ref = oracle.projection(an, wn)
    mag = np.abs(an) @ np.abs(wn).T
    # one bf16 step of the result (at most 2^-7 relative) plus the fp32 sum's rounding
    bound = 2.0 ** -7 * np.abs(ref) + K * 2.0 ** -23 * mag
    ad, wd, rd = a.cuda(), w.cuda(), r.cuda()
    bits = {}
    for M in ROWS:
        out = _run(ad[:M], wd)
        got = out.double().cpu().numpy()
        err = np.abs(got - ref[:M])
        assert np.all(err <= bound[:M]), (K, M, float(np.max(err / bound[:M])))
        assert np.mean(got == ref[:M]) >= 0.99, (K, M, float(np.mean(got == ref[:M])))
        # residual epilogue: bf16(R + bf16(acc)), the sum formed in fp32
        out_r = _run(ad[:M], wd, rd[:M])
        want_r = (rd[:M].float() + out.float()).to(torch.bfloat16)
        assert torch.equal(out_r.view(torch.int16), want_r.view(torch.int16)), (K, M)
        bits[M] = _bits(out)
    for (M1, b1), (M2, b2) in itertools.combinations(bits.items(), 2):
        n = min(M1, M2)
        assert np.array_equal(b1[:n], b2[:n]), (K, M1, M2)


def test_strided_operands_and_residual_in_place():
    # rows of a wider matrix (lda > K), a weight slice (ldw > K), and the residual
    # updated in place (out == residual), as a caller's fused buffers would do
    K, Nw = 512, 96
    g = torch.Generator().manual_seed(5)
    big = torch.randn((40, K + 64), generator=g).to(torch.bfloat16).cuda()
    wbig = (torch.randn((Nw, K + 32), generator=g) * 0.05).to(torch.bfloat16).cuda()
    a, w = big[:, 16:16 + K], wbig[:, :K]
    assert a.stride(0) == K + 64 and w.stride(0) == K + 32
    ref = _run(a.contiguous(), w.contiguous())
    assert torch.equal(_run(a, w).view(torch.int16), ref.view(torch.int16))
    res = torch.randn((40, Nw), generator=g).to(torch.bfloat16).cuda()
    want = (res.float() + ref.float()).to(torch.bfloat16)
    import invariant_rl_logprob_amd as ril
    ril.ril_proj_bf16(a, w, res, residual=res)
    torch.cuda.synchronize()
    assert torch.equal(res.view(torch.int16), want.view(torch.int16))


def test_output_rounding_is_nearest_even_on_ties():
    """The projection's bf16 store rounds to nearest, ties to even (Bitwise-consistent RL
    post, section 4.4, condition 1), checked through the GEMM itself.  Each output is
    x + s*y*2^-j for bf16 x, y with y a few half-units of x's last place: two products
    whose fp32 sum is exact, so the fp32 accumulator holds the exact value and the bf16
    store alone decides the bits.  Many of these sums fall exactly halfway between two
    bf16 values (both parities of x's last bit); two rows check the tie at the top of
    the range (bf16's largest value plus half its spacing rounds to infinity) and the
    value just below it.  Expected: the oracle's projection, bf16 of the exact sum."""
    rng = np.random.default_rng(8)
    M, K = 300, 1024  # M > 256: the 256 x 256 kernel; its first 256 / 64 / 16 rows: the others
    E = rng.integers(-100, 101, M)
    x = rng.choice([-1.0, 1.0], M) * (1 + rng.integers(0, 128, M) / 128.0) * np.ldexp(1.0, E)
    y = rng.choice([-1.0, 1.0], M) * (1 + rng.integers(0, 8, M) / 8.0) * np.ldexp(1.0, E - 8 + rng.integers(0, 3, M))
    x[-2:] = float.fromhex("0x1.fep127")          # bf16's largest finite value
    y[-2:] = [2.0 ** 119, 2.0 ** 118]            # half its spacing (a tie), a quarter
    a = np.zeros((M, K))
    a[:, 0], a[:, 1] = x, y
    w = np.zeros((16, K))
    w[:, 0] = 1.0
    w[:, 1] = np.where(np.arange(16) < 8, 1.0, -1.0) * np.ldexp(1.0, -(np.arange(16) % 8))
    assert np.array_equal(oracle.bf16(a), a) and np.array_equal(oracle.bf16(w), w)
    exact = a @ w.T
    _, ex = np.frexp(exact)
    frac = np.abs(exact) / np.ldexp(1.0, ex - 8) % 1.0
    tie = frac == 0.5
    assert tie.sum() >= 150                                # plenty of exact ties
    want = oracle.projection(a, w)
    assert np.isinf(want[-2, 0]) and want[-1, 0] == x[-1]
    up = np.abs(want[tie]) > np.abs(exact[tie])
    assert up.sum() >= 50 and (~up).sum() >= 50            # both ways to the even value
    dev = lambda v: torch.from_numpy(v).to(torch.bfloat16).cuda()  # noqa: E731
    A, W = dev(a), dev(w)
    want_bits = torch.from_numpy(want).to(torch.bfloat16).view(torch.int16).numpy()
    for m in (M, 256, 64, 16):
        got = _bits(_run(A[:m].contiguous(), W))
        assert np.array_equal(got, want_bits[:m]), m
