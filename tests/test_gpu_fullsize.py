"""GPU tests at the full decode workload (64 rows, 32 q / 8 kv heads, head_dim 128,
contexts in [512, 8192], lm-head 4096 x 129280), in the launch configuration bench.py
times: sampled rows against the fp64 oracle, prefill vs decode bitwise on every row for
the last 16 and the last 64 positions, and the decode step bitwise across batch sizes
1..64, eight row permutations each."""

import numpy as np
import pytest
import torch

import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def full():
    from gqa_case import GQACase
    w = wl.GQA_DECODE_B64
    rows = list(range(w.rows))
    case = GQACase(w, rows, device="cuda", shuffle_seed=0x5EED, copies=4, max_tokens=w.rows * 64)
    n = 16
    case.write_history("d", rows, n)
    dec = torch.stack([case.decode_back("d", rows, back) for back in range(n, 0, -1)], dim=1)
    case.write_history("p", rows, n)
    pre = case.prefill_last("p", rows, n)
    torch.cuda.synchronize()
    return case, rows, dec, pre


def _bits(t):
    return t.detach().cpu().view(torch.int32).numpy()


def test_full_prefill_equals_decode(full):
    case, rows, dec, pre = full
    assert np.array_equal(_bits(dec), _bits(pre))


def test_full_last_64_positions_prefill_equals_decode(full):
    case, rows, _, _ = full
    n = 64
    case.write_history("d64", rows, n)
    dec = torch.stack([case.decode_back("d64", rows, back) for back in range(n, 0, -1)], dim=1)
    case.write_history("p64", rows, n)
    pre = case.prefill_last("p64", rows, n)
    assert np.array_equal(_bits(dec), _bits(pre))


def test_full_sampled_rows_match_oracle(full):
    case, rows, dec, pre = full
    lp = dec[:, -1].cpu().numpy()
    for r in (0, 17, 40, 63):
        want, _ = case.oracle_row(r)
        assert abs(lp[r] - want) <= 2e-2, (r, lp[r], want)


def test_full_batch_size_and_permutation_invariance(full):
    case, rows, dec, pre = full
    ref = _bits(dec[:, -1])
    rng = np.random.default_rng(11)
    for size in (1, 2, 3, 4, 8, 16, 32, 63, 64):
        for _ in range(8):
            pick = [int(x) for x in rng.permutation(len(rows))[:size]]
            got = _bits(case.decode_back("d", pick, 1))
            assert np.array_equal(got, ref[pick]), (size, pick[:8])
