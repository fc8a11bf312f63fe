"""GPU tests of the long-context mixed batch (GQA 64 q / 8 kv heads, 8192 -> 4096 output
projection): long sequences prefilled in chunks of several sizes, every prefill call also
carrying the decode rows that advance in that step, in seeded orders.  The logprob of
every position is bitwise identical across chunk sizes and batch mixes, the decode rows'
logprobs equal those of plain decode steps, and sampled positions match the fp64 oracle."""

import numpy as np
import pytest
import torch

import workloads as wl

pytestmark = pytest.mark.gpu

TOL = 2e-2

# Scaled: two sequences of 4396 tokens (a ragged last chunk), chunk sizes 256 and 1024,
# six decode rows whose contexts span a tile, a split and several splits.
SMALL = wl.LongMix(n_seqs=2, seq_len=4396, chunks=(256, 1024), decode_tokens=4)
SMALL_CTX = [4, 65, 513, 1100, 3000, 5000]


def _bits(t):
    return t.detach().cpu().contiguous().view(torch.int32).numpy()


def test_long_mix_chunk_and_mix_invariance_small():
    from long_case import LongMixCase
    c = LongMixCase(SMALL, rows=len(SMALL_CTX), decode_ctx=SMALL_CTX)
    ref_dec = c.decode_reference()
    runs = [c.run_schedule(256, 0, "a"), c.run_schedule(1024, 0, "b"), c.run_schedule(1024, 1, "c")]
    long0, dec0 = runs[0]
    assert bool(torch.isfinite(long0).all()) and bool(torch.isfinite(dec0).all())
    for lp_long, lp_dec in runs[1:]:
        assert np.array_equal(_bits(lp_long), _bits(long0))
        assert np.array_equal(_bits(lp_dec), _bits(dec0))
    assert np.array_equal(_bits(dec0), _bits(ref_dec))
    got = long0.cpu().numpy()
    for s, p in ((0, 0), (0, 255), (0, 256), (1, 1023), (1, 1024), (0, 4395)):
        lp_o = c.oracle_long(s, p)
        assert abs(got[s, p] - lp_o) <= TOL, (s, p, got[s, p], lp_o)
    dec = dec0.cpu().numpy()
    for r, j in ((0, 0), (3, 2), (5, 3)):
        lp_o = c.oracle_decode(r, j)
        assert abs(dec[r, j] - lp_o) <= TOL, (r, j, dec[r, j], lp_o)
