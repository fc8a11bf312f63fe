"""GPU tests of the Mamba-2 SSD mixer through the C ABI (Bitwise-consistent RL post, section
6: decode replays the prefill's chunked arithmetic; the zero-mismatch-rl README's
key-features table).

* Parity: the mixer output and the logprob of every checked position against the fp64
  oracle, which runs the recurrence one position at a time (oracle/ssd.py), at chunk
  boundaries (127, 128, 255, 256) and ragged positions.
* Invariance, bitwise: decode steps equal the prefill recompute; a sequence cut into
  prefill calls of any lengths (1, 33, 94, 127, 128, 129, ...) equals one whole-sequence
  call and equals decoding it position by position; a row's bits do not depend on its
  batch-mates or their order; a slot reused by a new sequence starts from zero state.

The output bar: the GPU rounds three operands to bf16 inside the chunk form (the decayed
C.B weights, the state entering a chunk, the decayed B of a chunk's state sums), each a
relative 2^-9, on top of the output's own bf16 rounding; with |y| ~ 1 that is within
2e-2 + 2e-2 |y| elementwise."""

import numpy as np
import pytest
import torch

import workloads as wl

pytestmark = pytest.mark.gpu

TOL = 2e-2
SMALL = wl.scaled(wl.SSD_DECODE_B64, rows=6, n_heads=8, n_groups=2, vocab=1000, d_head=256, recompute_tokens=16)
SMALL_CTX = [1, 100, 128, 129, 300, 700]


def _case(ctx=SMALL_CTX, **kw):
    from ssd_case import SSDCase
    return SSDCase(SMALL, list(range(len(ctx))), ctx=ctx, **kw)


def _bits(t):
    return t.detach().cpu().contiguous().view(torch.int32).numpy()


def _check_y(y_gpu, y_oracle, what):
    y_gpu = y_gpu.float().cpu().numpy()
    err = np.abs(y_gpu - y_oracle) - (TOL + TOL * np.abs(y_oracle))
    assert np.all(err <= 0), (what, float(np.max(np.abs(y_gpu - y_oracle))))


def test_ssd_decode_matches_oracle():
    c = _case()
    rows = list(range(6))
    c.history("d", rows, 1)
    lp = c.decode_back("d", rows, 1).cpu().numpy()
    y = c.y_out(len(rows))
    for i, r in enumerate(rows):
        lp_o, y_o = c.oracle_row(r)
        _check_y(y[i], y_o, r)
        assert abs(lp[i] - lp_o) <= TOL, (r, lp[i], lp_o)


def test_ssd_prefill_equals_decode_bitwise_across_chunk_boundaries():
    c = _case(ctx=[130, 257, 300, 700])
    rows = [0, 1, 2, 3]
    n = 16  # the windows cross positions 127/128 (row 0) and 255/256 (row 1)
    c.history("d", rows, n)
    dec, ys = [], []
    for back in range(n, 0, -1):
        dec.append(c.decode_back("d", rows, back))
        ys.append(c.y_out(len(rows)).clone())
    dec = torch.stack(dec, dim=1)
    c.history("p", rows, n)
    pre = c.prefill_last("p", rows, n)
    assert np.array_equal(_bits(dec), _bits(pre))
    yp = c.y_out(len(rows) * n).view(len(rows), n, SMALL.n_heads, SMALL.head_dim)
    for j in range(n):
        assert torch.equal(ys[j].view(torch.int16), yp[:, j].contiguous().view(torch.int16)), j
    dn = dec.cpu().numpy()
    for i, r in enumerate(rows):
        for back in (1, 3, n):
            lp_o, _ = c.oracle_row(r, back)
            assert abs(dn[i, n - back] - lp_o) <= TOL, (r, back)


def test_ssd_any_cut_of_a_sequence_gives_the_same_bits():
    L = 300
    c = _case(ctx=[L], tags=4)
    whole = c.run_positions("whole", 0, 0, L)
    cuts = []
    at = 0
    for step in (1, 33, 94, 127, 128, 129, 5, 1):
        at += step
        cuts.append(at)
    pieces = c.run_positions("cut", 0, 0, L, cuts=cuts)
    assert np.array_equal(_bits(whole), _bits(pieces))
    # position by position through the decode entry point
    c.sess.ensure(("dec", 0), 1)
    steps = [c.decode_back("dec", [0], L - p)[0] for p in range(L)]
    assert np.array_equal(_bits(whole), _bits(torch.stack(steps)))
    wl_ = whole.cpu().numpy()
    for p in (0, 1, 127, 128, 129, 255, 256, L - 1):
        lp_o, _ = c.oracle_row(0, L - p)
        assert abs(wl_[p] - lp_o) <= TOL, p
    _check_y(c.y_out(1)[0], c.oracle_y(0)[L - 1], "last decode step")


def test_ssd_batch_composition_and_order():
    c = _case()
    rows = list(range(6))
    c.history("d", rows, 1)
    ref = _bits(c.decode_back("d", rows, 1))
    rng = np.random.default_rng(5)
    for size in (1, 2, 4, 6):
        pick = [int(x) for x in rng.permutation(6)[:size]]
        assert np.array_equal(_bits(c.decode_back("d", pick, 1)), ref[pick]), pick


def test_ssd_reused_slot_starts_from_zero_state():
    c = _case(ctx=[700, 300])
    c.history("a", [0], 1)
    first = _bits(c.decode_back("a", [1], 300))  # row 1 at position 0 in a fresh slot
    # release row 0's slot (its state and chunk inputs are those of 699 positions) and
    # start row 1 over in it
    slot = c.sess.pages[("a", 0)][0]
    c.sess.release(("a", 0))
    c.sess.ensure(("b", 1), 1)
    assert c.sess.pages[("b", 1)] == [slot]
    again = _bits(c.decode_back("b", [1], 300))
    assert np.array_equal(first, again)


def test_ssd_repeated_decode_step_gives_the_same_bits():
    """A decode step can be replayed: the step that completes a chunk writes the next
    chunk's state beside the one it reads (row 0's position 255 completes chunk 1)."""
    c = _case(ctx=[256, 300])
    rows = [0, 1]
    c.history("d", rows, 2)
    a1 = _bits(c.decode_back("d", rows, 2))
    a2 = _bits(c.decode_back("d", rows, 2))
    b1 = _bits(c.decode_back("d", rows, 1))
    b2 = _bits(c.decode_back("d", rows, 1))
    assert np.array_equal(a1, a2) and np.array_equal(b1, b2)
    c.history("p", rows, 2)
    pre = _bits(c.prefill_last("p", rows, 2))
    assert np.array_equal(pre[:, 0], a1) and np.array_equal(pre[:, 1], b1)
