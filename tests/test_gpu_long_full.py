"""The long-context mixed batch at its own size: 8 sequences of 131072 tokens (GQA 64 q /
8 kv heads, head_dim 128, 8192 -> 4096 output projection, the 4096 x 129280 lm-head)
prefilled in chunks of 512, 2048 and 8192 tokens, two seeded batch mixes each, every
prefill call also carrying the 256 decode rows (contexts U[1024, 131072]) that advance in
that step.  The post's phase-consistency contract (Bitwise-consistent RL post, section 2):
* every one of the 1,048,576 long positions has the same bits in all six runs;
* the decode rows' 16 positions, computed inside the mixed prefill calls, equal 16 plain
  decode steps of all 256 rows, bit for bit;
* positions at the chunk boundaries (511, 512, 2047, 2048, 8191, 8192) and the last
  position match the fp64 oracle within 2e-2 nats, as do sampled decode rows.
The six schedules share one set of inputs (a module fixture) and run as separate tests so
each stays well inside its time limit."""

import numpy as np
import pytest
import torch

import workloads as wl

pytestmark = pytest.mark.gpu

TOL = 2e-2
SCHEDULES = [(8192, 0), (8192, 1), (2048, 0), (2048, 1), (512, 0), (512, 1)]
BOUNDARY = (511, 512, 2047, 2048, 8191, 8192, 131071)

_state = {}


def _bits(t):
    return t.detach().cpu().contiguous().view(torch.int32).numpy()


@pytest.fixture(scope="module")
def case():
    from long_case import LongMixCase
    c = LongMixCase(wl.LONG_MIX, progress=lambda msg: print("[long]", msg, flush=True))
    print(f"[long] {len(c.seqs)} x {c.L} tokens, {len(c.rows)} decode rows, sum ctx {sum(c.ctx.values())}",
          flush=True)
    yield c
    c.sess.close()
    _state.clear()
    del c
    torch.cuda.empty_cache()


def _reference(case):
    if "ref" not in _state:
        _state["ref"] = _bits(case.decode_reference())
    return _state["ref"]


def _first_run(case):
    if "long" not in _state:
        chunk, mix = SCHEDULES[0]
        lp_long, lp_dec = case.run_schedule(chunk, mix, ("full", chunk, mix))
        _state["long"], _state["dec"] = _bits(lp_long), _bits(lp_dec)
        _state["long_f"] = lp_long.cpu().numpy()
        _state["dec_f"] = lp_dec.cpu().numpy()
    return _state["long"], _state["dec"]


@pytest.mark.timeout(600)
def test_full_decode_rows_plain_steps(case):
    ref = _reference(case)
    assert ref.shape == (256, 16)
    assert np.all(np.isfinite(ref.view(np.float32)))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("chunk,mix", SCHEDULES)
def test_full_schedule_bitwise_equal(case, chunk, mix):
    ref = _reference(case)
    long0, dec0 = _first_run(case)
    if (chunk, mix) == SCHEDULES[0]:
        lp_long, lp_dec = long0, dec0
    else:
        lo, de = case.run_schedule(chunk, mix, ("full", chunk, mix))
        lp_long, lp_dec = _bits(lo), _bits(de)
    print(f"[long] chunk {chunk} mix {mix} done", flush=True)
    assert np.all(np.isfinite(lp_long.view(np.float32)))
    assert np.array_equal(lp_long, long0), (chunk, mix, int(np.sum(lp_long != long0)))
    assert np.array_equal(lp_dec, ref), (chunk, mix, int(np.sum(lp_dec != ref)))


@pytest.mark.timeout(600)
def test_full_boundary_positions_match_oracle(case):
    _first_run(case)
    got = _state["long_f"]
    for s in (0, 7):
        for p in BOUNDARY:
            lp_o = case.oracle_long(s, p)
            assert abs(got[s, p] - lp_o) <= TOL, (s, p, float(got[s, p]), lp_o)
    dec = _state["dec_f"]
    longest = max(case.rows, key=lambda r: case.ctx[r])
    for r, j in ((0, 0), (longest, 15)):
        lp_o = case.oracle_decode(r, j)
        assert abs(dec[r, j] - lp_o) <= TOL, (r, j, float(dec[r, j]), lp_o)
