"""The product's S13 measurement (invariant_rl_logprob_amd.metrics) against the oracle's
independent diff/k3 definitions, plus its exact-zero and bit-pattern behaviour."""

import numpy as np

import oracle
from invariant_rl_logprob_amd.metrics import mismatch

RNG = np.random.default_rng(5)


def test_mismatch_matches_oracle_definitions():
    a = (-RNG.random(5000) * 12).astype(np.float32)
    b = (a + RNG.normal(0, 1e-3, a.size)).astype(np.float32)
    m = mismatch(a, b)
    d = oracle.diff_stats(a, b)
    assert m["max"] == d["max"] and m["mean"] == d["mean"] and m["std"] == d["std"] and m["p_max"] == d["p_max"]
    assert abs(m["k3"] - oracle.k3_mean(b, a)) <= 1e-18
    assert not m["bitwise_equal"] and m["tokens"] == 5000


def test_mismatch_zero_iff_bits_equal():
    a = (-RNG.random(100) * 12).astype(np.float32)
    m = mismatch(a, a.copy())
    assert m["bitwise_equal"] and m["max"] == m["mean"] == m["std"] == m["k3"] == 0.0
    b = a.copy()
    b[7] = np.nextafter(b[7], np.float32(0))
    m = mismatch(a, b)
    assert not m["bitwise_equal"] and m["max"] > 0 and m["k3"] > 0
