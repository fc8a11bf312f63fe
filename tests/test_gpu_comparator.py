"""GPU tests of the comparator policy (ril_set_policy RIL_POLICY_SHAPE_DERIVED), the
non-invariant build the benchmark reports beside the method: it is still a correct
forward (oracle parity within the same tolerance), it really departs from the invariant
bits, and switching back to RIL_POLICY_INVARIANT restores them exactly."""

import numpy as np
import pytest
import torch

import workloads as wl
from invariant_rl_logprob_amd import RIL_POLICY_INVARIANT, RIL_POLICY_SHAPE_DERIVED, RilError

pytestmark = pytest.mark.gpu

TOL = 2e-2


def _bits(t):
    return t.detach().cpu().contiguous().view(torch.int32).numpy()


def test_gqa_comparator_correct_and_reversible():
    from gqa_case import GQACase
    w = wl.scaled(wl.GQA_DECODE_B64, rows=5, vocab=2100, recompute_tokens=1)
    ctx = [1, 70, 600, 1100, 3000]
    rows = list(range(5))
    c = GQACase(w, rows, ctx=ctx)
    c.write_history("d", rows, 1)
    inv = c.decode_back("d", rows, 1)
    inv_att = _bits(c.sess.attn_out(5))
    oracle_lp = [c.oracle_row(r)[0] for r in rows]
    differs = False
    for split in (0, 64, 256, 1024):
        c.sess.set_policy(RIL_POLICY_SHAPE_DERIVED, split)
        lp = c.decode_back("d", rows, 1).cpu().numpy()
        for i in rows:
            assert abs(lp[i] - oracle_lp[i]) <= TOL, (split, i, lp[i], oracle_lp[i])
        differs |= not np.array_equal(_bits(c.sess.attn_out(5)), inv_att)
    assert differs, "the shape-derived splits never changed a bit"
    c.sess.set_policy(RIL_POLICY_INVARIANT)
    assert np.array_equal(_bits(c.decode_back("d", rows, 1)), _bits(inv))
    with pytest.raises(RilError):
        c.sess.set_policy(RIL_POLICY_SHAPE_DERIVED, 100)


def test_mla_comparator_split_k_correct_and_reversible():
    from mla_case import MLACase
    w = wl.scaled(wl.MLA_DECODE_B128, rows=4, n_heads=64, vocab=1000, d_head=256, recompute_tokens=1)
    ctx = [1, 700, 2100, 4200]
    rows = list(range(4))
    c = MLACase(w, rows, ctx=ctx)
    c.write_history("d", rows, 1)
    inv = c.decode_back("d", rows, 1)
    # the head's 32768 -> 256 projection has fewer tiles than compute units: split-K
    c.sess.set_policy(RIL_POLICY_SHAPE_DERIVED)
    lp = c.decode_back("d", rows, 1).cpu().numpy()
    for i, r in enumerate(rows):
        lp_o, _ = c.oracle_row(r)
        assert abs(lp[i] - lp_o) <= TOL, (r, lp[i], lp_o)
    c.sess.set_policy(RIL_POLICY_INVARIANT)
    assert np.array_equal(_bits(c.decode_back("d", rows, 1)), _bits(inv))
