"""GPU tests at the full MLA workloads, in the launch configuration bench.py times:
absorbed MLA decode (128 rows, 128 heads, contexts 4096..32768) and sparse MLA over the
indexer's top-2048 (32 rows, contexts 65536).  Every row: prefill recompute of its last
16 positions bitwise equal to 16 decode steps (selection lists too, for the sparse
kind); sampled rows: oracle parity (and exact selection)."""

import numpy as np
import pytest
import torch

import workloads as wl

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.detach().cpu().contiguous().view(torch.int32).numpy()


def test_full_mla_prefill_equals_decode_and_oracle():
    from mla_case import MLACase
    w = wl.MLA_DECODE_B128
    rows = list(range(w.rows))
    c = MLACase(w, rows, max_rows=w.rows, max_tokens=w.rows * 16)
    n = 16
    c.write_history("d", rows, n)
    dec = torch.stack([c.decode_back("d", rows, b) for b in range(n, 0, -1)], dim=1)
    att = c.attn_out(len(rows)).float().cpu().numpy()
    c.write_history("p", rows, n)
    pre = c.prefill_last("p", rows, n)
    assert np.array_equal(_bits(dec), _bits(pre))
    lp = dec[:, -1].cpu().numpy()
    for r in (0, 77):
        lp_o, o_o = c.oracle_row(r)
        assert np.max(np.abs(att[r] - o_o)) < 2e-2, r
        assert abs(lp[r] - lp_o) <= 2e-2, (r, lp[r], lp_o)


def test_full_sparse_prefill_equals_decode_and_oracle():
    from sparse_case import SparseCase
    w = wl.SPARSE_MLA_B32
    rows = list(range(w.rows))
    c = SparseCase(w, rows, max_rows=w.rows, max_tokens=w.rows * 16)
    n = 16
    c.write_history("d", rows, n)
    dec, sels = [], []
    for b in range(n, 0, -1):
        s = torch.zeros((len(rows), w.topk), dtype=torch.int32, device="cuda")
        dec.append(c.decode_back("d", rows, b, selected_out=s))
        sels.append(s)
    dec = torch.stack(dec, dim=1)
    sel_dec = torch.stack(sels, dim=1)
    att = c.attn_out(len(rows)).float().cpu().numpy()
    c.write_history("p", rows, n)
    sel_pre = torch.zeros((len(rows) * n, w.topk), dtype=torch.int32, device="cuda")
    pre = c.prefill_last("p", rows, n, selected_out=sel_pre)
    assert np.array_equal(_bits(dec), _bits(pre))
    assert torch.equal(sel_dec.reshape(-1, w.topk), sel_pre)
    lp = dec[:, -1].cpu().numpy()
    last = sel_dec[:, -1].cpu().numpy()
    for r in (0, 21):
        lp_o, o_o, _, sel_o = c.oracle_row(r)
        assert np.array_equal(last[r], sel_o), r
        assert np.max(np.abs(att[r] - o_o)) < 2e-2, r
        assert abs(lp[r] - lp_o) <= 2e-2, (r, lp[r], lp_o)
