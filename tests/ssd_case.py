"""Shared harness for the Mamba-2 SSD mixer: session, history laid down by prefill calls,
decode steps, prefill of given positions, the mixer output view and the oracle for one
position.  Every computation goes through the C ABI."""

from __future__ import annotations

from typing import Dict, Sequence

import torch

import workloads as wl
from invariant_rl_logprob_amd import RIL_ATTN_SSD, ril_ws_attn_offset
from invariant_rl_logprob_amd.session import Session


class SSDCase:
    def __init__(self, w: wl.SSDDecode, rows: Sequence[int], *, ctx: Sequence[int] = None, device="cuda",
                 shuffle_seed=99, tags=2, max_rows=None, max_tokens=None, head=None):
        self.w = w
        self.rows = list(rows)
        self.data: Dict[int, dict] = {}
        for i, r in enumerate(self.rows):
            self.data[r] = wl.ssd_row(r, w, device=device, ctx=None if ctx is None else ctx[i])
        self.params = wl.ssd_params(w, device=device)
        if head is not None:
            self.params.update(head)
        self.max_tokens = max_tokens or max(len(self.rows) * w.recompute_tokens, 256)
        self.sess = Session(n_q_heads=w.n_heads, n_kv_heads=w.n_groups, head_dim=w.head_dim, vocab=w.vocab,
                            d_head=w.d_head, w_lm=self.params["w_lm"], w_o=self.params.get("w_o"),
                            max_rows=max_rows or max(len(self.rows), 1), max_tokens=self.max_tokens,
                            max_ctx=max(d["ctx"] for d in self.data.values()), pool_pages=tags * len(self.rows) + 4,
                            softmax_scale=1.0, rms_eps=w.rms_eps, shuffle_seed=shuffle_seed,
                            attn_kind=RIL_ATTN_SSD, ssm_A=self.params["A"], ssm_D=self.params["D"], device=device)
        self._oracle: Dict[int, tuple] = {}

    def ctx(self, r):
        return self.data[r]["ctx"]

    def _slices(self, r, a, b):
        d = self.data[r]
        return d["C"][a:b], d["B"][a:b], d["x"][a:b], d["dt"][a:b], d["target"][a:b]

    def prefill(self, tag, rows, starts, ends) -> torch.Tensor:
        """One prefill call: positions [starts[i], ends[i]) of each row; fp32 [total]."""
        cs, bs, xs, dts, ts = [], [], [], [], []
        for r, a, b in zip(rows, starts, ends):
            C, B, x, dt, t = self._slices(r, a, b)
            cs.append(C)
            bs.append(B)
            xs.append(x)
            dts.append(dt)
            ts.append(t)
        return self.sess.prefill([(tag, r) for r in rows], list(starts), targets=ts, qs=cs, ks=bs, vs=xs, dts=dts)

    def run_positions(self, tag, r, a, b, cuts: Sequence[int] = ()) -> torch.Tensor:
        """Positions [a, b) of one row in prefill calls cut at the offsets `cuts` (each call
        at most max_tokens long); fp32 [b - a]."""
        edges = sorted({a, b, *(a + c for c in cuts if 0 < c < b - a)})
        out = []
        for lo, hi in zip(edges, edges[1:]):
            for s in range(lo, hi, self.max_tokens):
                out.append(self.prefill(tag, [r], [s], [min(hi, s + self.max_tokens)]))
        return torch.cat(out)

    def history(self, tag, rows, upto_back: int) -> None:
        """Positions [0, ctx - upto_back) of each row, laid down by prefill calls."""
        for r in rows:
            n = self.ctx(r) - upto_back
            self.sess.ensure((tag, r), 1)
            if n > 0:
                self.run_positions(tag, r, 0, n)

    def decode_back(self, tag, rows, back: int) -> torch.Tensor:
        cs, bs, xs, dts, ts, ctx = [], [], [], [], [], []
        for r in rows:
            p = self.ctx(r) - back
            C, B, x, dt, t = self._slices(r, p, p + 1)
            cs.append(C[0])
            bs.append(B[0])
            xs.append(x[0])
            dts.append(dt[0])
            ts.append(t[0])
            ctx.append(p + 1)
        st = torch.stack
        return self.sess.decode([(tag, r) for r in rows], ctx, targets=st(ts).to(torch.int32), q=st(cs), k=st(bs),
                                v=st(xs), dt=st(dts))

    def prefill_last(self, tag, rows, c: int, chunks: Sequence[int] = None) -> torch.Tensor:
        """The last c positions of each row (after history to ctx - c) in calls of the given
        chunk lengths, all rows packed per call; fp32 [rows, c]."""
        chunks = list(chunks) if chunks else [c]
        assert sum(chunks) == c
        outs, done = [], 0
        for ch in chunks:
            starts = [self.ctx(r) - c + done for r in rows]
            outs.append(self.prefill(tag, rows, starts, [s + ch for s in starts]).view(len(rows), ch))
            done += ch
        return torch.cat(outs, dim=1)

    def y_out(self, rows: int) -> torch.Tensor:
        """bf16 [rows, H, 64] mixer output of the last call (a workspace view)."""
        off = ril_ws_attn_offset(self.sess.model)
        n = rows * self.w.n_heads * self.w.head_dim
        return self.sess.ws[off: off + 2 * n].view(torch.bfloat16).view(rows, self.w.n_heads, self.w.head_dim)

    def oracle_y(self, r):
        """The oracle's unrounded y [ctx, H, 64] of row r (every position), cached."""
        if r not in self._oracle:
            import oracle
            d = self.data[r]
            cpu = {k: v.cpu() for k, v in d.items() if k != "ctx"}
            y, _ = oracle.ssd_scan(cpu["x"], cpu["B"], cpu["C"], cpu["dt"].double().numpy(),
                                   self.params["A"].double().cpu().numpy(), self.params["D"].double().cpu().numpy())
            self._oracle[r] = y
        return self._oracle[r]

    def oracle_row(self, r, back: int = 1, with_logprob=True):
        """(logprob, unrounded y [H, 64]) of row r at position ctx - back."""
        import oracle
        p = self.ctx(r) - back
        y = self.oracle_y(r)[p]
        lp = None
        if with_logprob:
            lp = oracle.head_logprob(y, self.params["w_lm"].float().cpu().numpy(), int(self.data[r]["target"][p]),
                                     self.w.rms_eps, w_o=self.params["w_o"].float().cpu().numpy())
        return lp, y
