"""Shared GQA test/bench harness: build a session for a workload, lay down history,
run decode steps and prefill recomputes.  Inputs come from ``workloads``; every
computation goes through the C ABI."""

from __future__ import annotations

import math
from typing import Dict, List, Sequence

import torch

import workloads as wl
from invariant_rl_logprob_amd.session import Session


class GQACase:
    def __init__(self, w: wl.GQADecode, rows: Sequence[int], *, ctx: Sequence[int] = None,
                 device="cuda", shuffle_seed=1234, copies=2, max_tokens=None, head=None, kv_dtype=0,
                 k_scale_exp=0, v_scale_exp=0, lm_dtype=0):
        self.w = w
        self.kv = (kv_dtype, k_scale_exp, v_scale_exp)
        self.lm_dtype = lm_dtype
        self.rows = list(rows)
        self.device = device
        self.data: Dict[int, dict] = {}
        for i, r in enumerate(self.rows):
            self.data[r] = wl.gqa_row(r, w, device=device, ctx=None if ctx is None else ctx[i])
        self.head = head if head is not None else wl.gqa_head_weights(w, device=device)
        max_ctx = max(d["ctx"] for d in self.data.values())
        pages = sum(math.ceil(d["ctx"] / 16) for d in self.data.values()) * copies + 8
        R = w.recompute_tokens
        self.sess = Session(n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads, head_dim=w.head_dim,
                            vocab=w.vocab, d_head=w.d_head, w_lm=self.head["w_lm"], w_o=self.head.get("w_o"),
                            max_rows=max(len(self.rows), 1), max_tokens=max_tokens or len(self.rows) * R,
                            max_ctx=max_ctx, pool_pages=pages, softmax_scale=1.0 / math.sqrt(w.head_dim),
                            rms_eps=w.rms_eps, shuffle_seed=shuffle_seed, kv_dtype=kv_dtype,
                            k_scale_exp=k_scale_exp, v_scale_exp=v_scale_exp, lm_dtype=lm_dtype, device=device)

    def ctx(self, r):
        return self.data[r]["ctx"]

    def step_inputs(self, rows, back: int):
        """Decode inputs of each row at position ctx - back (back = 1: the last position)."""
        q, k, v, t, c = [], [], [], [], []
        for r in rows:
            d = self.data[r]
            R = d["q"].shape[0]
            p = d["ctx"] - back
            q.append(d["q"][R - back])
            k.append(d["k"][p])
            v.append(d["v"][p])
            t.append(d["target"][R - back])
            c.append(p + 1)
        st = lambda xs: torch.stack(xs).contiguous()  # noqa: E731
        return st(q), st(k), st(v), torch.stack(t).to(torch.int32), c

    def write_history(self, tag, rows, upto_back: int):
        """Positions [0, ctx - upto_back) of each row into the pages of (tag, row)."""
        seqs, starts, ks, vs = [], [], [], []
        for r in rows:
            d = self.data[r]
            n = d["ctx"] - upto_back
            if n <= 0:
                self.sess.ensure((tag, r), 1)
                continue
            seqs.append((tag, r))
            starts.append(0)
            ks.append(d["k"][:n])
            vs.append(d["v"][:n])
        if seqs:
            self.sess.write_kv(seqs, starts, ks, vs)

    def decode_back(self, tag, rows, back: int) -> torch.Tensor:
        q, k, v, t, c = self.step_inputs(rows, back)
        return self.sess.decode([(tag, r) for r in rows], c, targets=t, q=q, k=k, v=v)

    def prefill_last(self, tag, rows, c: int, chunks: Sequence[int] = None) -> torch.Tensor:
        """Prefill each row's last c positions (after history [0, ctx-c)); chunks split the c
        tokens into consecutive prefill calls.  Returns fp32 [len(rows), c]."""
        chunks = list(chunks) if chunks else [c]
        assert sum(chunks) == c
        outs = []
        done = 0
        for ch in chunks:
            seqs, starts, qs, ks, vs, ts = [], [], [], [], [], []
            for r in rows:
                d = self.data[r]
                R = d["q"].shape[0]
                p0 = d["ctx"] - c + done
                seqs.append((tag, r))
                starts.append(p0)
                qs.append(d["q"][R - c + done: R - c + done + ch])
                ks.append(d["k"][p0: p0 + ch])
                vs.append(d["v"][p0: p0 + ch])
                ts.append(d["target"][R - c + done: R - c + done + ch])
            lp = self.sess.prefill(seqs, starts, targets=ts, qs=qs, ks=ks, vs=vs)
            outs.append(lp.view(len(rows), ch))
            done += ch
        return torch.cat(outs, dim=1)

    def oracle_row(self, r, back: int = 1):
        """fp64 oracle logprob and attention output of row r at position ctx - back."""
        import oracle
        d = self.data[r]
        R = d["q"].shape[0]
        p = d["ctx"] - back
        q = oracle.widen(d["q"][R - back])
        K = oracle.widen(d["k"][: p + 1])
        V = oracle.widen(d["v"][: p + 1])
        if self.kv[0] == 1:  # FP8 cache: the model attends over what the cache gives back
            K = oracle.kv_fp8_roundtrip(K, self.kv[1])
            V = oracle.kv_fp8_roundtrip(V, self.kv[2])
        scale = 1.0 / math.sqrt(self.w.head_dim)
        o = oracle.gqa_row_attention(q, K, V, scale)
        w_o = self.head.get("w_o")
        lp = oracle.gqa_row_logprob(q, K, V, scale, self.head["w_lm"].float().cpu().numpy(),
                                    int(d["target"][R - back]), self.w.rms_eps,
                                    w_o=None if w_o is None else w_o.float().cpu().numpy(),
                                    lm_w8a8=self.lm_dtype == 1)
        return lp, o
