"""Shared harness for sparse (indexer + top-k) MLA: session, history, decode steps,
prefill recompute, and the oracle for one row.  Every computation goes through the C ABI."""

from __future__ import annotations

import math
from typing import Dict, Sequence

import torch

import workloads as wl
from invariant_rl_logprob_amd import RIL_ATTN_MLA_SPARSE, ril_ws_attn_offset
from invariant_rl_logprob_amd.session import Session


class SparseCase:
    def __init__(self, w: wl.SparseMLADecode, rows: Sequence[int], *, ctx: Sequence[int] = None, device="cuda",
                 shuffle_seed=777, copies=2, split_entries=256, max_rows=None, max_tokens=None, head=None,
                 kv_dtype=0, scale_exp=0, max_ctx=None):
        self.w = w
        self.rows = list(rows)
        self.data: Dict[int, dict] = {}
        for i, r in enumerate(self.rows):
            self.data[r] = wl.sparse_row(r, w, device=device, ctx=None if ctx is None else ctx[i])
        self.head = head if head is not None else wl.mla_head_weights(
            wl.MLADecode(n_heads=w.n_heads, kv_rank=w.kv_rank, vocab=w.vocab, d_head=w.d_head, seed=w.seed),
            device=device)
        max_ctx = max_ctx or max(d["ctx"] for d in self.data.values())
        pages = sum(math.ceil(d["ctx"] / 16) for d in self.data.values()) * copies + 8
        self.scale = 1.0 / math.sqrt(w.scale_dim)
        self.sess = Session(n_q_heads=w.n_heads, n_kv_heads=1, head_dim=w.kv_rank, rope_dim=w.rope_dim,
                            index_heads=w.index_heads, index_dim=w.index_dim, topk=w.topk, vocab=w.vocab,
                            d_head=w.d_head, w_lm=self.head["w_lm"], w_o=self.head.get("w_o"),
                            max_rows=max_rows or max(len(self.rows), 1),
                            max_tokens=max_tokens or len(self.rows) * w.recompute_tokens, max_ctx=max_ctx,
                            pool_pages=pages, softmax_scale=self.scale, rms_eps=w.rms_eps,
                            shuffle_seed=shuffle_seed, split_tokens=split_entries,
                            attn_kind=RIL_ATTN_MLA_SPARSE, kv_dtype=kv_dtype, k_scale_exp=scale_exp,
                            v_scale_exp=scale_exp, device=device)
        self.fp8_exp = scale_exp if kv_dtype else None  # FP8 latent cache: its scale exponent

    def ctx(self, r):
        return self.data[r]["ctx"]

    def write_history(self, tag, rows, upto_back: int):
        seqs, starts, cs, ks = [], [], [], []
        for r in rows:
            d = self.data[r]
            n = d["ctx"] - upto_back
            if n <= 0:
                self.sess.ensure((tag, r), 1)
                continue
            seqs.append((tag, r))
            starts.append(0)
            cs.append(d["c"][:n])
            ks.append(d["k_index"][:n])
        if seqs:
            self.sess.write_kv(seqs, starts, cs, None, k_index=ks)

    def decode_back(self, tag, rows, back: int, selected_out=None, ctx_bound=None) -> torch.Tensor:
        q, c, qi, ki, t, ctx = [], [], [], [], [], []
        for r in rows:
            d = self.data[r]
            R = d["q"].shape[0]
            p = d["ctx"] - back
            q.append(d["q"][R - back])
            qi.append(d["q_index"][R - back])
            c.append(d["c"][p])
            ki.append(d["k_index"][p])
            t.append(d["target"][R - back])
            ctx.append(p + 1)
        st = torch.stack
        return self.sess.decode([(tag, r) for r in rows], ctx, targets=st(t).to(torch.int32), q=st(q), k=st(c),
                                q_index=st(qi), k_index=st(ki), selected_out=selected_out, ctx_bound=ctx_bound)

    def prefill_last(self, tag, rows, n: int, selected_out=None) -> torch.Tensor:
        seqs, starts, qs, cs, qis, kis, ts = [], [], [], [], [], [], []
        for r in rows:
            d = self.data[r]
            R = d["q"].shape[0]
            p0 = d["ctx"] - n
            seqs.append((tag, r))
            starts.append(p0)
            qs.append(d["q"][R - n:])
            qis.append(d["q_index"][R - n:])
            cs.append(d["c"][p0:])
            kis.append(d["k_index"][p0:])
            ts.append(d["target"][R - n:])
        return self.sess.prefill(seqs, starts, targets=ts, qs=qs, ks=cs, q_index=qis, k_index=kis,
                                 selected_out=selected_out).view(len(rows), n)

    def attn_out(self, rows: int) -> torch.Tensor:
        off = ril_ws_attn_offset(self.sess.model)
        n = rows * self.w.n_heads * self.w.kv_rank
        return self.sess.ws[off: off + 2 * n].view(torch.bfloat16).view(rows, self.w.n_heads, self.w.kv_rank)

    def cached(self, c):
        """The latent rows as the cache gives them back: the bf16 values, or with an FP8
        cache the oracle's E4M3 round trip of them at the cache's scale."""
        if self.fp8_exp is None:
            return c
        import oracle
        return oracle.kv_fp8_roundtrip(c.float().cpu().numpy(), self.fp8_exp)

    def oracle_row(self, r, back: int = 1, with_logprob=True):
        """(lp, attention output, fp32 indexer scores, selection) of row r at position ctx - back."""
        import oracle
        d = self.data[r]
        R = d["q"].shape[0]
        p = d["ctx"] - back
        scores = oracle.indexer_scores_fp32(d["q_index"][R - back], d["k_index"][: p + 1])
        sel = oracle.topk_select(scores, self.w.topk, tie="lowest")
        o = oracle.sparse_mla_row_attention(d["q"][R - back], self.cached(d["c"][: p + 1]), sel, self.scale,
                                            self.w.kv_rank)
        lp = None
        if with_logprob:
            lp = oracle.head_logprob(o, self.head["w_lm"].float().cpu().numpy(), int(d["target"][R - back]),
                                     self.w.rms_eps, w_o=self.head["w_o"].float().cpu().numpy())
        return lp, o, scores, sel
