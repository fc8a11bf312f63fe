"""Shared MLA test/bench harness: session, latent history, decode steps, prefill
recompute and the oracle for one row.  Every computation goes through the C ABI."""

from __future__ import annotations

import math
from typing import Dict, Sequence

import torch

import workloads as wl
from invariant_rl_logprob_amd import RIL_ATTN_MLA
from invariant_rl_logprob_amd.session import Session


class MLACase:
    def __init__(self, w: wl.MLADecode, rows: Sequence[int], *, ctx: Sequence[int] = None, device="cuda",
                 shuffle_seed=4321, copies=2, split_tokens=2048, max_rows=None, max_tokens=None, head=None,
                 proj_dtype=0, kv_dtype=0, scale_exp=0):
        self.w = w
        self.rows = list(rows)
        self.data: Dict[int, dict] = {}
        for i, r in enumerate(self.rows):
            self.data[r] = wl.mla_row(r, w, device=device, ctx=None if ctx is None else ctx[i])
        self.head = head if head is not None else wl.mla_head_weights(w, device=device)
        max_ctx = max(d["ctx"] for d in self.data.values())
        pages = sum(math.ceil(d["ctx"] / 16) for d in self.data.values()) * copies + 8
        self.scale = 1.0 / math.sqrt(w.scale_dim)
        self.sess = Session(n_q_heads=w.n_heads, n_kv_heads=1, head_dim=w.kv_rank, rope_dim=w.rope_dim,
                            vocab=w.vocab, d_head=w.d_head, w_lm=self.head["w_lm"], w_o=self.head.get("w_o"),
                            max_rows=max_rows or max(len(self.rows), 1),
                            max_tokens=max_tokens or len(self.rows) * w.recompute_tokens, max_ctx=max_ctx,
                            pool_pages=pages, softmax_scale=self.scale, rms_eps=w.rms_eps,
                            shuffle_seed=shuffle_seed, split_tokens=split_tokens, attn_kind=RIL_ATTN_MLA,
                            proj_dtype=proj_dtype, kv_dtype=kv_dtype, k_scale_exp=scale_exp,
                            v_scale_exp=scale_exp, device=device)
        self.proj_w8a8 = proj_dtype == 1
        self.fp8_exp = scale_exp if kv_dtype else None  # FP8 latent cache: its scale exponent

    def ctx(self, r):
        return self.data[r]["ctx"]

    def write_history(self, tag, rows, upto_back: int):
        seqs, starts, cs = [], [], []
        for r in rows:
            d = self.data[r]
            n = d["ctx"] - upto_back
            if n <= 0:
                self.sess.ensure((tag, r), 1)
                continue
            seqs.append((tag, r))
            starts.append(0)
            cs.append(d["c"][:n])
        if seqs:
            self.sess.write_kv(seqs, starts, cs, None)

    def decode_back(self, tag, rows, back: int) -> torch.Tensor:
        q, c, t, ctx = [], [], [], []
        for r in rows:
            d = self.data[r]
            R = d["q"].shape[0]
            p = d["ctx"] - back
            q.append(d["q"][R - back])
            c.append(d["c"][p])
            t.append(d["target"][R - back])
            ctx.append(p + 1)
        return self.sess.decode([(tag, r) for r in rows], ctx, targets=torch.stack(t).to(torch.int32),
                                q=torch.stack(q), k=torch.stack(c))

    def prefill_last(self, tag, rows, c: int) -> torch.Tensor:
        seqs, starts, qs, cs, ts = [], [], [], [], []
        for r in rows:
            d = self.data[r]
            R = d["q"].shape[0]
            p0 = d["ctx"] - c
            seqs.append((tag, r))
            starts.append(p0)
            qs.append(d["q"][R - c:])
            cs.append(d["c"][p0:])
            ts.append(d["target"][R - c:])
        return self.sess.prefill(seqs, starts, targets=ts, qs=qs, ks=cs).view(len(rows), c)

    def attn_out(self, rows: int) -> torch.Tensor:
        off = self.sess.ws_attn_offset if hasattr(self.sess, "ws_attn_offset") else None
        from invariant_rl_logprob_amd import ril_ws_attn_offset
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
        import oracle
        d = self.data[r]
        R = d["q"].shape[0]
        p = d["ctx"] - back
        o = oracle.mla_row_attention(d["q"][R - back], self.cached(d["c"][: p + 1]), self.scale, self.w.kv_rank)
        lp = None
        if with_logprob:
            lp = oracle.head_logprob(o, self.head["w_lm"].float().cpu().numpy(), int(d["target"][R - back]),
                                     self.w.rms_eps, w_o=self.head["w_o"].float().cpu().numpy(),
                                     proj_w8a8=self.proj_w8a8)
        return lp, o
