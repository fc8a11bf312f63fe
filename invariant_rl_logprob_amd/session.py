"""Host-side resource handling around the C ABI (no arithmetic of the method).

A ``Session`` owns one model handle, its workspace, a KV pool with its host page
allocator, and a page list per sequence.  It turns per-sequence torch tensors into
the C batch descriptors and calls the library on the current torch stream.  Device
memory comes from torch; every computation happens in libril.so.
"""

from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence

import torch

from . import (RIL_ATTN_GQA, RIL_ATTN_SSD, RIL_INPUT_QKV, RIL_INPUT_TOKENS, make_decode_batch, make_prefill_batch,
               ril_decode_graph_create, ril_decode_step_logprobs, ril_graph_destroy, ril_graph_launch, ril_kv_alloc, ril_kv_assign, ril_kv_free, ril_kv_page_bytes,
               ril_kv_release, ril_kv_write, ril_lm_head_packed_bytes, ril_model_create, ril_model_desc,
               ril_model_destroy, ril_pack_lm_head, ril_prefill_logprobs, ril_set_policy,
               ril_lm_head_fp8_packed_bytes, ril_pack_lm_head_fp8, RIL_LM_BF16, RIL_LM_W8A8_FP8,
               ril_lm_head_logprobs, RIL_PROJ_BF16, RIL_PROJ_W8A8_FP8, ril_proj_fp8_bytes, ril_quantize_weight_fp8,
               ril_workspace_bytes, ril_ws_attn_offset)

PAGE = 16


def _i32(x, device):
    return torch.as_tensor(x, dtype=torch.int32).to(device)


def _cat(xs):
    return None if xs is None else torch.cat(list(xs)).contiguous()


def _c(x):
    return None if x is None else x.contiguous()


class Session:
    """One model + one KV pool on one device."""

    def __init__(self, *, n_q_heads, n_kv_heads, head_dim, vocab, d_head, w_lm, max_rows, max_tokens,
                 max_ctx, pool_pages, softmax_scale, rms_eps=1e-6, split_tokens=512, shuffle_seed=0,
                 input_mode=RIL_INPUT_QKV, d_model=0, embed=None, w_qkv=None, w_o=None, norm_attn=None,
                 norm_final=None, attn_kind=RIL_ATTN_GQA, rope_dim=0, index_heads=0, index_dim=0, topk=0,
                 kv_dtype=0, k_scale_exp=0, v_scale_exp=0, d_ff=0, w_gate_up=None, w_down=None, norm_mlp=None,
                 lm_dtype=RIL_LM_BF16, proj_dtype=RIL_PROJ_BF16, ssm_A=None, ssm_D=None, device="cuda"):
        self.device = torch.device(device)
        # SSD mixer: one cache slot ("page") per sequence; A and D fp32 [H] on the device
        self.ssd = attn_kind == RIL_ATTN_SSD
        if self.ssd:
            ssm_A = ssm_A.to(self.device, torch.float32).contiguous()
            ssm_D = ssm_D.to(self.device, torch.float32).contiguous()
        # the lm-head weight lives in the library's packed layout (w_lm stays row-major):
        # bf16 operands, or block-FP8 codes and scales for the W8A8 head
        w_lm = w_lm.contiguous()
        fp8 = lm_dtype == RIL_LM_W8A8_FP8
        nbytes = (ril_lm_head_fp8_packed_bytes if fp8 else ril_lm_head_packed_bytes)(vocab, d_head)
        self.w_lm_packed = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        self.pack_lm_head = ril_pack_lm_head_fp8 if fp8 else ril_pack_lm_head
        self.pack_lm_head(w_lm, self.w_lm_packed)
        if proj_dtype == RIL_PROJ_W8A8_FP8:
            # each projection weight in its block-FP8 form (codes, then block exponents)
            def q8(w):
                if w is None:
                    return None
                w = w.contiguous()
                out = torch.empty(ril_proj_fp8_bytes(*w.shape), dtype=torch.uint8, device=self.device)
                ril_quantize_weight_fp8(w, out)
                return out
            w_qkv, w_o, w_gate_up, w_down = q8(w_qkv), q8(w_o), q8(w_gate_up), q8(w_down)
        self._keep = [embed, w_qkv, w_o, norm_attn, norm_final, w_gate_up, w_down, norm_mlp, ssm_A, ssm_D]
        p = lambda t: None if t is None else t.data_ptr()  # noqa: E731
        self.desc = ril_model_desc(attn_kind, input_mode, d_model, n_q_heads, n_kv_heads, head_dim, rope_dim,
                                   index_heads, index_dim, topk, d_head, vocab, PAGE, split_tokens, max_rows,
                                   max_tokens, max_ctx, softmax_scale, rms_eps, p(embed), p(w_qkv), p(w_o),
                                   p(norm_attn), p(norm_final), p(self.w_lm_packed), kv_dtype, k_scale_exp,
                                   v_scale_exp, d_ff, p(w_gate_up), p(w_down), p(norm_mlp), lm_dtype,
                                   proj_dtype, 128 if self.ssd else 0, 128 if self.ssd else 0, p(ssm_A),
                                   p(ssm_D))
        self.model = ril_model_create(self.desc)
        self.H, self.Hkv, self.D = n_q_heads, n_kv_heads, head_dim
        self.max_ctx = max_ctx
        self.ws = torch.empty(ril_workspace_bytes(self.model), dtype=torch.uint8, device=self.device)
        self.page_bytes = ril_kv_page_bytes(self.model)
        self.pool = torch.empty(pool_pages * self.page_bytes, dtype=torch.uint8, device=self.device)
        self.kv = ril_kv_alloc(self.model, self.pool, shuffle_seed)
        self.pages: Dict[object, List[int]] = {}
        self._ids: Dict[object, torch.Tensor] = {}  # page lists as int32 tensors, per sequence

    def lm_head(self, z, targets) -> torch.Tensor:
        """The head alone: logprobs (fp32 [rows]) of targets for normalised bf16 rows z."""
        out = torch.empty(z.shape[0], dtype=torch.float32, device=self.device)
        ril_lm_head_logprobs(self.model, z, _i32(targets, self.device), out, self.ws)
        return out

    def set_policy(self, policy: int, attn_split_tokens: int = 0) -> None:
        """Switch the comparator policy (benchmarking only) and grow the workspace if
        the policy needs more."""
        ril_set_policy(self.model, policy, attn_split_tokens)
        need = ril_workspace_bytes(self.model)
        if need > self.ws.numel():
            self.ws = torch.empty(need, dtype=torch.uint8, device=self.device)

    def close(self):
        if getattr(self, "kv", None):
            ril_kv_free(self.kv)
            self.kv = None
        if getattr(self, "model", None):
            ril_model_destroy(self.model)
            self.model = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- pages ---------------------------------------------------------------
    def ensure(self, seq, n_tokens: int) -> None:
        have = self.pages.setdefault(seq, [])
        need = (1 if self.ssd else math.ceil(n_tokens / PAGE)) - len(have)
        if need > 0:
            have.extend(ril_kv_assign(self.kv, need))

    def release(self, seq) -> None:
        ids = self.pages.pop(seq, [])
        self._ids.pop(seq, None)
        if ids:
            ril_kv_release(self.kv, ids)

    def _page_ids(self, seq) -> torch.Tensor:
        lst = self.pages[seq]
        t = self._ids.get(seq)
        if t is None or t.numel() != len(lst):
            t = torch.tensor(lst, dtype=torch.int32)
            self._ids[seq] = t
        return t

    def page_table(self, seqs: Sequence, ctx_bound: int) -> torch.Tensor:
        stride = 1 if self.ssd else max(1, math.ceil(ctx_bound / PAGE))
        t = torch.full((len(seqs), stride), -1, dtype=torch.int32)
        for i, s in enumerate(seqs):
            ids = self._page_ids(s)
            n = min(stride, ids.numel())
            t[i, :n] = ids[:n]
        return t.to(self.device)

    # -- calls -----------------------------------------------------------------
    def _packed(self, seqs, starts, lens):
        cu = [0]
        for n in lens:
            cu.append(cu[-1] + int(n))
        bound = max(int(s) + int(n) for s, n in zip(starts, lens))
        for s, st, n in zip(seqs, starts, lens):
            self.ensure(s, int(st) + int(n))
        return cu, bound

    def write_kv(self, seqs, starts, ks, vs, k_index=None) -> None:
        """The shared write path alone: k/v [n_i, ...] (and indexer keys) of sequence i at
        positions starts[i].."""
        lens = [k.shape[0] for k in ks]
        cu, bound = self._packed(seqs, starts, lens)
        k, v, ki = _cat(ks), _cat(vs), _cat(k_index)
        cu_t, st_t = _i32(cu, self.device), _i32(list(starts), self.device)
        pt = self.page_table(seqs, bound)
        b = make_prefill_batch(cu_tokens=cu_t, start_pos=st_t, page_table=pt, max_ctx_bound=bound,
                               k=k, v=v, k_index=ki, total_tokens=cu[-1])
        ril_kv_write(self.model, self.kv, b)
        self._last = (k, v, ki, cu_t, st_t, pt)

    def prefill(self, seqs, starts, *, targets, qs=None, ks=None, vs=None, tokens=None, q_index=None,
                k_index=None, selected_out=None, ctx_bound: Optional[int] = None, dts=None) -> torch.Tensor:
        """Packed prefill of sequences seqs[i] at positions starts[i].. ; returns fp32 [total]."""
        src = tokens if tokens is not None else qs
        lens = [t.shape[0] for t in src]
        cu, bound = self._packed(seqs, starts, lens)
        bound = ctx_bound or bound
        q, k, v, tok, qi, ki, dt = (_cat(qs), _cat(ks), _cat(vs), _cat(tokens), _cat(q_index), _cat(k_index),
                                    _cat(dts))
        tgt = torch.cat(list(targets)).to(torch.int32).contiguous()
        cu_t, st_t = _i32(cu, self.device), _i32(list(starts), self.device)
        pt = self.page_table(seqs, bound)
        out = torch.empty(cu[-1], dtype=torch.float32, device=self.device)
        b = make_prefill_batch(cu_tokens=cu_t, start_pos=st_t, page_table=pt, max_ctx_bound=bound,
                               target_ids=tgt, token_ids=tok, q=q, k=k, v=v, q_index=qi, k_index=ki,
                               selected_out=selected_out, total_tokens=cu[-1], dt=dt)
        ril_prefill_logprobs(self.model, self.kv, b, out, self.ws)
        self._last = (q, k, v, tok, qi, ki, tgt, cu_t, st_t, pt, dt)
        return out

    def _decode_batch(self, seqs, ctx, targets, q, k, v, tokens, q_index, k_index, selected_out, ctx_bound,
                      dt=None):
        ctx = [int(c) for c in ctx]
        for s, c in zip(seqs, ctx):
            self.ensure(s, c)
        bound = ctx_bound or max(ctx)
        keep = {"ctx": _i32(ctx, self.device), "pt": self.page_table(seqs, bound),
                "tgt": targets.to(torch.int32).contiguous(), "tok": _c(tokens), "q": _c(q), "k": _c(k),
                "v": _c(v), "qi": _c(q_index), "ki": _c(k_index), "dt": _c(dt)}
        b = make_decode_batch(ctx_len=keep["ctx"], page_table=keep["pt"], max_ctx_bound=bound,
                              target_ids=keep["tgt"], token_ids=keep["tok"], q=keep["q"], k=keep["k"],
                              v=keep["v"], q_index=keep["qi"], k_index=keep["ki"], selected_out=selected_out,
                              dt=keep["dt"])
        return b, keep

    def decode(self, seqs, ctx, *, targets, q=None, k=None, v=None, tokens=None, q_index=None, k_index=None,
               selected_out=None, ctx_bound: Optional[int] = None, dt=None) -> torch.Tensor:
        """One decode step: row i of sequence seqs[i] at context ctx[i]; returns fp32 [rows]."""
        b, keep = self._decode_batch(seqs, ctx, targets, q, k, v, tokens, q_index, k_index, selected_out,
                                     ctx_bound, dt)
        out = torch.empty(len(seqs), dtype=torch.float32, device=self.device)
        ril_decode_step_logprobs(self.model, self.kv, b, out, self.ws)
        self._last = keep
        return out

    def prepare_decode(self, seqs, ctx, *, targets, q=None, k=None, v=None, tokens=None, q_index=None,
                       k_index=None, ctx_bound: Optional[int] = None, dt=None):
        """Build a decode batch once; returns (launch, out) where launch() enqueues the step
        on the current stream with no host-side tensor work (for timed loops)."""
        b, keep = self._decode_batch(seqs, ctx, targets, q, k, v, tokens, q_index, k_index, None, ctx_bound, dt)
        out = torch.empty(len(seqs), dtype=torch.float32, device=self.device)
        stream = torch.cuda.current_stream(self.device).cuda_stream

        def launch():
            ril_decode_step_logprobs(self.model, self.kv, b, out, self.ws, stream)

        launch.keep = keep  # the descriptor's tensors live as long as the launcher
        return launch, out

    def decode_graph(self, seqs, ctx_bound: int, *, ctx, targets, q=None, k=None, v=None, tokens=None,
                     q_index=None, k_index=None) -> "DecodeGraph":
        """Capture a decode step of rows seqs into a HIP graph over fixed buffers (pages are
        assigned up to ctx_bound now); replay it with DecodeGraph.run."""
        return DecodeGraph(self, seqs, ctx_bound, ctx=ctx, targets=targets, q=q, k=k, v=v, tokens=tokens,
                           q_index=q_index, k_index=k_index)

    def attn_out(self, rows: int) -> torch.Tensor:
        """bf16 [rows, Hq, D] attention output of the last call (a workspace view)."""
        off = ril_ws_attn_offset(self.model)
        n = rows * self.H * self.D
        return self.ws[off: off + 2 * n].view(torch.bfloat16).view(rows, self.H, self.D)


class DecodeGraph:
    """One captured decode step (ril_decode_graph_create) and the fixed device buffers its
    replays read.  run() copies a step's inputs into those buffers on the current stream and
    replays the graph there: the same kernels, with the same arguments, as Session.decode."""

    def __init__(self, sess: Session, seqs, ctx_bound: int, *, ctx, targets, q, k, v, tokens, q_index, k_index):
        self.sess = sess
        b, keep = sess._decode_batch(seqs, ctx, targets, q, k, v, tokens, q_index, k_index, None, ctx_bound)
        # the batch's tensors are fresh copies, owned here: replays read them in place
        self.buf = {key: (t.clone() if t is not None else None) for key, t in keep.items()}
        self.batch = make_decode_batch(ctx_len=self.buf["ctx"], page_table=self.buf["pt"], max_ctx_bound=ctx_bound,
                                       target_ids=self.buf["tgt"], token_ids=self.buf["tok"], q=self.buf["q"],
                                       k=self.buf["k"], v=self.buf["v"], q_index=self.buf["qi"],
                                       k_index=self.buf["ki"], selected_out=None)
        self.out = torch.empty(len(seqs), dtype=torch.float32, device=sess.device)
        self.seqs = list(seqs)
        self.bound = int(ctx_bound)
        self.handle = ril_decode_graph_create(sess.model, sess.kv, self.batch, self.out, sess.ws)

    def run(self, ctx, *, targets, q=None, k=None, v=None, tokens=None, q_index=None, k_index=None) -> torch.Tensor:
        """Replay with new inputs; returns the (reused) fp32 [rows] output buffer."""
        ctx = [int(c) for c in ctx]
        if len(ctx) != len(self.seqs) or max(ctx) > self.bound or min(ctx) < 1:
            raise ValueError(f"graph captured for {len(self.seqs)} rows with contexts <= {self.bound}")
        for s_, c in zip(self.seqs, ctx):
            self.sess.ensure(s_, c)
        self.buf["pt"].copy_(self.sess.page_table(self.seqs, self.bound))  # same stride, pages as of now
        self.buf["ctx"].copy_(torch.tensor(ctx, dtype=torch.int32), non_blocking=False)
        self.buf["tgt"].copy_(targets.to(torch.int32))
        for key, t in (("tok", tokens), ("q", q), ("k", k), ("v", v), ("qi", q_index), ("ki", k_index)):
            if t is not None:
                self.buf[key].copy_(t)
        ril_graph_launch(self.handle, torch.cuda.current_stream(self.sess.device).cuda_stream)
        return self.out

    def replay(self) -> None:
        """Replay on the current stream with the buffers as they are (for timed loops)."""
        ril_graph_launch(self.handle, torch.cuda.current_stream(self.sess.device).cuda_stream)

    def close(self) -> None:
        if getattr(self, "handle", None):
            ril_graph_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
