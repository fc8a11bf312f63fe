"""Python binding of libril.so, the C ABI declared in include/ril.h.

Argument marshalling only: every step of the forward runs in the library's HIP
kernels.  The functions keep the C names (ril_model_create, ril_kv_alloc,
ril_prefill_logprobs, ril_decode_step_logprobs, ...) and take torch tensors where
the C side takes device pointers; torch supplies device memory and the stream.

Importing this package fails loudly if libril.so is missing or does not load:
there is no fallback of any kind.
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libril.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python invariant_rl_logprob_amd/build.py` "
        "(or __graft_entry__.build()); there is no fallback path")
_lib = ctypes.CDLL(LIB_PATH)

RIL_OK, RIL_EINVAL, RIL_ERANGE, RIL_ENOSPC, RIL_EUNSUPPORTED, RIL_EHIP = 0, -1, -2, -3, -4, -5
RIL_ATTN_GQA, RIL_ATTN_MLA, RIL_ATTN_MLA_SPARSE, RIL_ATTN_SSD = 0, 1, 2, 3
RIL_INPUT_TOKENS, RIL_INPUT_QKV = 0, 1
RIL_POLICY_INVARIANT, RIL_POLICY_SHAPE_DERIVED = 0, 1
RIL_KV_BF16, RIL_KV_FP8_E4M3 = 0, 1
RIL_LM_BF16, RIL_LM_W8A8_FP8 = 0, 1
RIL_PROJ_BF16, RIL_PROJ_W8A8_FP8 = 0, 1

_c_int, _c_float, _vp = ctypes.c_int32, ctypes.c_float, ctypes.c_void_p


class ril_model_desc(ctypes.Structure):
    _fields_ = [
        ("attn_kind", _c_int), ("input_mode", _c_int), ("d_model", _c_int),
        ("n_q_heads", _c_int), ("n_kv_heads", _c_int), ("head_dim", _c_int), ("rope_dim", _c_int),
        ("index_heads", _c_int), ("index_dim", _c_int), ("topk", _c_int),
        ("d_head", _c_int), ("vocab", _c_int), ("page_tokens", _c_int),
        ("split_tokens", _c_int), ("max_rows", _c_int), ("max_tokens", _c_int),
        ("max_ctx", _c_int), ("softmax_scale", _c_float), ("rms_eps", _c_float),
        ("embed", _vp), ("w_qkv", _vp), ("w_o", _vp), ("norm_attn", _vp),
        ("norm_final", _vp), ("w_lm", _vp),
        ("kv_dtype", _c_int), ("k_scale_exp", _c_int), ("v_scale_exp", _c_int),
        ("d_ff", _c_int), ("w_gate_up", _vp), ("w_down", _vp), ("norm_mlp", _vp),
        ("lm_dtype", _c_int),
        ("proj_dtype", _c_int),
        ("ssm_state", _c_int), ("ssm_chunk", _c_int), ("ssm_A", _vp), ("ssm_D", _vp),
    ]


class ril_prefill_batch(ctypes.Structure):
    _fields_ = [
        ("n_seqs", _c_int), ("total_tokens", _c_int), ("max_ctx_bound", _c_int),
        ("cu_tokens", _vp), ("start_pos", _vp), ("page_table", _vp), ("page_stride", _c_int),
        ("target_ids", _vp), ("token_ids", _vp), ("q", _vp), ("k", _vp), ("v", _vp),
        ("q_index", _vp), ("k_index", _vp), ("selected_out", _vp), ("dt", _vp),
    ]


class ril_decode_batch(ctypes.Structure):
    _fields_ = [
        ("n_rows", _c_int), ("max_ctx_bound", _c_int), ("ctx_len", _vp), ("page_table", _vp),
        ("page_stride", _c_int), ("target_ids", _vp), ("token_ids", _vp),
        ("q", _vp), ("k", _vp), ("v", _vp), ("q_index", _vp), ("k_index", _vp), ("selected_out", _vp),
        ("dt", _vp),
    ]


def _sig(name, res, args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = args
    return f


_model_create = _sig("ril_model_create", _c_int, [ctypes.POINTER(ril_model_desc), ctypes.POINTER(_vp)])
_model_destroy = _sig("ril_model_destroy", None, [_vp])
_workspace_bytes = _sig("ril_workspace_bytes", ctypes.c_size_t, [_vp])
_kv_page_bytes = _sig("ril_kv_page_bytes", ctypes.c_size_t, [_vp])
_lm_head_packed_bytes = _sig("ril_lm_head_packed_bytes", ctypes.c_size_t, [_c_int, _c_int])
_pack_lm_head = _sig("ril_pack_lm_head", _c_int, [_vp, _c_int, _c_int, _vp, ctypes.c_size_t, _vp])
_lm_head_fp8_packed_bytes = _sig("ril_lm_head_fp8_packed_bytes", ctypes.c_size_t, [_c_int, _c_int])
_pack_lm_head_fp8 = _sig("ril_pack_lm_head_fp8", _c_int, [_vp, _c_int, _c_int, _vp, ctypes.c_size_t, _vp])
_lm_head_logprobs = _sig("ril_lm_head_logprobs", _c_int,
                         [_vp, _c_int, _vp, _c_int, _vp, _vp, _vp, ctypes.c_size_t, _vp])
_hbm_read_probe_words = _sig("ril_hbm_read_probe_words", _c_int, [])
_hbm_read_probe = _sig("ril_hbm_read_probe", _c_int, [_vp, ctypes.c_size_t, _vp, _vp])
_quantize_rows_fp8 = _sig("ril_quantize_rows_fp8", _c_int, [_vp, _c_int, _c_int, _c_int, _vp, _vp, _vp])
_proj_fp8_bytes = _sig("ril_proj_fp8_bytes", ctypes.c_size_t, [_c_int, _c_int])
_quantize_weight_fp8 = _sig("ril_quantize_weight_fp8", _c_int, [_vp, _c_int, _c_int, _vp, ctypes.c_size_t, _vp])
_proj_w8a8 = _sig("ril_proj_w8a8", _c_int,
                  [_vp, _vp, _c_int, _c_int, _vp, ctypes.c_size_t, _c_int, _vp, _c_int, _vp])
_proj_bf16 = _sig("ril_proj_bf16", _c_int,
                  [_vp, _c_int, _c_int, _c_int, _vp, _c_int, _c_int, _vp, _c_int, _vp, _c_int, _vp])
_ws_attn_offset = _sig("ril_ws_attn_offset", ctypes.c_size_t, [_vp])
_kv_alloc = _sig("ril_kv_alloc", _c_int, [_vp, _vp, ctypes.c_size_t, ctypes.c_uint64, ctypes.POINTER(_vp)])
_kv_assign = _sig("ril_kv_assign", _c_int, [_vp, _c_int, ctypes.POINTER(_c_int)])
_kv_release = _sig("ril_kv_release", _c_int, [_vp, _c_int, ctypes.POINTER(_c_int)])
_kv_free_pages = _sig("ril_kv_free_pages", _c_int, [_vp])
_kv_total_pages = _sig("ril_kv_total_pages", _c_int, [_vp])
_kv_free = _sig("ril_kv_free", None, [_vp])
_prefill = _sig("ril_prefill_logprobs", _c_int,
                [_vp, _vp, ctypes.POINTER(ril_prefill_batch), _vp, _vp, ctypes.c_size_t, _vp])
_decode = _sig("ril_decode_step_logprobs", _c_int,
               [_vp, _vp, ctypes.POINTER(ril_decode_batch), _vp, _vp, ctypes.c_size_t, _vp])
_decode_noalloc = _sig("ril_decode_step_logprobs_noalloc", _c_int,
                       [_vp, _vp, ctypes.POINTER(ril_decode_batch), _vp, _vp])
_kv_write = _sig("ril_kv_write", _c_int, [_vp, _vp, ctypes.POINTER(ril_prefill_batch), _vp])
_graph_create = _sig("ril_decode_graph_create", _c_int,
                     [_vp, _vp, ctypes.POINTER(ril_decode_batch), _vp, _vp, ctypes.c_size_t, ctypes.POINTER(_vp)])
_graph_launch = _sig("ril_graph_launch", _c_int, [_vp, _vp])
_graph_destroy = _sig("ril_graph_destroy", None, [_vp])
_last_error = _sig("ril_last_error", ctypes.c_char_p, [])
_set_policy = _sig("ril_set_policy", _c_int, [_vp, _c_int, _c_int])
_trace_enable = _sig("ril_trace_enable", _c_int, [_c_int])
_trace_read = _sig("ril_trace_read", _c_int, [_c_int, ctypes.POINTER(ctypes.c_double),
                                              ctypes.POINTER(ctypes.c_int64)])

EXPORTED = ("ril_model_create", "ril_model_destroy", "ril_workspace_bytes", "ril_kv_page_bytes",
            "ril_lm_head_packed_bytes", "ril_pack_lm_head", "ril_lm_head_fp8_packed_bytes", "ril_pack_lm_head_fp8",
            "ril_quantize_rows_fp8", "ril_proj_fp8_bytes", "ril_quantize_weight_fp8", "ril_proj_w8a8", "ril_proj_bf16",
            "ril_lm_head_logprobs", "ril_hbm_read_probe_words", "ril_hbm_read_probe",
            "ril_ws_attn_offset", "ril_kv_alloc", "ril_kv_assign", "ril_kv_release",
            "ril_kv_free_pages", "ril_kv_total_pages", "ril_kv_free", "ril_prefill_logprobs",
            "ril_decode_step_logprobs", "ril_decode_step_logprobs_noalloc", "ril_kv_write", "ril_last_error", "ril_set_policy", "ril_trace_enable",
            "ril_trace_read", "ril_decode_graph_create", "ril_graph_launch", "ril_graph_destroy")

# kernel ids of the trace hook
RIL_K_KV_WRITE, RIL_K_ATTN_SPLIT, RIL_K_ATTN_MERGE, RIL_K_ATTN_PREFILL = 0, 1, 2, 3
RIL_K_RMSNORM, RIL_K_GEMM, RIL_K_LM_HEAD, RIL_K_VOCAB_MERGE = 4, 5, 6, 7
RIL_K_INDEXER, RIL_K_TOPK, RIL_K_SILU_MUL = 8, 9, 10
RIL_K_QUANT_ROWS, RIL_K_LM_HEAD_FP8, RIL_K_GEMM_FP8 = 11, 12, 13
RIL_K_SSD_CHUNK, RIL_K_SSD_OUT, RIL_K_COUNT = 14, 15, 16
KERNEL_NAMES = ("kv_write", "attn_split", "attn_merge", "attn_prefill", "rmsnorm", "gemm", "lm_head",
                "vocab_merge", "indexer", "topk", "silu_mul", "quant_rows", "lm_head_fp8", "gemm_fp8",
                "ssd_chunk", "ssd_out")


class RilError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what} failed with status {status}: {ril_last_error()}")


def _check(status, what):
    if status != RIL_OK:
        raise RilError(status, what)


def _ptr(t):
    """Device (or host) address of a tensor, or None."""
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream


def ril_last_error() -> str:
    s = _last_error()
    return s.decode() if s else ""


def ril_model_create(desc: ril_model_desc) -> int:
    h = _vp()
    _check(_model_create(ctypes.byref(desc), ctypes.byref(h)), "ril_model_create")
    return h.value


def ril_model_destroy(model: int) -> None:
    _model_destroy(model)


def ril_workspace_bytes(model: int) -> int:
    return int(_workspace_bytes(model))


def ril_kv_page_bytes(model: int) -> int:
    return int(_kv_page_bytes(model))


def ril_lm_head_packed_bytes(vocab: int, d_head: int) -> int:
    return int(_lm_head_packed_bytes(vocab, d_head))


def ril_pack_lm_head(w, packed, stream=None) -> None:
    """Pack the row-major bf16 device matrix w [V, K] into `packed` (a device byte
    tensor of at least ril_lm_head_packed_bytes(V, K) bytes), on the stream."""
    V, K = w.shape
    _check(_pack_lm_head(_ptr(w), V, K, _ptr(packed), packed.numel() * packed.element_size(), _stream(stream)),
           "ril_pack_lm_head")


def ril_lm_head_fp8_packed_bytes(vocab: int, d_head: int) -> int:
    return int(_lm_head_fp8_packed_bytes(vocab, d_head))


def ril_pack_lm_head_fp8(w, packed, stream=None) -> None:
    """Quantize the row-major bf16 device matrix w [V, K] to block FP8 and pack it into
    `packed` (a device byte tensor of at least ril_lm_head_fp8_packed_bytes(V, K) bytes),
    on the stream."""
    V, K = w.shape
    _check(_pack_lm_head_fp8(_ptr(w), V, K, _ptr(packed), packed.numel() * packed.element_size(),
                             _stream(stream)), "ril_pack_lm_head_fp8")


def ril_quantize_rows_fp8(x, codes, exps, stream=None) -> None:
    """Block-FP8 quantization of the bf16 device rows x [rows, K] (row stride x.stride(0))
    into codes (uint8 [rows, K]) and exps (int32 [rows, K/128], biased E8M0), on the
    stream."""
    rows, K = x.shape
    if codes.numel() < rows * K or exps.numel() < rows * (K // 128):
        raise ValueError("ril_quantize_rows_fp8: output tensors too small")
    _check(_quantize_rows_fp8(_ptr(x), rows, K, x.stride(0), _ptr(codes), _ptr(exps), _stream(stream)),
           "ril_quantize_rows_fp8")


def ril_proj_fp8_bytes(N: int, K: int) -> int:
    return int(_proj_fp8_bytes(N, K))


def ril_quantize_weight_fp8(w, dst, stream=None) -> None:
    """Block-FP8 quantization of the row-major bf16 device matrix w [N, K] into dst (a
    device byte tensor of at least ril_proj_fp8_bytes(N, K) bytes: codes, then the block
    exponents), on the stream."""
    N, K = w.shape
    _check(_quantize_weight_fp8(_ptr(w), N, K, _ptr(dst), dst.numel() * dst.element_size(), _stream(stream)),
           "ril_quantize_weight_fp8")


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def ril_proj_w8a8(codes, exps, w8, N: int, out, stream=None) -> None:
    """out[rows, N] = bf16(A W^T) for rows given as block-FP8 codes (uint8 [rows, K],
    contiguous) and exps (int32 [rows, K/128], contiguous) and W as written by
    ril_quantize_weight_fp8 (N rows, a uint8 device tensor); out is a bf16 device tensor
    [rows, >= N] with unit column stride (row stride out.stride(0))."""
    import torch
    rows, K = codes.shape
    _need(codes.dtype == torch.uint8 and codes.is_contiguous(), "ril_proj_w8a8: codes must be contiguous uint8")
    _need(exps.dtype == torch.int32 and exps.is_contiguous() and exps.numel() >= rows * (K // 128),
          "ril_proj_w8a8: exps must be contiguous int32 [rows, K/128]")
    _need(w8.dtype == torch.uint8 and w8.is_contiguous(), "ril_proj_w8a8: w8 must be a contiguous uint8 buffer")
    _need(out.dtype == torch.bfloat16 and out.dim() == 2 and out.stride(1) == 1 and out.shape[0] >= rows
          and out.shape[1] >= N, "ril_proj_w8a8: out must be bf16 [rows, >= N] with unit column stride")
    _check(_proj_w8a8(_ptr(codes), _ptr(exps), rows, K, _ptr(w8), w8.numel(), N, _ptr(out), out.stride(0),
                      _stream(stream)), "ril_proj_w8a8")


def ril_proj_bf16(a, w, out, residual=None, stream=None) -> None:
    """out[rows, N] = bf16(a w^T), or bf16(residual + bf16(a w^T)): the model's bf16
    projection GEMM alone.  a is bf16 [rows, K] and w bf16 [N, K] (unit column stride, row
    strides a.stride(0), w.stride(0)); out and residual bf16 [rows, >= N] with unit column
    stride; all device tensors."""
    import torch
    rows, K = a.shape
    N = w.shape[0]
    for t, nm in ((a, "a"), (w, "w"), (out, "out")) + (((residual, "residual"),) if residual is not None else ()):
        _need(t.dtype == torch.bfloat16 and t.dim() == 2 and t.stride(1) == 1,
              f"ril_proj_bf16: {nm} must be a 2-d bf16 tensor with unit column stride")
    _need(w.shape[1] == K, "ril_proj_bf16: w must be [N, K]")
    _need(out.shape[0] >= rows and out.shape[1] >= N, "ril_proj_bf16: out must be [rows, >= N]")
    _need(residual is None or (residual.shape[0] >= rows and residual.shape[1] >= N),
          "ril_proj_bf16: residual must be [rows, >= N]")
    _check(_proj_bf16(_ptr(a), rows, K, a.stride(0), _ptr(w), N, w.stride(0), _ptr(residual),
                      0 if residual is None else residual.stride(0), _ptr(out), out.stride(0), _stream(stream)),
           "ril_proj_bf16")


def ril_lm_head_logprobs(model: int, z, targets, logprob_out, ws, stream=None) -> None:
    """The head alone: logprobs of targets (int32 device [rows]) for the normalised bf16
    device rows z [rows, d_head] (row stride z.stride(0)) into logprob_out (fp32 [rows])."""
    rows = z.shape[0]
    if targets.numel() < rows or logprob_out.numel() < rows:
        raise ValueError("ril_lm_head_logprobs: targets / logprob_out shorter than z")
    _check(_lm_head_logprobs(model, rows, _ptr(z), z.stride(0), _ptr(targets), _ptr(logprob_out), _ptr(ws),
                             ws.numel() * ws.element_size(), _stream(stream)), "ril_lm_head_logprobs")


def ril_hbm_read_probe_words() -> int:
    return int(_hbm_read_probe_words())


def ril_hbm_read_probe(src, out, stream=None) -> None:
    """Benchmarking only: one nontemporal grid-stride read of the device tensor src, folded
    into out (device uint32/int32 of at least ril_hbm_read_probe_words() entries)."""
    if out.numel() < ril_hbm_read_probe_words():
        raise ValueError("ril_hbm_read_probe: out too small")
    _check(_hbm_read_probe(_ptr(src), src.numel() * src.element_size(), _ptr(out), _stream(stream)),
           "ril_hbm_read_probe")


def ril_ws_attn_offset(model: int) -> int:
    return int(_ws_attn_offset(model))


def ril_kv_alloc(model: int, pool, shuffle_seed: int = 0) -> int:
    """Wrap a device byte tensor as the KV pool; returns the kv handle."""
    h = _vp()
    nbytes = pool.numel() * pool.element_size()
    _check(_kv_alloc(model, _ptr(pool), nbytes, shuffle_seed, ctypes.byref(h)), "ril_kv_alloc")
    return h.value


def ril_kv_assign(kv: int, n_pages: int):
    arr = (_c_int * max(1, n_pages))()
    _check(_kv_assign(kv, n_pages, arr), "ril_kv_assign")
    return [arr[i] for i in range(n_pages)]


def ril_kv_release(kv: int, page_ids) -> None:
    arr = (_c_int * max(1, len(page_ids)))(*page_ids)
    _check(_kv_release(kv, len(page_ids), arr), "ril_kv_release")


def ril_kv_free_pages(kv: int) -> int:
    return int(_kv_free_pages(kv))


def ril_kv_total_pages(kv: int) -> int:
    return int(_kv_total_pages(kv))


def ril_kv_free(kv: int) -> None:
    _kv_free(kv)


def make_prefill_batch(*, cu_tokens, start_pos, page_table, max_ctx_bound, target_ids=None,
                       token_ids=None, q=None, k=None, v=None, q_index=None, k_index=None,
                       selected_out=None, total_tokens=None, dt=None) -> ril_prefill_batch:
    """Build the C descriptor from device tensors (the tensors must outlive the call)."""
    n = cu_tokens.numel() - 1
    if total_tokens is None:
        raise ValueError("total_tokens (a host integer) is required")
    return ril_prefill_batch(n, int(total_tokens), int(max_ctx_bound), _ptr(cu_tokens), _ptr(start_pos),
                             _ptr(page_table), page_table.shape[1], _ptr(target_ids), _ptr(token_ids),
                             _ptr(q), _ptr(k), _ptr(v), _ptr(q_index), _ptr(k_index), _ptr(selected_out),
                             _ptr(dt))


def make_decode_batch(*, ctx_len, page_table, max_ctx_bound, target_ids, token_ids=None, q=None,
                      k=None, v=None, q_index=None, k_index=None, selected_out=None, dt=None) -> ril_decode_batch:
    return ril_decode_batch(ctx_len.numel(), int(max_ctx_bound), _ptr(ctx_len), _ptr(page_table),
                            page_table.shape[1], _ptr(target_ids), _ptr(token_ids), _ptr(q), _ptr(k), _ptr(v),
                            _ptr(q_index), _ptr(k_index), _ptr(selected_out), _ptr(dt))


def ril_prefill_logprobs(model: int, kv: int, batch: ril_prefill_batch, logprob_out, ws,
                         stream=None) -> None:
    _check(_prefill(model, kv, ctypes.byref(batch), _ptr(logprob_out), _ptr(ws),
                    ws.numel() * ws.element_size(), _stream(stream)), "ril_prefill_logprobs")


def ril_decode_step_logprobs(model: int, kv: int, batch: ril_decode_batch, logprob_out, ws,
                             stream=None) -> None:
    _check(_decode(model, kv, ctypes.byref(batch), _ptr(logprob_out), _ptr(ws),
                   ws.numel() * ws.element_size(), _stream(stream)), "ril_decode_step_logprobs")


RIL_NOALLOC_SCRATCH_BYTES = 64 << 20  # include/ril.h


def ril_decode_step_logprobs_noalloc(model: int, kv: int, batch: ril_decode_batch, logprob_out,
                                     stream=None) -> None:
    """ril_decode_step_logprobs on the library's static device scratch (no workspace)."""
    _check(_decode_noalloc(model, kv, ctypes.byref(batch), _ptr(logprob_out), _stream(stream)),
           "ril_decode_step_logprobs_noalloc")


def ril_decode_graph_create(model: int, kv: int, batch: ril_decode_batch, logprob_out, ws) -> int:
    """Capture one decode step into a HIP graph (nothing runs); returns the graph handle."""
    g = _vp()
    _check(_graph_create(model, kv, ctypes.byref(batch), _ptr(logprob_out), _ptr(ws),
                         ws.numel() * ws.element_size(), ctypes.byref(g)), "ril_decode_graph_create")
    return g.value


def ril_graph_launch(graph: int, stream=None) -> None:
    _check(_graph_launch(graph, _stream(stream)), "ril_graph_launch")


def ril_graph_destroy(graph: int) -> None:
    _graph_destroy(graph)


def ril_kv_write(model: int, kv: int, batch: ril_prefill_batch, stream=None) -> None:
    _check(_kv_write(model, kv, ctypes.byref(batch), _stream(stream)), "ril_kv_write")


def ril_set_policy(model: int, policy: int, attn_split_tokens: int = 0) -> None:
    """Comparator switch (benchmarking only): RIL_POLICY_SHAPE_DERIVED lets the kernels
    choose their splits from the call's shape; RIL_POLICY_INVARIANT restores the method."""
    _check(_set_policy(model, policy, attn_split_tokens), "ril_set_policy")


def ril_trace_enable(on: bool) -> None:
    _check(_trace_enable(1 if on else 0), "ril_trace_enable")


def ril_trace_read(kernel: int):
    """(total milliseconds, launches) of one kernel since the last ril_trace_enable."""
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    _check(_trace_read(kernel, ctypes.byref(ms), ctypes.byref(n)), "ril_trace_read")
    return ms.value, n.value
