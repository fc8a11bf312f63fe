"""CPU tests of the C ABI: the library loads, exports every symbol include/*.h declares,
validates descriptions and batches on the host, and its page allocator behaves.
No kernel is launched: every call here either fails validation (nothing enqueued)
or is host-only."""

import ctypes
import os
import re

import pytest
import torch

import invariant_rl_logprob_amd as ril

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    inc = os.path.join(ROOT, "include")
    src = "".join(open(os.path.join(inc, f)).read() for f in sorted(os.listdir(inc)) if f.endswith(".h"))
    return sorted(set(re.findall(r"\b(ril_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(ril.LIB_PATH)
    names = _declared()
    assert "ril_prefill_logprobs" in names and "ril_decode_step_logprobs" in names and "ril_kv_alloc" in names
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(ril.EXPORTED)


def _desc(**kw):
    # fake device addresses: model_create only validates them (16-byte aligned, non-null)
    base = dict(attn_kind=0, input_mode=ril.RIL_INPUT_QKV, d_model=0, n_q_heads=32, n_kv_heads=8,
                head_dim=128, rope_dim=0, index_heads=0, index_dim=0, topk=0, d_head=4096, vocab=129280, page_tokens=16, split_tokens=512,
                max_rows=64, max_tokens=1024, max_ctx=8192, softmax_scale=0.088388, rms_eps=1e-6,
                embed=None, w_qkv=None, w_o=None, norm_attn=None, norm_final=None, w_lm=0x10000)
    base.update(kw)
    d = ril.ril_model_desc()
    for k, v in base.items():
        setattr(d, k, v)
    return d


def test_model_create_validates():
    m = ril.ril_model_create(_desc())
    assert ril.ril_workspace_bytes(m) > 0
    assert ril.ril_kv_page_bytes(m) == 8 * 2 * 16 * 128 * 2
    ril.ril_model_destroy(m)
    bad = [dict(head_dim=96), dict(n_kv_heads=5), dict(n_q_heads=48, n_kv_heads=2), dict(page_tokens=32),
           dict(split_tokens=100), dict(vocab=0), dict(w_lm=None), dict(w_lm=0x10008), dict(d_head=4000),
           dict(max_ctx=0), dict(softmax_scale=0.0), dict(input_mode=7),
           dict(input_mode=ril.RIL_INPUT_TOKENS, d_model=256, d_head=256)]
    for b in bad:
        with pytest.raises(ril.RilError):
            ril.ril_model_create(_desc(**b))
        assert ril.ril_last_error()


def test_fp8_kv_cache_descriptor():
    m = ril.ril_model_create(_desc(kv_dtype=ril.RIL_KV_FP8_E4M3, k_scale_exp=-2, v_scale_exp=3))
    assert ril.ril_kv_page_bytes(m) == 8 * 2 * 16 * 128  # one byte per value: half of bf16
    ril.ril_model_destroy(m)
    mla = dict(attn_kind=ril.RIL_ATTN_MLA, n_q_heads=128, n_kv_heads=1, head_dim=512, rope_dim=64,
               d_head=65536, split_tokens=2048)
    # the MLA latent in FP8: 16 x 576 codes per page (the sparse kind adds its fp32 keys)
    m = ril.ril_model_create(_desc(kv_dtype=ril.RIL_KV_FP8_E4M3, k_scale_exp=2, v_scale_exp=2, **mla))
    assert ril.ril_kv_page_bytes(m) == 16 * 576
    ril.ril_model_destroy(m)
    sp = dict(mla, attn_kind=ril.RIL_ATTN_MLA_SPARSE, index_heads=64, index_dim=128, topk=2048, split_tokens=256)
    m = ril.ril_model_create(_desc(kv_dtype=ril.RIL_KV_FP8_E4M3, **sp))
    assert ril.ril_kv_page_bytes(m) == 16 * 576 + 16 * 128 * 4
    ril.ril_model_destroy(m)
    for b in (dict(kv_dtype=2), dict(kv_dtype=-1), dict(kv_dtype=ril.RIL_KV_FP8_E4M3, k_scale_exp=33),
              dict(kv_dtype=ril.RIL_KV_FP8_E4M3, v_scale_exp=-40), dict(k_scale_exp=1),
              dict(kv_dtype=ril.RIL_KV_FP8_E4M3, k_scale_exp=1, v_scale_exp=2, **mla)):  # one latent scale
        with pytest.raises(ril.RilError):
            ril.ril_model_create(_desc(**b))
        assert ril.ril_last_error()


def test_mlp_block_descriptor():
    tok = dict(input_mode=ril.RIL_INPUT_TOKENS, d_model=256, d_head=256, n_q_heads=4, n_kv_heads=4,
               head_dim=64, vocab=2048, embed=0x20000, w_qkv=0x30000, w_o=0x40000)
    m = ril.ril_model_create(_desc(**tok, d_ff=512, w_gate_up=0x50000, w_down=0x60000))
    plain = ril.ril_model_create(_desc(**tok))
    assert ril.ril_workspace_bytes(m) > ril.ril_workspace_bytes(plain)
    ril.ril_model_destroy(m)
    ril.ril_model_destroy(plain)
    for b in (dict(tok, d_ff=500, w_gate_up=0x50000, w_down=0x60000),      # not a multiple of 32
              dict(tok, d_ff=512, w_gate_up=0x50000),                        # no w_down
              dict(tok, d_ff=512, w_gate_up=0x50008, w_down=0x60000),        # misaligned
              dict(tok, w_gate_up=0x50000, w_down=0x60000),                  # weights without d_ff
              dict(d_ff=512, w_gate_up=0x50000, w_down=0x60000)):            # QKV input
        with pytest.raises(ril.RilError):
            ril.ril_model_create(_desc(**b))
        assert ril.ril_last_error()


def test_w8a8_lm_head_descriptor_and_sizes():
    m = ril.ril_model_create(_desc(lm_dtype=ril.RIL_LM_W8A8_FP8))
    plain = ril.ril_model_create(_desc())
    # activation codes (1 byte / value) and exponents (4 bytes / 128 values) per row
    R = 1024
    assert ril.ril_workspace_bytes(m) - ril.ril_workspace_bytes(plain) >= R * 4096 + R * 32 * 4
    ril.ril_model_destroy(m)
    ril.ril_model_destroy(plain)
    for b in (dict(lm_dtype=2), dict(lm_dtype=-1), dict(lm_dtype=ril.RIL_LM_W8A8_FP8, d_head=4064)):
        with pytest.raises(ril.RilError):
            ril.ril_model_create(_desc(**b))
        assert ril.ril_last_error()
    n_vt = (129280 + 255) // 256
    assert ril.ril_lm_head_fp8_packed_bytes(129280, 4096) == n_vt * 256 * 4096 + 2 * n_vt * 32 * 4
    assert ril.ril_lm_head_fp8_packed_bytes(300, 128) == 512 * 128 + 4 * 1 * 4
    for v, k in ((0, 128), (10, 96), (10, 0), (10, 4000)):
        assert ril.ril_lm_head_fp8_packed_bytes(v, k) == 0


def test_w8a8_projection_descriptor_sizes_and_bad_arguments():
    # QKV input with an o-projection (K = Hq*D = 4096): W8A8 projections accepted, and the
    # workspace grows by the rows' codes and exponents
    m = ril.ril_model_create(_desc(w_o=0x20000, proj_dtype=ril.RIL_PROJ_W8A8_FP8))
    plain = ril.ril_model_create(_desc(w_o=0x20000))
    assert ril.ril_workspace_bytes(m) - ril.ril_workspace_bytes(plain) >= 1024 * 4096 + 1024 * 32 * 4
    ril.ril_model_destroy(m)
    ril.ril_model_destroy(plain)
    for b in (dict(proj_dtype=2), dict(proj_dtype=-1),
              dict(w_o=0x20000, proj_dtype=ril.RIL_PROJ_W8A8_FP8, n_q_heads=8, n_kv_heads=8, head_dim=64),  # K 512: ok
              dict(input_mode=ril.RIL_INPUT_TOKENS, d_model=160, d_head=160, embed=0x30000, w_qkv=0x40000,
                   w_o=0x20000, proj_dtype=ril.RIL_PROJ_W8A8_FP8)):  # d_model 160: not a multiple of 128
        if b.get("n_q_heads") == 8:
            ril.ril_model_destroy(ril.ril_model_create(_desc(**b)))
            continue
        with pytest.raises(ril.RilError):
            ril.ril_model_create(_desc(**b))
        assert ril.ril_last_error()
    assert ril.ril_proj_fp8_bytes(300, 256) == 300 * 256 + 3 * 2 * 4
    assert ril.ril_proj_fp8_bytes(128, 128) == 128 * 128 + 4
    for n, k in ((0, 128), (10, 96), (10, 0), (10, 4000)):
        assert ril.ril_proj_fp8_bytes(n, k) == 0
    lib = ctypes.CDLL(ril.LIB_PATH)
    lib.ril_quantize_weight_fp8.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                            ctypes.c_size_t, ctypes.c_void_p]
    lib.ril_proj_w8a8.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                  ctypes.c_size_t, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]
    need = ril.ril_proj_fp8_bytes(300, 256)
    # every case fails validation before anything is enqueued
    assert lib.ril_quantize_weight_fp8(0x10000, 300, 200, 0x900000, need, None) == ril.RIL_EINVAL     # K % 128
    assert lib.ril_quantize_weight_fp8(0x10000, 300, 256, 0x900000, need - 1, None) == ril.RIL_EINVAL  # short
    assert lib.ril_quantize_weight_fp8(0x10008, 300, 256, 0x900000, need, None) == ril.RIL_EINVAL     # misaligned
    assert lib.ril_quantize_weight_fp8(0x10000, 300, 256, 0x10000, need, None) == ril.RIL_EINVAL      # overlap
    assert lib.ril_quantize_weight_fp8(None, 300, 256, 0x900000, need, None) == ril.RIL_EINVAL
    wn = ril.ril_proj_fp8_bytes(64, 256)
    assert lib.ril_proj_w8a8(0x10000, 0x20000, 4, 200, 0x30000, wn, 64, 0x40000, 64, None) == ril.RIL_EINVAL  # K % 128
    assert lib.ril_proj_w8a8(0x10000, 0x20000, 4, 256, 0x30000, wn, 64, 0x40000, 32, None) == ril.RIL_EINVAL  # ldo < N
    assert lib.ril_proj_w8a8(0x10008, 0x20000, 4, 256, 0x30000, wn, 64, 0x40000, 64, None) == ril.RIL_EINVAL  # align
    assert lib.ril_proj_w8a8(0x10000, 0x20002, 4, 256, 0x30000, wn, 64, 0x40000, 64, None) == ril.RIL_EINVAL  # exps
    assert lib.ril_proj_w8a8(0x10000, 0x20000, 4, 256, None, wn, 64, 0x40000, 64, None) == ril.RIL_EINVAL
    # a weight buffer too short for N x K (a wrong N or K would read past it)
    assert lib.ril_proj_w8a8(0x10000, 0x20000, 4, 256, 0x30000, wn - 1, 64, 0x40000, 64, None) == ril.RIL_EINVAL
    assert lib.ril_proj_w8a8(0x10000, 0x20000, 4, 256, 0x30000, wn, 65, 0x40000, 65, None) == ril.RIL_EINVAL
    assert lib.ril_proj_w8a8(0x10000, 0x20000, 0, 256, 0x30000, wn, 64, 0x40000, 64, None) == ril.RIL_OK  # nothing


def test_proj_bf16_rejects_bad_arguments():
    lib = ctypes.CDLL(ril.LIB_PATH)
    i, p = ctypes.c_int32, ctypes.c_void_p
    lib.ril_proj_bf16.argtypes = [p, i, i, i, p, i, i, p, i, p, i, p]
    A, W, R, C = 0x10000, 0x20000, 0x30000, 0x40000
    ok = dict(A=A, rows=4, K=256, lda=256, W=W, N=64, ldw=256, R=None, ldr=0, C=C, ldo=64)

    def call(**kw):
        a = dict(ok, **kw)
        return lib.ril_proj_bf16(a["A"], a["rows"], a["K"], a["lda"], a["W"], a["N"], a["ldw"], a["R"], a["ldr"],
                                 a["C"], a["ldo"], None)
    # every case fails validation before anything is enqueued
    assert call(K=200, lda=200, ldw=200) == ril.RIL_EINVAL   # K % 32
    assert call(lda=128) == ril.RIL_EINVAL                   # lda < K
    assert call(lda=260) == ril.RIL_EINVAL                   # lda % 8
    assert call(ldw=252) == ril.RIL_EINVAL                   # ldw < K
    assert call(ldo=32) == ril.RIL_EINVAL                    # ldo < N
    assert call(R=R, ldr=32) == ril.RIL_EINVAL               # ldr < N
    assert call(A=A + 8) == ril.RIL_EINVAL                   # A misaligned
    assert call(W=W + 2) == ril.RIL_EINVAL                   # W misaligned
    assert call(C=C + 1) == ril.RIL_EINVAL                   # out misaligned
    assert call(W=None) == ril.RIL_EINVAL
    assert call(N=0) == ril.RIL_EINVAL
    assert call(lda=1 << 24) == ril.RIL_EINVAL               # 32-bit tile offsets
    assert call(rows=0) == ril.RIL_OK                        # nothing to do


def test_w8a8_pack_and_quantize_reject_bad_arguments():
    lib = ctypes.CDLL(ril.LIB_PATH)
    lib.ril_pack_lm_head_fp8.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                         ctypes.c_size_t, ctypes.c_void_p]
    lib.ril_quantize_rows_fp8.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    need = ril.ril_lm_head_fp8_packed_bytes(300, 256)
    # every case fails validation before anything is enqueued
    assert lib.ril_pack_lm_head_fp8(0x10000, 300, 200, 0x900000, need, None) == ril.RIL_EINVAL   # K % 128
    assert lib.ril_pack_lm_head_fp8(0x10000, 300, 256, 0x900000, need - 1, None) == ril.RIL_EINVAL
    assert lib.ril_pack_lm_head_fp8(0x10008, 300, 256, 0x900000, need, None) == ril.RIL_EINVAL   # misaligned
    assert lib.ril_pack_lm_head_fp8(0x10000, 300, 256, 0x10000, need, None) == ril.RIL_EINVAL    # overlap
    assert lib.ril_pack_lm_head_fp8(None, 300, 256, 0x900000, need, None) == ril.RIL_EINVAL
    assert lib.ril_quantize_rows_fp8(0x10000, 4, 200, 256, 0x20000, 0x30000, None) == ril.RIL_EINVAL  # K % 128
    assert lib.ril_quantize_rows_fp8(0x10000, 4, 256, 128, 0x20000, 0x30000, None) == ril.RIL_EINVAL  # ld < K
    assert lib.ril_quantize_rows_fp8(0x10000, 4, 256, 260, 0x20000, 0x30000, None) == ril.RIL_EINVAL  # ld % 8
    assert lib.ril_quantize_rows_fp8(0x10000, -1, 256, 256, 0x20000, 0x30000, None) == ril.RIL_EINVAL
    assert lib.ril_quantize_rows_fp8(0x10000, 4, 256, 256, 0x20008, 0x30000, None) == ril.RIL_EINVAL  # codes align
    assert lib.ril_quantize_rows_fp8(0x10000, 4, 256, 256, 0x20000, 0x30002, None) == ril.RIL_EINVAL  # exps align
    assert lib.ril_quantize_rows_fp8(0x10000, 0, 256, 256, 0x20000, 0x30000, None) == ril.RIL_OK      # nothing to do


def test_workspace_monotone_in_limits():
    sizes = []
    for mr, mt, mc in [(8, 64, 1024), (16, 64, 1024), (16, 128, 1024), (16, 128, 4096)]:
        m = ril.ril_model_create(_desc(max_rows=mr, max_tokens=mt, max_ctx=mc))
        sizes.append(ril.ril_workspace_bytes(m))
        ril.ril_model_destroy(m)
    assert sizes == sorted(sizes) and len(set(sizes)) == len(sizes)


def test_page_allocator():
    m = ril.ril_model_create(_desc())
    pb = ril.ril_kv_page_bytes(m)
    pool = torch.empty(pb * 10 + 17, dtype=torch.uint8)  # host memory stands in for the pool
    kv = ril.ril_kv_alloc(m, pool, 0)
    assert ril.ril_kv_total_pages(kv) == 10 and ril.ril_kv_free_pages(kv) == 10
    a = ril.ril_kv_assign(kv, 4)
    assert a == [0, 1, 2, 3]
    with pytest.raises(ril.RilError) as e:
        ril.ril_kv_assign(kv, 7)
    assert e.value.status == ril.RIL_ENOSPC and ril.ril_kv_free_pages(kv) == 6
    with pytest.raises(ril.RilError):
        ril.ril_kv_release(kv, [1, 1])
    with pytest.raises(ril.RilError):
        ril.ril_kv_release(kv, [5])
    assert ril.ril_kv_free_pages(kv) == 6
    ril.ril_kv_release(kv, [2, 0])
    assert ril.ril_kv_free_pages(kv) == 8
    ril.ril_kv_free(kv)
    kv = ril.ril_kv_alloc(m, pool, 1234)
    got = ril.ril_kv_assign(kv, 10)
    assert sorted(got) == list(range(10)) and got != list(range(10))
    kv2 = ril.ril_kv_alloc(m, pool, 1234)
    assert ril.ril_kv_assign(kv2, 10) == got  # seeded: reproducible
    ril.ril_kv_free(kv)
    ril.ril_kv_free(kv2)
    with pytest.raises(ril.RilError):
        ril.ril_kv_alloc(m, torch.empty(pb - 1, dtype=torch.uint8), 0)
    ril.ril_model_destroy(m)


def test_calls_fail_validation_without_enqueueing():
    m = ril.ril_model_create(_desc(max_rows=4, max_tokens=32, max_ctx=256))
    pool = torch.empty(ril.ril_kv_page_bytes(m) * 4, dtype=torch.uint8)
    kv = ril.ril_kv_alloc(m, pool, 0)
    ws = torch.empty(ril.ril_workspace_bytes(m), dtype=torch.uint8)
    i32 = lambda *x: torch.tensor(x, dtype=torch.int32)  # noqa: E731
    pt = torch.zeros(4, 16, dtype=torch.int32)
    out = torch.empty(4)
    q = torch.empty(4, 32, 128, dtype=torch.bfloat16)
    ok = dict(ctx_len=i32(5, 6), page_table=pt[:2], max_ctx_bound=256, target_ids=i32(1, 2), q=q, k=q, v=q)
    cases = [
        dict(ok, max_ctx_bound=257),                      # beyond the model's max_ctx
        dict(ok, page_table=torch.zeros(2, 15, dtype=torch.int32)),  # stride too small
        dict(ok, ctx_len=i32(*range(5))),                 # 5 rows > max_rows
        dict(ok, q=None),
        dict(ok, ctx_len=i32(), page_table=pt[:0], target_ids=i32()),  # an empty batch: rejected
    ]
    for c in cases:
        b = ril.make_decode_batch(**c)
        with pytest.raises(ril.RilError):
            ril.ril_decode_step_logprobs(m, kv, b, out, ws, stream=0)
    b = ril.make_decode_batch(**ok)
    with pytest.raises(ril.RilError) as e:
        ril.ril_decode_step_logprobs(m, kv, b, out, ws[:-1], stream=0)
    assert e.value.status == ril.RIL_ERANGE
    pb = ril.make_prefill_batch(cu_tokens=i32(0, 3), start_pos=i32(0), page_table=pt[:1], max_ctx_bound=3,
                                target_ids=i32(1, 2, 3), q=q, k=q, v=q, total_tokens=33)
    with pytest.raises(ril.RilError):
        ril.ril_prefill_logprobs(m, kv, pb, out, ws, stream=0)
    # an empty prefill (no sequence, no token) is rejected too, before anything is enqueued
    pe = ril.make_prefill_batch(cu_tokens=i32(0), start_pos=i32(), page_table=pt[:0], max_ctx_bound=3,
                                target_ids=i32(), q=q, k=q, v=q, total_tokens=0)
    with pytest.raises(ril.RilError):
        ril.ril_prefill_logprobs(m, kv, pe, out, ws, stream=0)
    ril.ril_kv_free(kv)
    ril.ril_model_destroy(m)


def test_lm_head_packed_bytes_and_pack_validation():
    # ceil(V/256) vocabulary tiles of 256 columns, K bf16 each
    assert ril.ril_lm_head_packed_bytes(129280, 4096) == 505 * 256 * 4096 * 2
    assert ril.ril_lm_head_packed_bytes(1000, 64) == 4 * 256 * 64 * 2
    for v, k in ((0, 64), (1000, 48), (1000, 0), (-1, 64)):
        assert ril.ril_lm_head_packed_bytes(v, k) == 0
    lib = ctypes.CDLL(ril.LIB_PATH)
    f = lib.ril_pack_lm_head
    f.restype = ctypes.c_int32
    f.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t,
                  ctypes.c_void_p]
    need = ril.ril_lm_head_packed_bytes(1000, 64)
    src, dst = 0x100000, 0x800000
    bad = [(None, 1000, 64, dst, need),            # null source
           (src, 1000, 64, None, need),            # null destination
           (src + 8, 1000, 64, dst, need),         # misaligned
           (src, 1000, 64, dst, need - 1),         # short destination
           (src, 1000, 48, dst, need),             # K not a multiple of 32
           (src, 1000, 64, src + 1024, need)]      # overlap
    for args in bad:
        assert f(*args, None) == ril.RIL_EINVAL, args
        assert ril.ril_last_error()


def test_hbm_read_probe_rejects_bad_pointers():
    lib = ctypes.CDLL(ril.LIB_PATH)
    lib.ril_hbm_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    assert ril.ril_hbm_read_probe_words() > 0
    assert lib.ril_hbm_read_probe(None, 1024, 0x20000, None) == ril.RIL_EINVAL
    assert lib.ril_hbm_read_probe(0x10008, 1024, 0x20000, None) == ril.RIL_EINVAL
    assert lib.ril_hbm_read_probe(0x10000, 1024, None, None) == ril.RIL_EINVAL
