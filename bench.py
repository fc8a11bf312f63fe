#!/usr/bin/env python3
"""Invariant decode tokens/s + attention HBM GB/s at diff = 0 (prefill vs decode), one MI355X.

Default workload ("gqa_decode_b64"): 64 paged GQA decode rows, 32 q / 8 kv heads,
head_dim 128, bf16 KV in 16-token pages with a random page table, contexts uniform in
[512, 8192], q/K/V ~ N(0, 1); attention output -> RMSNorm -> lm-head 4096 x 129280
(N(0, 0.02)) -> logprob of a sampled token id per row.

--workload mla_decode_b128: 128 absorbed-MLA decode rows, 128 heads sharing one paged
latent row of 512 + 64 dims, contexts uniform in [4096, 32768], scale 1/sqrt(192);
attention output -> absorbed value/output projection 65536 -> 4096 -> RMSNorm -> the
same lm-head.

Synthetic, seeded inputs (workloads module), resident in HBM before timing starts.
A step = one ril_decode_step_logprobs call for all rows.  Before timing, every row's
last 16 positions are produced both by 16 decode steps and by one prefill recompute;
the JSON line reports their diff (must be 0, bit for bit).

    python bench.py [--workload W] [--steps K] [--warmup W] [--gpus 1] [--cpu-rows R] [--no-cpu]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

HBM_PEAK_GBPS = 8000.0        # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
MFMA_FP8_PEAK_TFLOPS = 5000.0   # MI355X dense fp8 MFMA, published
METRIC = "invariant decode tokens/s + attn HBM GB/s at diff=0 (prefill vs decode)"


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def measured_traffic(kernel: str, bytes_per_launch=None):
    """HBM bytes per launch (fetch + write) from the committed rocprofv3 PMC summary,
    scaled by the copy calibration; None if the kernel's sources changed since or if the
    profiled launch moved other algorithmic bytes than this one (another shape)."""
    try:
        with open(os.path.join(ROOT, "profiles", "hbm_traffic.json")) as f:
            rec = json.load(f)[kernel]
    except (OSError, KeyError, ValueError):
        return None
    if bytes_per_launch is not None and int(bytes_per_launch) != rec.get("algorithmic_bytes"):
        return None
    h = hashlib.sha256()
    for s in rec["sources"]:
        with open(os.path.join(ROOT, "invariant_rl_logprob_amd", "csrc", s), "rb") as f:
            h.update(f.read())
    if h.hexdigest()[:16] != rec["source_sha16"]:
        return None
    return rec["fetch_bytes"] + rec["write_bytes"]


def host_info():
    """The host the oracle timing ran on: logical CPUs and the CPU model."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "cpu_model": model}


def measured_peaks():
    """Practical HBM ceilings beside the published 8 TB/s, HIP events around 5 launches on
    2 GiB: the library's nontemporal read probe (the path's streaming kernels read; this is
    their ceiling) and a device copy (read + write bytes / time)."""
    import torch
    import invariant_rl_logprob_amd as ril
    n = 2 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    out = torch.empty(ril.ril_hbm_read_probe_words(), dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    res = {}
    for name, fn, moved in (("read_peak_gbps", lambda: ril.ril_hbm_read_probe(src, out), n),
                            ("copy_peak_gbps", lambda: dst.copy_(src), 2 * n)):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(5):
            fn()
        b.record()
        torch.cuda.synchronize()
        res[name] = round(moved * 5 / (a.elapsed_time(b) * 1e-3) / 1e9, 1)
    del src, dst, out
    torch.cuda.empty_cache()
    log(f"measured HBM ceilings: {res}")
    return res


def lm_head_sweep(w, lm8, args):
    """The lm-head alone (ril_lm_head_logprobs) at M = 64, 128, 1024, 8192 and 65536 normalised
    rows: time per launch (HIP events, no trace hook), TFLOP/s against the dtype's dense
    MFMA peak, weight-stream GB/s, and whether the first 64 rows' logprobs keep their bits
    at every M (one K order per column)."""
    import numpy as np
    import torch
    import workloads as wl
    from invariant_rl_logprob_amd.session import Session
    Ms = [64, 128, 1024, 8192, 65536]
    w_lm = wl.gqa_head_weights(w, device="cuda")["w_lm"]
    sess = Session(n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads, head_dim=w.head_dim, vocab=w.vocab,
                   d_head=w.d_head, w_lm=w_lm, max_rows=64, max_tokens=max(Ms), max_ctx=64, pool_pages=8,
                   softmax_scale=1.0, lm_dtype=1 if lm8 else 0)
    del w_lm
    g = torch.Generator(device="cuda").manual_seed(77)
    z = torch.randn(max(Ms), w.d_head, generator=g, device="cuda").to(torch.bfloat16)
    t = torch.randint(0, w.vocab, (max(Ms),), generator=g, device="cuda").to(torch.int32)
    wbytes = ((w.vocab + 255) // 256) * 256 * w.d_head * (1 if lm8 else 2)
    peak = MFMA_FP8_PEAK_TFLOPS if lm8 else MFMA_BF16_PEAK_TFLOPS
    out, ref = [], None
    for M in Ms:
        launch = lambda: sess.lm_head(z[:M], t[:M])  # noqa: E731
        first = launch()
        bits = first[:64].cpu().view(torch.int32).numpy()
        ref = bits if ref is None else ref
        ms = time_launch(launch, 3 if M >= 8192 else 10, 1)
        tf = 2.0 * M * w.d_head * w.vocab / (ms * 1e-3) / 1e12
        out.append({"M": M, "us": round(ms * 1e3, 1), "tflops": round(tf, 1), "frac_of_mfma_peak": round(tf / peak, 4),
                    "weight_gbps": round(wbytes / (ms * 1e-3) / 1e9, 1),
                    "first_64_rows_bitwise_equal": bool(np.array_equal(bits, ref))})
    log(f"lm-head sweep ({'W8A8' if lm8 else 'bf16'}): {out}")
    del z, sess
    torch.cuda.empty_cache()
    return {"head": "W8A8 block FP8 (e4m3, E8M0 scales)" if lm8 else "bf16", "mfma_peak_tflops": peak, "rows": out}


def proj_w8a8_sweep():
    """The W8A8 projection GEMM alone (ril_proj_w8a8, codes and exponents from
    ril_quantize_rows_fp8 / ril_quantize_weight_fp8) on the long workload's o-projection
    shape, K = 8192 -> N = 4096, at M = 256 (a decode step's rows) and 8192 (a prefill
    chunk): time per launch (HIP events), TFLOP/s against the dense FP8 MFMA peak, and the
    rows' bits at both M (one K order for every M)."""
    import numpy as np
    import torch
    import invariant_rl_logprob_amd as ril
    N, K = 4096, 8192
    g = torch.Generator(device="cuda").manual_seed(91)
    w = (torch.randn(N, K, generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    w8 = torch.empty(ril.ril_proj_fp8_bytes(N, K), dtype=torch.uint8, device="cuda")
    ril.ril_quantize_weight_fp8(w, w8)
    del w
    out, first = [], None
    xs = torch.randn(8192, K, generator=g, device="cuda").to(torch.bfloat16)
    for M in (256, 8192):
        x = xs[:M]
        codes = torch.empty((M, K), dtype=torch.uint8, device="cuda")
        exps = torch.empty((M, K // 128), dtype=torch.int32, device="cuda")
        ril.ril_quantize_rows_fp8(x, codes, exps)
        y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        ms = time_launch(lambda: ril.ril_proj_w8a8(codes, exps, w8, N, y), 10 if M <= 256 else 3, 1)
        bits = y[:64].view(torch.int16).cpu().numpy()
        first = bits if first is None else first
        tf = 2.0 * M * N * K / (ms * 1e-3) / 1e12
        out.append({"M": M, "us": round(ms * 1e3, 1), "tflops": round(tf, 1),
                    "frac_of_fp8_mfma_peak": round(tf / MFMA_FP8_PEAK_TFLOPS, 4),
                    "weight_gbps": round(N * K / (ms * 1e-3) / 1e9, 1),
                    "first_64_rows_bitwise_equal": bool(np.array_equal(bits, first))})
        del x, codes, exps, y
    del xs
    log(f"W8A8 projection sweep (K {K} -> N {N}): {out}")
    torch.cuda.empty_cache()
    return {"shape": f"K {K} -> N {N}", "rows": out}


def lm_head_rows(M):
    """One untimed and three timed launches of the bf16 lm-head (ril_lm_head_logprobs) on M
    N(0,1) rows of the GQA workload's head: the command the lm-head kernel profiles use."""
    import torch
    import workloads as wl
    from invariant_rl_logprob_amd.session import Session
    w = wl.GQA_DECODE_B64
    w_lm = wl.gqa_head_weights(w, device="cuda")["w_lm"]
    sess = Session(n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads, head_dim=w.head_dim, vocab=w.vocab,
                   d_head=w.d_head, w_lm=w_lm, max_rows=64, max_tokens=M, max_ctx=64, pool_pages=8,
                   softmax_scale=1.0)
    del w_lm
    g = torch.Generator(device="cuda").manual_seed(77)
    z = torch.randn(M, w.d_head, generator=g, device="cuda").to(torch.bfloat16)
    t = torch.randint(0, w.vocab, (M,), generator=g, device="cuda").to(torch.int32)
    ms = time_launch(lambda: sess.lm_head(z, t), 3, 1)
    tf = 2.0 * M * w.d_head * w.vocab / (ms * 1e-3) / 1e12
    return {"lm_head_rows": M, "us_per_launch": round(ms * 1e3, 1), "tflops": round(tf, 1),
            "frac_of_mfma_peak": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)}


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        return os.cpu_count()


def timed_steps(launch, steps, warmup):
    """Warm up, then time `steps` launches between two synchronisations with HIP events on
    the launch stream: that pass gives the step time.  A second pass of `steps` launches runs
    with the library's trace hook (HIP events around every kernel on that stream) and gives
    each kernel's average duration; the hook's events add about 10% to a step, so the step
    time never comes from the traced pass."""
    import torch
    import invariant_rl_logprob_amd as ril
    for _ in range(warmup):
        launch()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        launch()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    ril.ril_trace_enable(True)
    for _ in range(steps):
        launch()
    torch.cuda.synchronize()
    kern = {}
    for kid, name in enumerate(ril.KERNEL_NAMES):
        tot, cnt = ril.ril_trace_read(kid)
        if cnt:
            kern[name] = {"avg_us": 1e3 * tot / cnt, "launches": cnt}
    ril.ril_trace_enable(False)
    return ms, kern


def time_launch(launch, steps, warmup):
    """ms per launch over `steps` launches between two HIP events (no per-kernel trace)."""
    import torch
    for _ in range(warmup):
        launch()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        launch()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def graph_leg(sess, seqs, c, kw, eager_launch, eager_out, args):
    """The same decode step captured in a HIP graph: replay time next to the eager call's
    (both timed without the trace hook), and whether the replay's bits equal the eager ones."""
    import numpy as np
    import torch
    def host_us(launch, n=20):  # host time to enqueue one step (the GPU queue never fills at n)
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(n):
            launch()
        dt = time.perf_counter() - t
        torch.cuda.synchronize()
        return 1e6 * dt / n

    g = sess.decode_graph(seqs, max(c), ctx=c, **kw)
    try:
        eager_ms = time_launch(eager_launch, args.steps, args.warmup)
        e_bits = eager_out.cpu().view(torch.int32).numpy().copy()
        graph_ms = time_launch(g.replay, args.steps, args.warmup)
        equal = bool(np.array_equal(g.out.cpu().view(torch.int32).numpy(), e_bits))
        eager_host, graph_host = host_us(eager_launch), host_us(g.replay)
    finally:
        g.close()
    return {"rows": len(seqs), "eager_ms_per_step": round(eager_ms, 4), "graph_ms_per_step": round(graph_ms, 4),
            "graph_speedup": round(eager_ms / graph_ms, 3), "eager_host_enqueue_us": round(eager_host, 1),
            "graph_host_enqueue_us": round(graph_host, 1), "bitwise_equal_to_eager": equal}


def tiny_graph_leg(args):
    """cfg-1 decoder (token input, one layer, 4 sequences): one decode step eager vs graph."""
    import torch
    import workloads as wl
    from invariant_rl_logprob_amd import RIL_INPUT_TOKENS
    from invariant_rl_logprob_amd.session import Session
    W = wl.TINY
    wts = wl.tiny_weights(W, device="cuda")
    toks = [wl.tiny_tokens(i, W, device="cuda") for i in range(len(W.lengths))]
    s = Session(n_q_heads=W.n_q_heads, n_kv_heads=W.n_kv_heads, head_dim=W.head_dim, vocab=W.vocab,
                d_head=W.d_model, d_model=W.d_model, w_lm=wts["w_lm"], embed=wts["embed"], w_qkv=wts["w_qkv"],
                w_o=wts["w_o"], norm_attn=wts["norm_attn"], norm_final=wts["norm_final"], max_rows=8,
                max_tokens=512, max_ctx=max(W.lengths), pool_pages=4096, softmax_scale=1.0 / math.sqrt(W.head_dim),
                rms_eps=W.rms_eps, shuffle_seed=3, input_mode=RIL_INPUT_TOKENS)
    P = W.prompt_tokens
    ids = list(range(len(W.lengths)))
    seqs = [("t", i) for i in ids]
    s.prefill(seqs, [0] * len(ids), targets=[toks[i][1:P + 1] for i in ids], tokens=[toks[i][:P] for i in ids])
    tok = torch.stack([toks[i][P] for i in ids]).to(torch.int32)
    tgt = torch.stack([toks[i][P + 1] for i in ids]).to(torch.int32)
    c = [P + 1] * len(ids)
    launch, out = s.prepare_decode(seqs, c, targets=tgt, tokens=tok)
    return graph_leg(s, seqs, c, {"targets": tgt, "tokens": tok}, launch, out, args)


def diff_check(case, rows, n=16):
    """n decode steps per row vs one prefill recompute of the same n positions."""
    import torch
    from invariant_rl_logprob_amd.metrics import mismatch
    case.write_history("d", rows, n)
    dec = torch.stack([case.decode_back("d", rows, back) for back in range(n, 0, -1)], dim=1)
    case.write_history("p", rows, n)
    pre = case.prefill_last("p", rows, n)
    torch.cuda.synchronize()
    d = mismatch(dec, pre)
    log(f"prefill vs decode over {d['tokens']} tokens: {d}")
    return dec, d


def roofline_hbm(kernel, achieved_gbps, bytes_per_launch, avg_us):
    return {"bound": "hbm", "achieved": round(achieved_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved_gbps / HBM_PEAK_GBPS, 4), "traffic": measured_traffic(kernel, bytes_per_launch),
            "kernel": kernel, "algorithmic_bytes_per_launch": int(bytes_per_launch),
            "avg_launch_us": round(avg_us, 2)}


def comparator(sess, prepare, rows, ref_last, attn_bytes, splits, args):
    """X1: the same kernels with shape-derived work splits (ril_set_policy
    RIL_POLICY_SHAPE_DERIVED): the KV split from the batch (or each fixed override in
    `splits`, so the comparator is tuned as hard as the invariant build) and split-K
    for small projection grids.  Reports the best X1 step at the full batch, its diff
    against the invariant result (nonzero: X1 decode no longer equals prefill), and
    invariant vs X1 (shape rule) over batch sizes 1, 8 and all rows."""
    import invariant_rl_logprob_amd as ril
    from invariant_rl_logprob_amd.metrics import mismatch
    steps, warmup = max(10, args.steps // 2), max(2, args.warmup)

    def run(rs, policy, split=0):
        sess.set_policy(policy, split)
        launch, out = prepare(rs)
        ms, kern = timed_steps(launch, steps, warmup)
        attn_us = kern["attn_split"]["avg_us"] + kern["attn_merge"]["avg_us"]
        return ms, attn_us, kern, out

    try:
        trials = []
        for sp in [0] + list(splits):
            ms, attn_us, kern, out = run(rows, ril.RIL_POLICY_SHAPE_DERIVED, sp)
            t = {"attn_split": "shape rule" if sp == 0 else sp, "ms_per_step": round(ms, 4),
                 "tokens_per_s": round(len(rows) / (ms * 1e-3), 1),
                 "attn_hbm_gbps": round(attn_bytes / (attn_us * 1e-6) / 1e9, 1),
                 "kernels_avg_us": {k_: round(v_["avg_us"], 2) for k_, v_ in kern.items()}}
            if sp == 0:
                t["diff_vs_invariant"] = mismatch(out[:, None], ref_last[:, None])
            trials.append(t)
        best = min(trials, key=lambda t: t["ms_per_step"])
        sweep = []
        for b in sorted({1, 8, len(rows)}):
            rs = rows[:b]
            inv_ms = run(rs, ril.RIL_POLICY_INVARIANT)[0]
            x1_ms = run(rs, ril.RIL_POLICY_SHAPE_DERIVED)[0]
            sweep.append({"rows": b, "invariant_tokens_per_s": round(b / (inv_ms * 1e-3), 1),
                          "x1_tokens_per_s": round(b / (x1_ms * 1e-3), 1),
                          "invariant_over_x1": round(x1_ms / inv_ms, 4)})
    finally:
        sess.set_policy(ril.RIL_POLICY_INVARIANT)
    log(f"comparator: best {best['attn_split']} {best['tokens_per_s']} tok/s; sweep {sweep}")
    return {"kind": "same kernels, shape-derived split-KV and split-K (non-invariant)",
            "best": best, "trials": trials, "batch_sweep": sweep}


# ---------------------------------------------------------------------------
# GQA decode, 64 rows
# ---------------------------------------------------------------------------

def bench_gqa_fp8(args):
    return bench_gqa(args, fp8=True)


def bench_gqa_w8a8(args):
    return bench_gqa(args, lm8=True)


def bench_gqa_fp8_w8a8(args):
    return bench_gqa(args, fp8=True, lm8=True)


def bench_gqa(args, fp8=False, lm8=False):
    import numpy as np
    import torch
    import workloads as wl
    from gqa_case import GQACase

    w = wl.GQA_DECODE_B64
    rows = list(range(w.rows))
    t0 = time.time()
    case = GQACase(w, rows, device="cuda", shuffle_seed=0x5EED, copies=2, max_tokens=w.rows * 16,
                   kv_dtype=1 if fp8 else 0, lm_dtype=1 if lm8 else 0)
    ctx = [case.ctx(r) for r in rows]
    log(f"data ready in {time.time() - t0:.1f}s; sum ctx = {sum(ctx)}")
    dec, diff = diff_check(case, rows)

    q, k, v, tgt, c = case.step_inputs(rows, 1)
    launch, out = case.sess.prepare_decode([("d", r) for r in rows], c, targets=tgt, q=q, k=k, v=v)
    ms_step, kern = timed_steps(launch, args.steps, args.warmup)
    last_equal = bool(np.array_equal(out.cpu().view(torch.int32).numpy(),
                                     dec[:, -1].cpu().view(torch.int32).numpy()))

    Hkv, D, Hq = w.n_kv_heads, w.head_dim, w.n_q_heads
    kv_bytes = sum(ctx) * Hkv * D * 2 * (1 if fp8 else 2)  # each K/V byte once per kv head
    q_bytes = len(rows) * Hq * D * 2
    out_bytes = len(rows) * Hq * D * 2
    if lm8:  # E4M3 weight codes + their block scales, the rows' codes + scales
        n_vt = (w.vocab + 255) // 256
        lm_bytes = n_vt * 256 * w.d_head + 2 * n_vt * (w.d_head // 128) * 4 + len(rows) * w.d_head * (1 + 4 / 128)
    else:
        lm_bytes = w.vocab * w.d_head * 2 + len(rows) * w.d_head * 2
    lm_name = "lm_head_fp8" if lm8 else "lm_head"
    split_us, merge_us, lm_us = kern["attn_split"]["avg_us"], kern["attn_merge"]["avg_us"], kern[lm_name]["avg_us"]
    attn_gbps = (kv_bytes + q_bytes + out_bytes) / ((split_us + merge_us) * 1e-6) / 1e9
    split_gbps = (kv_bytes + q_bytes) / (split_us * 1e-6) / 1e9
    lm_gbps = lm_bytes / (lm_us * 1e-6) / 1e9
    if split_us >= lm_us:
        roof = roofline_hbm("attn_decode_split_fp8" if fp8 else "attn_decode_split", split_gbps, kv_bytes + q_bytes,
                            split_us)
    else:
        roof = roofline_hbm(lm_name, lm_gbps, lm_bytes, lm_us)

    x1 = None
    if not args.no_comparator:
        def prepare(rs):
            q_, k_, v_, t_, c_ = case.step_inputs(rs, 1)
            return case.sess.prepare_decode([("d", r) for r in rs], c_, targets=t_, q=q_, k=k_, v=v_)
        x1 = comparator(case.sess, prepare, rows, dec[:, -1], kv_bytes + q_bytes + out_bytes, (256, 512, 1024), args)
        x1["invariant_over_x1_best"] = round(x1["best"]["ms_per_step"] / ms_step, 4)

    sweep = None if args.no_lm_sweep else lm_head_sweep(w, lm8, args)
    proj_sweep = None if args.no_lm_sweep else proj_w8a8_sweep()
    peaks = measured_peaks()

    graph = None
    if not args.no_graph:
        graph = {"gqa_decode_b64": graph_leg(case.sess, [("d", r) for r in rows], c,
                                             {"targets": tgt, "q": q, "k": k, "v": v}, launch, out, args),
                 "tiny_decoder": tiny_graph_leg(args)}
        log(f"graph: {graph}")

    cpu = None
    if lm8:
        log("oracle: not timed here (its W8A8 head quantizes the whole 129280 x 4096 weight per row)")
    elif not args.no_cpu and args.cpu_rows > 0:
        import oracle  # the cpu_baseline leg: the fp64 oracle as it stands
        sample = rows[: args.cpu_rows]
        w_lm_cpu = case.head["w_lm"].cpu()
        host = {r: {key: case.data[r][key].cpu() for key in ("q", "k", "v", "target")} for r in sample}
        t1 = time.time()
        def kv(x):  # the FP8 cache gives back its decode of the stored codes
            return oracle.kv_fp8_roundtrip(oracle.widen(x), 0) if fp8 else x
        got = [oracle.gqa_row_logprob(host[r]["q"][-1], kv(host[r]["k"][: case.ctx(r)]),
                                      kv(host[r]["v"][: case.ctx(r)]), 1.0 / math.sqrt(D), w_lm_cpu,
                                      int(host[r]["target"][-1]), w.rms_eps)
               for r in sample]
        secs = time.time() - t1
        cpu = {"value": round(len(sample) / secs, 4), "unit": "tokens/s", "cores": blas_threads(), "kind": "oracle",
               **host_info(),
               "sample": f"{len(sample)} of the {len(rows)} decode rows (full attention over each row's "
                         f"context + the 4096x129280 lm-head in fp64), {secs:.1f} s",
               "max_abs_diff_vs_gpu": float(np.max(np.abs(np.array(got) - out.cpu().numpy()[: len(sample)])))}
        log(f"oracle: {cpu}")

    return {
        "value": round(len(rows) / (ms_step * 1e-3), 1), "ms_per_step": round(ms_step, 4),
        "dtype": "bf16 (attention), e4m3 (lm-head)" if lm8 else "bf16",
        "config": {"workload": "gqa_decode_b64" + ("_fp8" if fp8 else "") + ("_w8a8" if lm8 else "")
                   + ": 64 paged decode rows, 32 q / 8 kv heads, head_dim 128, ctx U[512,8192], 16-token pages, "
                     "random page table, lm-head 4096x129280"
                   + (", FP8 E4M3 KV cache (scale 1)" if fp8 else "")
                   + (", W8A8 block-FP8 lm-head (1x128 / 128x128 E8M0 scales)" if lm8 else ""),
                   "rows": len(rows), "sum_ctx": sum(ctx), "split_tokens": 512, "vocab_tile": 256,
                   "parallelism": "none (1 GPU)"},
        "attn_hbm_gbps": round(attn_gbps, 1), "attn_frac_of_peak": round(attn_gbps / HBM_PEAK_GBPS, 4),
        **peaks, "attn_frac_of_read_peak": round(attn_gbps / peaks["read_peak_gbps"], 4),
        "lm_head_sweep": sweep, "proj_w8a8_sweep": proj_sweep,
        "lm_head_gbps": round(lm_gbps, 1), "diff": diff, "timed_step_equals_checked_decode": last_equal,
        "kernels_avg_us": {k_: round(v_["avg_us"], 2) for k_, v_ in kern.items()},
        "comparator_x1": x1, "hip_graph": graph, "roofline": roof, "cpu_baseline": cpu,
    }


# ---------------------------------------------------------------------------
# absorbed MLA decode, 128 rows
# ---------------------------------------------------------------------------

def bench_mla(args, fp8=False):
    import numpy as np
    import torch
    import workloads as wl
    from mla_case import MLACase

    w = wl.MLA_DECODE_B128
    rows = list(range(w.rows))
    t0 = time.time()
    case = MLACase(w, rows, device="cuda", shuffle_seed=0x5EED, copies=2, max_rows=w.rows,
                   max_tokens=w.rows * w.recompute_tokens, kv_dtype=1 if fp8 else 0)
    ctx = [case.ctx(r) for r in rows]
    log(f"data ready in {time.time() - t0:.1f}s; sum ctx = {sum(ctx)}")
    dec, diff = diff_check(case, rows)

    q = torch.stack([case.data[r]["q"][-1] for r in rows])
    cl = torch.stack([case.data[r]["c"][case.ctx(r) - 1] for r in rows])
    tgt = torch.stack([case.data[r]["target"][-1] for r in rows])
    launch, out = case.sess.prepare_decode([("d", r) for r in rows], ctx, targets=tgt, q=q, k=cl)
    ms_step, kern = timed_steps(launch, args.steps, args.warmup)
    last_equal = bool(np.array_equal(out.cpu().view(torch.int32).numpy(),
                                     dec[:, -1].cpu().view(torch.int32).numpy()))

    H = w.n_heads
    kv_bytes = sum(ctx) * (w.kv_rank + w.rope_dim) * (1 if fp8 else 2)
    flops = sum(ctx) * H * 2 * ((w.kv_rank + w.rope_dim) + w.kv_rank)
    split_us, merge_us = kern["attn_split"]["avg_us"], kern["attn_merge"]["avg_us"]
    attn_gbps = kv_bytes / ((split_us + merge_us) * 1e-6) / 1e9
    split_gbps = kv_bytes / (split_us * 1e-6) / 1e9
    tflops = flops / (split_us * 1e-6) / 1e12
    roof = roofline_hbm("mla_split_fp8" if fp8 else "mla_split", split_gbps, kv_bytes, split_us)
    roof["mfma"] = {"achieved": round(tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "flops_per_launch": int(flops)}

    cpu = None
    if not args.no_cpu and args.cpu_rows > 0:
        import oracle  # the cpu_baseline leg
        sample = rows[: max(1, args.cpu_rows // 4)]
        w_lm_cpu = case.head["w_lm"].cpu()
        w_o_cpu = case.head["w_o"].cpu()
        host = {r: {key: case.data[r][key].cpu() for key in ("q", "c", "target")} for r in sample}
        t1 = time.time()
        got = []
        for r in sample:
            o = oracle.mla_row_attention(host[r]["q"][-1], case.cached(host[r]["c"][: case.ctx(r)]), case.scale,
                                         w.kv_rank)
            got.append(oracle.head_logprob(o, w_lm_cpu, int(host[r]["target"][-1]), w.rms_eps, w_o=w_o_cpu))
        secs = time.time() - t1
        cpu = {"value": round(len(sample) / secs, 4), "unit": "tokens/s", "cores": blas_threads(), "kind": "oracle",
               **host_info(), "sample": f"{len(sample)} of the {len(rows)} decode rows (MLA over each row's context, the "
                         f"65536x4096 projection and the lm-head in fp64), {secs:.1f} s",
               "max_abs_diff_vs_gpu": float(np.max(np.abs(np.array(got) - out.cpu().numpy()[: len(sample)])))}
        log(f"oracle: {cpu}")

    return {
        "value": round(len(rows) / (ms_step * 1e-3), 1), "ms_per_step": round(ms_step, 4),
        "config": {"workload": ("mla_decode_b128_fp8" if fp8 else "mla_decode_b128") + ": 128 absorbed-MLA decode "
                               "rows, 128 heads, latent 512 + rope 64" + (" in an FP8 E4M3 cache" if fp8 else "") +
                               ", ctx U[4096,32768], 16-token pages, random page table, o-proj 65536x4096, "
                               "lm-head 4096x129280",
                   "rows": len(rows), "sum_ctx": sum(ctx), "split_tokens": 2048, "parallelism": "none (1 GPU)"},
        "attn_hbm_gbps": round(attn_gbps, 1), "attn_frac_of_peak": round(attn_gbps / HBM_PEAK_GBPS, 4),
        "diff": diff, "timed_step_equals_checked_decode": last_equal,
        "kernels_avg_us": {k_: round(v_["avg_us"], 2) for k_, v_ in kern.items()},
        "roofline": roof, "cpu_baseline": cpu,
    }


# ---------------------------------------------------------------------------
# sparse MLA over the indexer's top-2048, 32 rows of 65536 positions
# ---------------------------------------------------------------------------

def bench_sparse(args, fp8=False):
    import numpy as np
    import torch
    import workloads as wl
    from sparse_case import SparseCase

    w = wl.SPARSE_MLA_B32
    rows = list(range(w.rows))
    t0 = time.time()
    case = SparseCase(w, rows, device="cuda", shuffle_seed=0x5EED, copies=2, max_rows=w.rows,
                      max_tokens=w.rows * w.recompute_tokens, kv_dtype=1 if fp8 else 0)
    ctx = [case.ctx(r) for r in rows]
    log(f"data ready in {time.time() - t0:.1f}s; sum ctx = {sum(ctx)}")
    dec, diff = diff_check(case, rows)

    d = case.data
    q = torch.stack([d[r]["q"][-1] for r in rows])
    qi = torch.stack([d[r]["q_index"][-1] for r in rows])
    cl = torch.stack([d[r]["c"][case.ctx(r) - 1] for r in rows])
    ki = torch.stack([d[r]["k_index"][case.ctx(r) - 1] for r in rows])
    tgt = torch.stack([d[r]["target"][-1] for r in rows])
    launch, out = case.sess.prepare_decode([("d", r) for r in rows], ctx, targets=tgt, q=q, k=cl, q_index=qi,
                                           k_index=ki)
    ms_step, kern = timed_steps(launch, args.steps, args.warmup)
    last_equal = bool(np.array_equal(out.cpu().view(torch.int32).numpy(),
                                     dec[:, -1].cpu().view(torch.int32).numpy()))

    # indexer: every position's fp32 key (512 B) once per row; 2 flops per multiply-add
    idx_bytes = sum(ctx) * w.index_dim * 4
    idx_flops = sum(ctx) * w.index_heads * w.index_dim * 2
    idx_us = kern["indexer"]["avg_us"]
    idx_gbps = idx_bytes / (idx_us * 1e-6) / 1e9
    idx_tflops = idx_flops / (idx_us * 1e-6) / 1e12
    # The indexer's terms are single fp32 fused multiply-adds (v_fma_f32: 2 flops, one
    # rounding) and packed fp32 forms are disabled, so its ALU ceiling is one FMA per lane
    # per clock: 256 CUs x 4 SIMDs x 16 lanes x 2 flops x 2.4 GHz = 78.6 TFLOP/s.  (The
    # published 157.3 TFLOP/s counts packed dual fp32 FMAs: 2x this.)
    FP32_FMA_PEAK_TFLOPS = 256 * 4 * 16 * 2 * 2.4e9 / 1e12
    roof = {"bound": "alu", "achieved": round(idx_tflops, 2), "peak": round(FP32_FMA_PEAK_TFLOPS, 2),
            "unit": "TFLOP/s", "frac": round(idx_tflops / FP32_FMA_PEAK_TFLOPS, 4),
            "traffic": measured_traffic("indexer"),
            "kernel": "indexer", "algorithmic_flops_per_launch": int(idx_flops), "avg_launch_us": round(idx_us, 2),
            "hbm_gbps": round(idx_gbps, 1)}
    sel_n = sum(min(c_, w.topk) for c_ in ctx)
    attn_bytes = sel_n * (w.kv_rank + w.rope_dim) * (1 if fp8 else 2)
    attn_us = kern["attn_split"]["avg_us"] + kern["attn_merge"]["avg_us"]

    cpu = None
    if not args.no_cpu and args.cpu_rows > 0:
        import oracle  # the cpu_baseline leg
        sample = rows[: max(1, args.cpu_rows // 6)]
        t1 = time.time()
        got = [case.oracle_row(r)[0] for r in sample]
        secs = time.time() - t1
        cpu = {"value": round(len(sample) / secs, 4), "unit": "tokens/s", "cores": blas_threads(), "kind": "oracle",
               **host_info(), "sample": f"{len(sample)} of the {len(rows)} decode rows (fp32 indexer over 65536 positions, "
                         f"top-2048, sparse MLA, projection and lm-head in fp64), {secs:.1f} s",
               "max_abs_diff_vs_gpu": float(np.max(np.abs(np.array(got) - out.cpu().numpy()[: len(sample)])))}
        log(f"oracle: {cpu}")

    return {
        "value": round(len(rows) / (ms_step * 1e-3), 1), "ms_per_step": round(ms_step, 4),
        "config": {"workload": ("sparse_mla_b32_fp8" if fp8 else "sparse_mla_b32") + ": 32 decode rows of 65536 "
                               "positions, fp32 indexer 64 heads x 128, stable top-2048 (ties to the lower "
                               "position), MLA 128 heads over the selection" + (" from an FP8 E4M3 latent cache"
                               if fp8 else "") + ", o-proj 65536x4096, lm-head 4096x129280",
                   "rows": len(rows), "sum_ctx": sum(ctx), "split_entries": 256, "parallelism": "none (1 GPU)"},
        "attn_hbm_gbps": round(attn_bytes / (attn_us * 1e-6) / 1e9, 1),
        "diff": diff, "timed_step_equals_checked_decode": last_equal,
        "kernels_avg_us": {k_: round(v_["avg_us"], 2) for k_, v_ in kern.items()},
        "roofline": roof, "cpu_baseline": cpu,
    }


# ---------------------------------------------------------------------------
# long context: 256 decode rows at contexts up to 128K, and the chunked prefill of
# 8 x 131072-token sequences mixed with those rows
# ---------------------------------------------------------------------------

def bench_long(args):
    import numpy as np
    import torch
    import invariant_rl_logprob_amd as ril
    import workloads as wl
    from invariant_rl_logprob_amd.metrics import mismatch
    from long_case import LongMixCase

    w = wl.LONG_MIX
    m = w.decode
    t0 = time.time()
    case = LongMixCase(w, progress=log)
    rows = case.rows
    ctx = [case.ctx[r] for r in rows]
    log(f"data ready in {time.time() - t0:.1f}s; decode sum ctx = {sum(ctx)}")
    ref = case.decode_reference()
    st = lambda key: torch.stack([case.dec[r][key][-1] for r in rows])  # noqa: E731
    launch, out = case.sess.prepare_decode([("D", r) for r in rows], ctx, targets=st("target"), q=st("q"),
                                           k=st("k"), v=st("v"))
    ms_step, kern = timed_steps(launch, args.steps, args.warmup)
    last_equal = bool(np.array_equal(out.cpu().view(torch.int32).numpy(), ref[:, -1].cpu().view(torch.int32).numpy()))
    kv_bytes = sum(ctx) * m.n_kv_heads * m.head_dim * 2 * 2
    q_bytes = len(rows) * m.n_q_heads * m.head_dim * 2
    split_us, merge_us = kern["attn_split"]["avg_us"], kern["attn_merge"]["avg_us"]
    split_gbps = (kv_bytes + q_bytes) / (split_us * 1e-6) / 1e9
    roof = roofline_hbm("attn_decode_split", split_gbps, kv_bytes + q_bytes, split_us)
    log(f"decode: {ms_step:.3f} ms/step, split {split_us:.1f} us ({split_gbps:.0f} GB/s)")

    # chunked prefill mixed with the decode rows; the trace hook times every kernel
    sched = [(8192, 0), (2048, 1), (512, 2)]
    runs, prefill = [], {}
    L, S = case.L, len(case.seqs)
    pos_sum = S * L * (L + 1) // 2  # sum over long positions of (p + 1)
    attn_flops = 4 * m.head_dim * m.n_q_heads * pos_sum
    for chunk, mix in sched:
        torch.cuda.synchronize()
        ril.ril_trace_enable(True)
        t1 = time.time()
        lp_long, lp_dec = case.run_schedule(chunk, mix, ("bench", chunk, mix))
        secs = time.time() - t1
        kt = {}
        for kid, name in enumerate(ril.KERNEL_NAMES):
            tot, cnt = ril.ril_trace_read(kid)
            if cnt:
                kt[name] = round(tot, 3)
        ril.ril_trace_enable(False)
        runs.append((lp_long, lp_dec))
        toks = S * L + len(rows) * case.nd
        ap_ms = kt.get("attn_prefill", float("nan"))
        lm_ms = kt.get("lm_head", float("nan"))
        prefill[f"chunk_{chunk}_mix_{mix}"] = {
            "wall_s": round(secs, 2), "tokens": toks, "tokens_per_s": round(toks / secs, 1),
            "kernel_ms": kt,
            "attn_prefill_tflops": round(attn_flops / (ap_ms * 1e-3) / 1e12, 1),
            "attn_prefill_frac_of_bf16_peak": round(attn_flops / (ap_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "lm_head_tflops": round(2.0 * toks * m.d_head * m.vocab / (lm_ms * 1e-3) / 1e12, 1)}
        log(f"prefill chunk {chunk} mix {mix}: {prefill[f'chunk_{chunk}_mix_{mix}']}")
    long0, dec0 = runs[0]
    diff_long = mismatch(long0.reshape(-1), runs[1][0].reshape(-1))
    diff_dec = mismatch(dec0.reshape(-1), ref.reshape(-1))
    for lp_long, lp_dec in runs[2:]:
        diff_long = max(diff_long, mismatch(long0.reshape(-1), lp_long.reshape(-1)), key=lambda d: d["max"])
    log(f"long positions across chunk sizes/mixes: {diff_long}; decode rows in mixes vs decode steps: {diff_dec}")

    cpu = None
    if not args.no_cpu and args.cpu_rows > 0:
        import oracle  # the cpu_baseline leg
        picks = [(0, 0), (0, L - 1), (1, 8191), (1, 8192)][: max(1, args.cpu_rows // 3)]
        t1 = time.time()
        got = [case.oracle_long(s_, p_) for s_, p_ in picks]
        secs = time.time() - t1
        gpu = long0.cpu().numpy()
        cpu = {"value": round(len(picks) / secs, 4), "unit": "tokens/s", "cores": blas_threads(), "kind": "oracle",
               **host_info(), "sample": f"{len(picks)} long-sequence positions {picks} (attention over up to 131072 positions, "
                         f"8192->4096 projection and lm-head in fp64), {secs:.1f} s",
               "max_abs_diff_vs_gpu": float(max(abs(gpu[s_, p_] - g_) for (s_, p_), g_ in zip(picks, got)))}
        log(f"oracle: {cpu}")

    return {
        "value": round(len(rows) / (ms_step * 1e-3), 1), "ms_per_step": round(ms_step, 4),
        "config": {"workload": "long_mix: 256 GQA decode rows (64 q / 8 kv heads, head_dim 128) at contexts "
                               "U[1024,131072], o-proj 8192x4096, lm-head 4096x129280; plus the chunked prefill "
                               "of 8 x 131072-token sequences mixed with those rows",
                   "rows": len(rows), "sum_ctx": sum(ctx), "split_tokens": 512, "parallelism": "none (1 GPU)"},
        "attn_split_hbm_gbps": round(split_gbps, 1), "decode_diff_vs_mixed_prefill": diff_dec,
        "long_positions_diff_across_chunks_and_mixes": diff_long,
        "timed_step_equals_checked_decode": last_equal,
        "kernels_avg_us": {k_: round(v_["avg_us"], 2) for k_, v_ in kern.items()},
        "prefill": prefill, "roofline": roof, "cpu_baseline": cpu,
    }


def long_decode_leg(args):
    """The long-context workload's decode step at its own size, next to the headline line:
    256 GQA decode rows (64 q / 8 kv heads, head_dim 128) at contexts U[1024, 131072]
    (about 73.5 GB of KV per step), the 8192 -> 4096 output projection and the 4096 x 129280
    lm-head.  Its 16 last positions are produced by 16 plain decode steps and by one prefill
    recompute (diff, must be 0); the step is timed like the headline's; the oracle times a
    sample of rows."""
    import numpy as np
    import torch
    import workloads as wl
    from invariant_rl_logprob_amd.metrics import mismatch
    from long_case import LongMixCase

    w = wl.LONG_MIX
    m = w.decode
    t0 = time.time()
    case = LongMixCase(w, n_seqs=0, progress=log, max_tokens=m.rows * w.decode_tokens)
    rows = case.rows
    ctx = [case.ctx[r] for r in rows]
    log(f"long decode: data ready in {time.time() - t0:.1f}s; sum ctx = {sum(ctx)}")
    ref = case.decode_reference()
    pre = case.decode_rows_recompute()
    torch.cuda.synchronize()
    diff = mismatch(ref, pre)
    log(f"long decode: decode steps vs prefill recompute over {diff['tokens']} tokens: {diff}")
    st = lambda key: torch.stack([case.dec[r][key][-1] for r in rows])  # noqa: E731
    launch, out = case.sess.prepare_decode([("D", r) for r in rows], ctx, targets=st("target"), q=st("q"),
                                           k=st("k"), v=st("v"))
    ms_step, kern = timed_steps(launch, args.steps, args.warmup)
    last_equal = bool(np.array_equal(out.cpu().view(torch.int32).numpy(), ref[:, -1].cpu().view(torch.int32).numpy()))
    kv_bytes = sum(ctx) * m.n_kv_heads * m.head_dim * 2 * 2
    q_bytes = len(rows) * m.n_q_heads * m.head_dim * 2
    split_us, merge_us = kern["attn_split"]["avg_us"], kern["attn_merge"]["avg_us"]
    split_gbps = (kv_bytes + q_bytes) / (split_us * 1e-6) / 1e9
    attn_gbps = (kv_bytes + 2 * q_bytes) / ((split_us + merge_us) * 1e-6) / 1e9
    roof = roofline_hbm("attn_decode_split__long_mix_b256", split_gbps, kv_bytes + q_bytes, split_us)
    log(f"long decode: {ms_step:.3f} ms/step, split {split_us:.1f} us ({split_gbps:.0f} GB/s)")
    cpu = None
    if not args.no_cpu and args.cpu_rows > 0:
        import oracle  # noqa: F401  (the cpu_baseline leg: case.oracle_decode runs the fp64 oracle)
        by_ctx = sorted(rows, key=lambda r: case.ctx[r])
        sample = [by_ctx[0], by_ctx[len(by_ctx) // 2]]
        t1 = time.time()
        got = [case.oracle_decode(r, case.nd - 1) for r in sample]
        secs = time.time() - t1
        gpu = ref[:, -1].cpu().numpy()
        cpu = {"value": round(len(sample) / secs, 4), "unit": "tokens/s", "cores": blas_threads(), "kind": "oracle",
               **host_info(), "sample": f"decode rows {sample} at contexts {[case.ctx[r] for r in sample]} (attention "
                                        f"over the whole context, 8192->4096 projection and lm-head in fp64), {secs:.1f} s",
               "max_abs_diff_vs_gpu": float(max(abs(gpu[r] - g_) for r, g_ in zip(sample, got)))}
        log(f"long decode oracle: {cpu}")
    res = {"value": round(len(rows) / (ms_step * 1e-3), 1), "unit": "tokens/s", "ms_per_step": round(ms_step, 4),
           "config": {"workload": "long_mix decode: 256 GQA decode rows (64 q / 8 kv heads, head_dim 128) at contexts "
                                  "U[1024,131072], 16-token pages, random page table, o-proj 8192x4096, "
                                  "lm-head 4096x129280",
                      "rows": len(rows), "sum_ctx": sum(ctx), "split_tokens": 512},
           "attn_hbm_gbps": round(attn_gbps, 1), "attn_frac_of_peak": round(attn_gbps / HBM_PEAK_GBPS, 4),
           "diff": diff, "timed_step_equals_checked_decode": last_equal,
           "kernels_avg_us": {k_: round(v_["avg_us"], 2) for k_, v_ in kern.items()},
           "roofline": roof, "cpu_baseline": cpu}
    case.sess.close()
    del case, ref, pre, out, launch
    torch.cuda.empty_cache()
    return res


def bench_mla_prefill(args, fp8=False):
    """The trainer-side recompute of one 32768-token absorbed-MLA sequence (128 heads,
    latent 512 + rope 64): every position's logprob from one prefill pass in 2048-token
    chunks, through the same split kernels decode runs (one query row per token).  Its last
    four positions are also produced by four plain decode steps on a second copy of the
    history (diff, must be 0).  Attention FLOPs count each (query, key) pair once per head:
    2 x (576 + 512) per pair."""
    import numpy as np
    import torch
    import invariant_rl_logprob_amd as ril
    import workloads as wl
    from invariant_rl_logprob_amd.metrics import mismatch
    from mla_case import MLACase

    L, CH, ND = 32768, 2048, 4
    w = wl.scaled(wl.MLA_DECODE_B128, rows=1, recompute_tokens=L)
    t0 = time.time()
    case = MLACase(w, [0], ctx=[L], device="cuda", shuffle_seed=0x5EED, copies=2, max_rows=128, max_tokens=CH,
                   kv_dtype=1 if fp8 else 0)
    d = case.data[0]
    log(f"mla prefill: data ready in {time.time() - t0:.1f}s")
    case.write_history("d", [0], ND)
    dec = torch.stack([case.decode_back("d", [0], b)[0] for b in range(ND, 0, -1)])

    def recompute():
        outs = []
        for p0 in range(0, L, CH):
            outs.append(case.sess.prefill([("p", 0)], [p0], targets=[d["target"][p0:p0 + CH]],
                                          qs=[d["q"][p0:p0 + CH]], ks=[d["c"][p0:p0 + CH]]))
        return torch.cat(outs)

    case.sess.ensure(("p", 0), L)
    lp = recompute()  # warm-up pass
    torch.cuda.synchronize()
    ril.ril_trace_enable(True)
    t1 = time.time()
    lp = recompute()
    torch.cuda.synchronize()
    secs = time.time() - t1
    kt = {}
    for kid, name in enumerate(ril.KERNEL_NAMES):
        tot, cnt = ril.ril_trace_read(kid)
        if cnt:
            kt[name] = round(tot, 3)
    ril.ril_trace_enable(False)
    diff = mismatch(dec, lp[L - ND:])
    attn_ms = kt.get("attn_split", float("nan"))
    flops = (L * (L + 1) // 2) * w.n_heads * 2 * ((w.kv_rank + w.rope_dim) + w.kv_rank)
    tflops = flops / (attn_ms * 1e-3) / 1e12
    log(f"mla prefill: {secs:.2f} s for {L} tokens, kernels {kt}, diff {diff}")
    res = {"value": round(L / secs, 1), "unit": "tokens/s", "ms_per_step": round(secs * 1e3, 3),
           "config": {"workload": f"mla_prefill_32k{'_fp8' if fp8 else ''}: the recompute of one {L}-token "
                                  "absorbed-MLA sequence, 128 heads, latent 512 + rope 64"
                                  + (" in an FP8 E4M3 cache" if fp8 else "") + f", chunks of {CH} tokens, "
                                  "o-proj 65536x4096, lm-head 4096x129280", "tokens": L, "chunk": CH},
           "kernel_ms": kt, "attn_split_tflops": round(tflops, 1),
           "attn_split_frac_of_bf16_peak": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
           "last_positions_vs_decode_steps": diff}
    case.sess.close()
    del case, d, lp, dec
    torch.cuda.empty_cache()
    return res


def bench_ssd(args):
    """Mamba-2 SSD mixer decode, 64 rows at contexts U[1024, 8192]: H = 128 heads of 64
    channels, 8 groups of 128 state rows, chunks of 128; the 8192 -> 4096 projection and
    the 4096 x 129280 lm-head.  History is laid down by prefill calls of 4096 tokens (timed:
    the trainer-side recompute rate of this mixer); the last 16 positions of every row are
    decoded step by step and recomputed by one prefill call (diff, must be 0); the decode
    step is timed like the other workloads.  The mixer-output kernel's algorithmic bytes
    per row: the fp32 state entering the chunk (H x 64 x 128 x 4 = 4 MiB) plus the chunk's
    earlier inputs (x, B, dt: 18.9 KB per position) and the row's own inputs."""
    import numpy as np
    import torch
    import invariant_rl_logprob_amd as ril
    import workloads as wl
    from invariant_rl_logprob_amd.metrics import mismatch
    from ssd_case import SSDCase

    w = wl.SSD_DECODE_B64
    rows = list(range(w.rows))
    t0 = time.time()
    case = SSDCase(w, rows, device="cuda", shuffle_seed=0x5EED, tags=2, max_rows=w.rows, max_tokens=4096)
    ctx = [case.ctx(r) for r in rows]
    log(f"ssd: data ready in {time.time() - t0:.1f}s; sum ctx = {sum(ctx)}")
    n = w.recompute_tokens
    torch.cuda.synchronize()
    ril.ril_trace_enable(True)
    t1 = time.time()
    case.history("d", rows, n)
    torch.cuda.synchronize()
    hist_s = time.time() - t1
    kt = {}
    for kid, name in enumerate(ril.KERNEL_NAMES):
        tot, cnt = ril.ril_trace_read(kid)
        if cnt:
            kt[name] = round(tot, 3)
    ril.ril_trace_enable(False)
    hist_tokens = sum(c_ - n for c_ in ctx)
    log(f"ssd: history {hist_tokens} tokens in {hist_s:.2f} s, kernel ms {kt}")
    dec = torch.stack([case.decode_back("d", rows, back) for back in range(n, 0, -1)], dim=1)
    case.history("p", rows, n)
    pre = case.prefill_last("p", rows, n)
    torch.cuda.synchronize()
    diff = mismatch(dec, pre)
    log(f"ssd: prefill vs decode over {diff['tokens']} tokens: {diff}")

    d = case.data
    pick = lambda key: torch.stack([d[r][key][case.ctx(r) - 1] for r in rows])  # noqa: E731
    launch, out = case.sess.prepare_decode([("d", r) for r in rows], ctx, targets=pick("target").to(torch.int32),
                                           q=pick("C"), k=pick("B"), v=pick("x"), dt=pick("dt"))
    ms_step, kern = timed_steps(launch, args.steps, args.warmup)
    last_equal = bool(np.array_equal(out.cpu().view(torch.int32).numpy(),
                                     dec[:, -1].cpu().view(torch.int32).numpy()))
    H, P, N, G, Q = w.n_heads, w.head_dim, w.d_state, w.n_groups, w.chunk
    per_pos = H * P * 2 + G * N * 2 + H * 4
    out_bytes = sum(H * P * N * 4 + ((c_ - 1) % Q) * per_pos + per_pos + G * N * 2 for c_ in ctx)
    out_us = kern["ssd_out"]["avg_us"]
    gbps = out_bytes / (out_us * 1e-6) / 1e9
    roof = roofline_hbm("ssd_out", gbps, out_bytes, out_us)

    cpu = None
    if not args.no_cpu and args.cpu_rows > 0:
        import oracle  # noqa: F401  (the cpu_baseline leg: case.oracle_row runs the fp64 recurrence)
        r0 = min(rows, key=lambda r: case.ctx(r))
        t2 = time.time()
        lp_o, _ = case.oracle_row(r0)
        secs = time.time() - t2
        cpu = {"value": round(1 / secs, 4), "unit": "tokens/s", "cores": blas_threads(), "kind": "oracle",
               **host_info(), "sample": f"decode row {r0} at context {case.ctx(r0)} (the recurrence over every "
                                        f"position, projection and lm-head in fp64), {secs:.1f} s",
               "max_abs_diff_vs_gpu": float(abs(lp_o - out.cpu().numpy()[rows.index(r0)]))}
        log(f"ssd oracle: {cpu}")
    res = {
        "value": round(len(rows) / (ms_step * 1e-3), 1), "ms_per_step": round(ms_step, 4),
        "config": {"workload": "ssd_decode_b64: 64 Mamba-2 mixer decode rows (128 heads x 64 channels, 8 groups "
                               "x 128 state rows, chunks of 128) at contexts U[1024,8192], o-proj 8192x4096, "
                               "lm-head 4096x129280", "rows": len(rows), "sum_ctx": sum(ctx), "chunk": Q},
        "history_prefill": {"tokens": hist_tokens, "seconds": round(hist_s, 3),
                            "tokens_per_s": round(hist_tokens / hist_s, 1), "kernel_ms": kt},
        "diff": diff, "timed_step_equals_checked_decode": last_equal,
        "kernels_avg_us": {k_: round(v_["avg_us"], 2) for k_, v_ in kern.items()},
        "roofline": roof, "cpu_baseline": cpu,
    }
    case.sess.close()
    return res


WORKLOADS = {"gqa_decode_b64": bench_gqa, "gqa_decode_b64_fp8": bench_gqa_fp8,
             "gqa_decode_b64_w8a8": bench_gqa_w8a8, "gqa_decode_b64_fp8_w8a8": bench_gqa_fp8_w8a8, "mla_decode_b128": bench_mla,
             "sparse_mla_b32": bench_sparse, "long_mix": bench_long,
             "mla_decode_b128_fp8": lambda a: bench_mla(a, fp8=True),
             "sparse_mla_b32_fp8": lambda a: bench_sparse(a, fp8=True),
             "mla_prefill_32k": bench_mla_prefill, "mla_prefill_32k_fp8": lambda a: bench_mla_prefill(a, fp8=True),
             "ssd_decode_b64": bench_ssd}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="gqa_decode_b64", choices=sorted(WORKLOADS))
    ap.add_argument("--cpu-rows", type=int, default=30, help="rows of the oracle timing sample")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle timing leg")
    ap.add_argument("--no-comparator", action="store_true", help="skip the shape-derived comparator leg")
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay leg")
    ap.add_argument("--no-lm-sweep", action="store_true", help="skip the lm-head M sweep (gqa workloads)")
    ap.add_argument("--no-long", action="store_true",
                    help="gqa_decode_b64: skip the long-context decode leg (256 rows at contexts to 131072)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (PMC byte-counter calibration)")
    ap.add_argument("--lm-head-rows", type=int, default=0,
                    help="only run the bf16 lm-head of the GQA workload on this many N(0,1) rows, one untimed "
                         "and three timed launches (kernel profiles at a chosen M)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "rows shard across GPUs by request with no exchange, but no multi-GPU run is made",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": 1 << 30, "launches": 3}))
        return

    if args.lm_head_rows > 0:
        print(json.dumps(lm_head_rows(args.lm_head_rows)), flush=True)
        return

    res = WORKLOADS[args.workload](args)
    if args.workload == "gqa_decode_b64" and not args.no_long:
        torch.cuda.empty_cache()
        res["long_mix_decode"] = long_decode_leg(args)
    line = {"metric": METRIC, "value": res.pop("value"), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": res.pop("ms_per_step"), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": res.pop("dtype", "bf16"), "data": "synthetic"}
    line.update(res)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
