"""Seeded synthetic inputs for the invariant-logprob path.

This module is the one place that both the GPU path's tests/bench and the
fp64 oracle draw their inputs from.  It holds none of the method's arithmetic:
it only draws random numbers, rounds them to the storage type, and describes the
workload shapes.

Every tensor is keyed by (workload seed, tensor kind, sequence id[, extra]),
never by a batch slot, so a sequence receives the same data in every batch it
is placed in (a requirement for the batch-invariance checks: the data generator
must not leak batch position into the values).

Random draws use ``torch.Generator`` seeded from a SplitMix64 hash of the key.
The draws are made on whichever device the caller asks for; CPU and GPU draws
differ (different engines), so a test generates once and copies the exact bf16
bits to the other side.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Dict, Sequence, Tuple

import torch

_MASK64 = (1 << 64) - 1


def _splitmix64(x: int) -> int:
    x = (x + 0x9E3779B97F4A7C15) & _MASK64
    z = x
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
    return z ^ (z >> 31)


def key(*parts) -> int:
    """Stable 63-bit key from ints and strings (order-sensitive)."""
    h = 0x1234_5678_9ABC_DEF0
    for p in parts:
        if isinstance(p, str):
            v = 0
            for ch in p.encode():
                v = ((v * 131) + ch) & _MASK64
        else:
            v = int(p) & _MASK64
        h = _splitmix64(h ^ v)
    return h & ((1 << 63) - 1)


def _gen(k: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(k)
    return g


def randn(shape, k: int, std: float = 1.0, device="cpu", dtype=torch.bfloat16) -> torch.Tensor:
    """N(0, std^2) draws rounded (RNE) to ``dtype``; keyed by ``k``."""
    x = torch.randn(tuple(shape), generator=_gen(k, device), device=device, dtype=torch.float32)
    if std != 1.0:
        x = x * std
    return x.to(dtype)


def randint(lo: int, hi_inclusive: int, shape, k: int, device="cpu") -> torch.Tensor:
    """Uniform integers in [lo, hi_inclusive] (int32); keyed by ``k``."""
    return torch.randint(lo, hi_inclusive + 1, tuple(shape), generator=_gen(k, device),
                         device=device, dtype=torch.int64).to(torch.int32)


# --------------------------------------------------------------------------
# Workload shapes.  Names say what the workload is; sizes are the workloads'.
# --------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class TinyDecoder:
    """One pre-norm decoder layer + final RMSNorm + lm-head, token input."""
    d_model: int = 256
    n_q_heads: int = 4
    n_kv_heads: int = 4
    head_dim: int = 64
    vocab: int = 2048
    lengths: Tuple[int, ...] = (33, 64, 97, 128)
    prompt_tokens: int = 16
    init_std: float = 0.02
    rms_eps: float = 1e-6
    page_tokens: int = 16
    seed: int = 0
    d_ff: int = 0                 # > 0: a SwiGLU MLP block (gate/up F each) after the attention block


@dataclasses.dataclass(frozen=True)
class GQADecode:
    """Paged GQA decode rows with q/K/V given, attention output -> RMSNorm -> lm-head."""
    rows: int = 64
    n_q_heads: int = 32
    n_kv_heads: int = 8
    head_dim: int = 128
    ctx_lo: int = 512
    ctx_hi: int = 8192
    vocab: int = 129280
    d_head: int = 4096
    o_proj_out: int = 0          # 0: no output projection before the final norm
    init_std: float = 0.02
    rms_eps: float = 1e-6
    page_tokens: int = 16
    recompute_tokens: int = 64   # q is drawn for the last this-many positions of each row
    seed: int = 1


TINY = TinyDecoder()
TINY_MLP = TinyDecoder(d_ff=512, seed=5)
GQA_DECODE_B64 = GQADecode()
# Long-context GQA (64 q / 8 kv heads) with an 8192 -> 4096 output projection.
GQA_LONG = GQADecode(rows=256, n_q_heads=64, n_kv_heads=8, head_dim=128, ctx_lo=1024,
                     ctx_hi=131072, vocab=129280, d_head=4096, o_proj_out=4096, seed=4)


# --------------------------------------------------------------------------
# Tiny decoder inputs
# --------------------------------------------------------------------------

def tiny_weights(w: TinyDecoder = TINY, device="cpu") -> Dict[str, torch.Tensor]:
    """bf16 weights in nn.Linear layout ([out, in]); RMSNorm gains are 1."""
    d, hq, hkv, hd, v = w.d_model, w.n_q_heads, w.n_kv_heads, w.head_dim, w.vocab
    s = w.seed
    return {
        "embed": randn((v, d), key(s, "embed"), w.init_std, device),
        "w_qkv": randn(((hq + 2 * hkv) * hd, d), key(s, "w_qkv"), w.init_std, device),
        "w_o": randn((d, hq * hd), key(s, "w_o"), w.init_std, device),
        "norm_attn": torch.ones(d, dtype=torch.bfloat16, device=device),
        "norm_final": torch.ones(d, dtype=torch.bfloat16, device=device),
        "w_lm": randn((v, d), key(s, "w_lm"), w.init_std, device),
        **({"w_gate_up": randn((2 * w.d_ff, d), key(s, "w_gate_up"), w.init_std, device),
            "w_down": randn((d, w.d_ff), key(s, "w_down"), w.init_std, device),
            "norm_mlp": torch.ones(d, dtype=torch.bfloat16, device=device)} if w.d_ff else {}),
    }


def tiny_tokens(seq_id: int, w: TinyDecoder = TINY, device="cpu") -> torch.Tensor:
    """Token ids of sequence ``seq_id`` (length ``w.lengths[seq_id]``), uniform in [0, vocab)."""
    n = w.lengths[seq_id]
    return randint(0, w.vocab - 1, (n,), key(w.seed, "tokens", seq_id), device)


# --------------------------------------------------------------------------
# GQA decode rows
# --------------------------------------------------------------------------

def gqa_ctx(row: int, w: GQADecode = GQA_DECODE_B64) -> int:
    """Context length of row ``row`` (including the token being decoded)."""
    return int(randint(w.ctx_lo, w.ctx_hi, (1,), key(w.seed, "ctx", row))[0])


def gqa_head_weights(w: GQADecode = GQA_DECODE_B64, device="cpu") -> Dict[str, torch.Tensor]:
    out = {"w_lm": randn((w.vocab, w.d_head), key(w.seed, "w_lm"), w.init_std, device)}
    if w.o_proj_out:
        out["w_o"] = randn((w.o_proj_out, w.n_q_heads * w.head_dim), key(w.seed, "w_o"),
                           w.init_std, device)
    return out


def gqa_row(row: int, w: GQADecode = GQA_DECODE_B64, device="cpu", ctx: int = None):
    """Data of one row: K, V for every position, q and targets for the last positions.

    Returns dict(ctx, k [ctx, Hkv, D], v [ctx, Hkv, D], q [R, Hq, D], target [R]) where
    q[j] and target[j] belong to position ctx - R + j (R = recompute_tokens, clipped to ctx).
    """
    L = gqa_ctx(row, w) if ctx is None else int(ctx)
    R = min(w.recompute_tokens, L)
    s = w.seed
    return {
        "ctx": L,
        "k": randn((L, w.n_kv_heads, w.head_dim), key(s, "k", row, L), 1.0, device),
        "v": randn((L, w.n_kv_heads, w.head_dim), key(s, "v", row, L), 1.0, device),
        "q": randn((R, w.n_q_heads, w.head_dim), key(s, "q", row, L), 1.0, device),
        "target": randint(0, w.vocab - 1, (R,), key(s, "target", row, L), device),
    }


@dataclasses.dataclass(frozen=True)
class LongMix:
    """Chunked prefill of long sequences mixed with decode rows (GQA_LONG's model):
    n_seqs sequences of seq_len tokens prefilled in chunks of each size in ``chunks``,
    interleaved with the decode rows of ``decode`` (contexts in [ctx_lo, ctx_hi]), each of
    which decodes its last ``decode_tokens`` positions during the prefill."""
    n_seqs: int = 8
    seq_len: int = 131072
    chunks: Tuple[int, ...] = (512, 2048, 8192)
    decode_tokens: int = 16
    decode: GQADecode = GQA_LONG
    seed: int = 4


LONG_MIX = LongMix()


def long_seq(seq: int, w: LongMix = LONG_MIX, device="cpu", length: int = None):
    """One long sequence: k, v [L, Hkv, D], q [L, Hq, D] and target [L] for every position."""
    m = w.decode
    L = w.seq_len if length is None else int(length)
    s = w.seed
    return {
        "len": L,
        "k": randn((L, m.n_kv_heads, m.head_dim), key(s, "long-k", seq, L), 1.0, device),
        "v": randn((L, m.n_kv_heads, m.head_dim), key(s, "long-v", seq, L), 1.0, device),
        "q": randn((L, m.n_q_heads, m.head_dim), key(s, "long-q", seq, L), 1.0, device),
        "target": randint(0, m.vocab - 1, (L,), key(s, "long-target", seq, L), device),
    }


def mix_schedule(w: LongMix, chunk: int, mix: int, rows: Sequence[int], seq_len: int = None):
    """A seeded batch mix: for each prefill step (one chunk of every long sequence), the
    decode rows that advance one position in it, and the order of the step's segments.
    Returns (steps_of_row {row: sorted step list of length decode_tokens}, order_seed)."""
    L = w.seq_len if seq_len is None else int(seq_len)
    n_steps = -(-L // chunk)
    assert n_steps >= w.decode_tokens, "every decode position needs a step of its own"
    g = _gen(key(w.seed, "mix", chunk, mix), "cpu")
    steps = {}
    for r in rows:
        pick = torch.randperm(n_steps, generator=g)[: w.decode_tokens]
        steps[r] = sorted(int(x) for x in pick)
    return steps, key(w.seed, "order", chunk, mix)


@dataclasses.dataclass(frozen=True)
class MLADecode:
    """Absorbed-MLA decode rows: q [H, 576] per position, one shared latent row
    [576] = 512 latent + 64 rope dims per cached token; softmax scale 1/sqrt(192)."""
    rows: int = 128
    n_heads: int = 128
    kv_rank: int = 512
    rope_dim: int = 64
    scale_dim: int = 192
    ctx_lo: int = 4096
    ctx_hi: int = 32768
    vocab: int = 129280
    d_head: int = 4096           # width after the absorbed value/output projection
    init_std: float = 0.02
    rms_eps: float = 1e-6
    page_tokens: int = 16
    recompute_tokens: int = 16
    seed: int = 2


MLA_DECODE_B128 = MLADecode()


def mla_ctx(row: int, w: MLADecode = MLA_DECODE_B128) -> int:
    return int(randint(w.ctx_lo, w.ctx_hi, (1,), key(w.seed, "ctx", row))[0])


def mla_head_weights(w: MLADecode = MLA_DECODE_B128, device="cpu") -> Dict[str, torch.Tensor]:
    """Absorbed value-up + output projection [d_head, H*512] and the lm-head [V, d_head]."""
    return {
        "w_o": randn((w.d_head, w.n_heads * w.kv_rank), key(w.seed, "w_vo"), w.init_std, device),
        "w_lm": randn((w.vocab, w.d_head), key(w.seed, "w_lm"), w.init_std, device),
    }


def mla_row(row: int, w: MLADecode = MLA_DECODE_B128, device="cpu", ctx: int = None):
    """Latent rows c [ctx, 576] of every position; q [R, H, 576] and targets [R] of the
    last R = recompute_tokens positions (q[j] belongs to position ctx - R + j)."""
    L = mla_ctx(row, w) if ctx is None else int(ctx)
    R = min(w.recompute_tokens, L)
    s = w.seed
    dq = w.kv_rank + w.rope_dim
    return {
        "ctx": L,
        "c": randn((L, dq), key(s, "c", row, L), 1.0, device),
        "q": randn((R, w.n_heads, dq), key(s, "q", row, L), 1.0, device),
        "target": randint(0, w.vocab - 1, (R,), key(s, "target", row, L), device),
    }


@dataclasses.dataclass(frozen=True)
class SparseMLADecode:
    """MLA decode over the top-k positions an indexer selects: per position an fp32
    indexer key [128] beside the bf16 latent row; per query an fp32 indexer query
    [64, 128].  tie_stress > 0 copies the indexer key of one position into that many
    other positions so exact score ties occur at known places."""
    rows: int = 32
    n_heads: int = 128
    kv_rank: int = 512
    rope_dim: int = 64
    scale_dim: int = 192
    index_heads: int = 64
    index_dim: int = 128
    topk: int = 2048
    ctx_lo: int = 65536
    ctx_hi: int = 65536
    vocab: int = 129280
    d_head: int = 4096
    init_std: float = 0.02
    rms_eps: float = 1e-6
    page_tokens: int = 16
    recompute_tokens: int = 16
    tie_stress: int = 0
    seed: int = 3


SPARSE_MLA_B32 = SparseMLADecode()


def sparse_row(row: int, w: SparseMLADecode = SPARSE_MLA_B32, device="cpu", ctx: int = None):
    """As mla_row, plus k_index [ctx, 128] fp32 and q_index [R, 64, 128] fp32."""
    L = int(randint(w.ctx_lo, w.ctx_hi, (1,), key(w.seed, "ctx", row))[0]) if ctx is None else int(ctx)
    R = min(w.recompute_tokens, L)
    s = w.seed
    dq = w.kv_rank + w.rope_dim
    k_index = randn((L, w.index_dim), key(s, "k_index", row, L), 1.0, device, dtype=torch.float32)
    if w.tie_stress:
        # one large key copied into tie_stress positions: those positions score exactly
        # alike and (being 8x larger) at the top, so the tie rule decides the selection
        big = randn((w.index_dim,), key(s, "tie_key", row, L), 8.0, device, dtype=torch.float32)
        dst = randint(0, L - 1, (w.tie_stress,), key(s, "tie_dst", row, L)).to(torch.int64).to(device)
        k_index[dst] = big
    return {
        "ctx": L,
        "c": randn((L, dq), key(s, "c", row, L), 1.0, device),
        "q": randn((R, w.n_heads, dq), key(s, "q", row, L), 1.0, device),
        "k_index": k_index,
        "q_index": randn((R, w.index_heads, w.index_dim), key(s, "q_index", row, L), 1.0, device,
                         dtype=torch.float32),
        "target": randint(0, w.vocab - 1, (R,), key(s, "target", row, L), device),
    }


def randu(shape, k: int, lo: float, hi: float, device="cpu") -> torch.Tensor:
    """Uniform fp32 draws in [lo, hi); keyed by ``k``."""
    return torch.rand(tuple(shape), generator=_gen(k, device), device=device, dtype=torch.float32) * (hi - lo) + lo


@dataclasses.dataclass(frozen=True)
class SSDDecode:
    """Mamba-2 mixer decode rows (the Nemotron family's SSD layer): H heads of 64
    channels, G groups of 128 state rows, chunks of 128 positions; per position x [H, 64],
    B and C [G, 128] (bf16, N(0, 1)) and dt [H] (fp32, log-uniform in [0.001, 0.1], the
    Mamba time-step range); per head A = -exp(U[0, ln 16]) and D = 1 + 0.1 N(0, 1) (fp32);
    the mixer output (H x 64 = 8192 wide) goes through an 8192 -> 4096 projection and the
    4096 x 129280 lm-head."""
    rows: int = 64
    n_heads: int = 128
    head_dim: int = 64
    n_groups: int = 8
    d_state: int = 128
    chunk: int = 128
    ctx_lo: int = 1024
    ctx_hi: int = 8192
    vocab: int = 129280
    d_head: int = 4096
    init_std: float = 0.02
    rms_eps: float = 1e-6
    recompute_tokens: int = 16
    seed: int = 6


SSD_DECODE_B64 = SSDDecode()


def ssd_ctx(row: int, w: SSDDecode = SSD_DECODE_B64) -> int:
    return int(randint(w.ctx_lo, w.ctx_hi, (1,), key(w.seed, "ctx", row))[0])


def ssd_params(w: SSDDecode = SSD_DECODE_B64, device="cpu") -> Dict[str, torch.Tensor]:
    """Per-head A (negative) and D, fp32, and the head: the projection [d_head, H*64] and
    the lm-head [V, d_head]."""
    H = w.n_heads
    return {
        "A": -torch.exp(randu((H,), key(w.seed, "A"), 0.0, math.log(16.0), device)),
        "D": 1.0 + 0.1 * randn((H,), key(w.seed, "D"), 1.0, device, torch.float32),
        "w_o": randn((w.d_head, H * w.head_dim), key(w.seed, "w_o"), w.init_std, device),
        "w_lm": randn((w.vocab, w.d_head), key(w.seed, "w_lm"), w.init_std, device),
    }


def ssd_row(row: int, w: SSDDecode = SSD_DECODE_B64, device="cpu", ctx: int = None):
    """Every position's inputs of one sequence of ctx positions: x [L, H, 64], B and C
    [L, G, 128], dt [L, H] fp32 and the sampled ids [L] whose logprobs are asked for."""
    L = ssd_ctx(row, w) if ctx is None else int(ctx)
    s = w.seed
    return {
        "ctx": L,
        "x": randn((L, w.n_heads, w.head_dim), key(s, "x", row, L), 1.0, device),
        "B": randn((L, w.n_groups, w.d_state), key(s, "B", row, L), 1.0, device),
        "C": randn((L, w.n_groups, w.d_state), key(s, "C", row, L), 1.0, device),
        "dt": torch.exp(randu((L, w.n_heads), key(s, "dt", row, L), math.log(1e-3), math.log(1e-1), device)),
        "target": randint(0, w.vocab - 1, (L,), key(s, "target", row, L), device),
    }


def scaled(w, **changes):
    """A smaller variant of a workload for oracle-sized parity runs."""
    return dataclasses.replace(w, **changes)

