"""fp64 CPU oracle for the invariant sampled-token logprob forward.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call, link
or execute anything in this package.  Its only callers are ``tests/``,
``__graft_entry__.smoke()`` (to check one small GPU invocation) and the
``cpu_baseline`` leg of ``bench.py`` (to time it beside the GPU).  It shares no
code, constants or helpers with the HIP library and imports nothing from it.

What it computes is the plain definition, per sequence *alone* (which is
itself the batch-invariance reference): plain NumPy in float64; bf16 rounding
(round-to-nearest-even, straight from float64) only where the numerical
contract stores a bf16 value; everything else float64.  The one exception is
the indexer's float32 scores, which decide an integer selection and so take the
kernel's float32 roundings: plain C loops over C99 ``fmaf`` (``indexer.c``,
built and loaded by ``cbuild.py`` with the host compiler).

Sources (cited by page title and section):
  * "vLLM Achieves Bitwise-Consistent RL Training: Eliminating Numerical Drift
    to Zero KL Divergence on DeepSeek-V4-Flash at 91% Throughput" -- called
    "Bitwise-consistent RL post" below;
  * "zero-mismatch-rl" GitHub README -- called "zero-mismatch-rl README".

Parity status per function is given in each docstring ("pinned by ..." names
the independent checks in ``tests/test_oracle_pins.py``).
"""

from .numerics import (  # noqa: F401
    bf16,
    widen,
    rmsnorm,
    log_softmax_at,
    lm_head_logprob,
    attention_row,
    projection,
    silu,
    swiglu_rounded_once,
)
from .models import (  # noqa: F401
    tiny_decoder_prefill,
    tiny_decoder_decode,
    gqa_row_attention,
    gqa_row_logprob,
    head_logprob,
    mla_row_attention,
    indexer_scores,
    indexer_scores_fp32,
    sparse_mla_row_attention,
    topk_select,
)
from .metrics import diff_stats, k3_mean  # noqa: F401
from .ssd import ssd_scan, ssd_outputs  # noqa: F401
from .fp8 import e4m3_decode, e4m3_encode, kv_fp8_roundtrip  # noqa: F401
from .fp8block import (  # noqa: F401
    block_exponent,
    quantize_rows,
    quantize_weight_blocks,
    w8a8_matmul,
    lm_head_logprob_w8a8,
)
