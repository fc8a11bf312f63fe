"""S13: train-inference mismatch of two logprob tensors, on the host in fp64.

diff (Bitwise-consistent RL post, section 2): max, mean and standard deviation of the
per-token |lp_rollout - lp_train| over the compared (valid) tokens, reported on
logprobs and on probabilities; k3 (section 3.2 figure) = r - 1 - log r with
r = p_train / p_rollout, averaged.  Acceptance is exact equality: every value 0 and the
bit patterns identical.
"""

from __future__ import annotations

import numpy as np


def mismatch(lp_rollout, lp_train) -> dict:
    """Inputs: equal-shape fp32 tensors/arrays (torch tensors are moved to the host)."""
    def host(x):
        try:
            import torch
            if isinstance(x, torch.Tensor):
                return x.detach().to("cpu").contiguous().numpy()
        except ImportError:  # pragma: no cover
            pass
        return np.asarray(x)

    a32, b32 = host(lp_rollout), host(lp_train)
    bitwise = bool(a32.shape == b32.shape and np.array_equal(a32.view(np.int32), b32.view(np.int32)))
    a = a32.astype(np.float64).ravel()
    b = b32.astype(np.float64).ravel()
    d = np.abs(a - b)
    dp = np.abs(np.exp(a) - np.exp(b))
    delta = b - a
    k3 = np.expm1(delta) - delta
    n = d.size
    return {
        "tokens": int(n), "bitwise_equal": bitwise,
        "max": float(d.max()) if n else 0.0, "mean": float(d.mean()) if n else 0.0,
        "std": float(d.std()) if n else 0.0,
        "p_max": float(dp.max()) if n else 0.0,
        "k3": float(k3.mean()) if n else 0.0,
    }
