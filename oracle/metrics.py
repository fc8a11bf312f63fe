"""Train-inference mismatch metrics (test infrastructure only).

diff and the k3 KL estimator as the Bitwise-consistent RL post defines them
(section 2: max, mean and standard deviation of the per-token difference over
valid tokens; section 3.2 figure: k3 = r - 1 - log r).
"""

from __future__ import annotations

import numpy as np


def diff_stats(lp_rollout, lp_train) -> dict:
    """max / mean / std of |lp_rollout - lp_train| and of |exp(lp_rollout) - exp(lp_train)|.

    The post writes the difference both on logprobs and on probabilities;
    both are reported and both are zero exactly when the bits agree.
    """
    a = np.asarray(lp_rollout, dtype=np.float64)
    b = np.asarray(lp_train, dtype=np.float64)
    d = np.abs(a - b)
    dp = np.abs(np.exp(a) - np.exp(b))
    return {
        "max": float(d.max(initial=0.0)), "mean": float(d.mean()) if d.size else 0.0,
        "std": float(d.std()) if d.size else 0.0,
        "p_max": float(dp.max(initial=0.0)), "p_mean": float(dp.mean()) if dp.size else 0.0,
        "p_std": float(dp.std()) if dp.size else 0.0,
    }


def k3_mean(lp_train, lp_rollout) -> float:
    """Mean k3 = r - 1 - log r over tokens, r = exp(lp_train - lp_rollout).

    The ratio direction is a reading (the post leaves r undefined): samples
    come from the rollout policy, so r = p_train / p_rollout.  Computed as
    expm1(delta) - delta to stay accurate for small delta.
    """
    delta = np.asarray(lp_train, dtype=np.float64) - np.asarray(lp_rollout, dtype=np.float64)
    return float(np.mean(np.expm1(delta) - delta)) if delta.size else 0.0
