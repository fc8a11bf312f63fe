"""Mamba-2 selective state-space mixer (SSD), one sequence at a time (test infrastructure
only).

Source: the Bitwise-consistent RL post, section 6 (Nemotron, a Mamba-2 / attention / MoE
hybrid: decode replays the prefill's chunked arithmetic instead of running its own
one-step recurrence) and the zero-mismatch-rl README's key-features table (Mamba-2,
decode replays the prefill chunk math).  The pages name the layer, not its equations;
the plainest reading is the standard Mamba-2 layer with one scalar decay per head:

  H heads of P channels; G groups of state rows (head h reads group h // (H / G)); per
  position t, with dt_t[h] > 0 given and A[h] < 0, D[h] model constants:

      a_t[h]  = exp(dt_t[h] * A[h])
      S_t[h]  = a_t[h] * S_{t-1}[h] + dt_t[h] * B_t[g] x_t[h]^T      (N x P, S_{-1} = 0)
      y_t[h]  = S_t[h]^T C_t[g] + D[h] * x_t[h]                      (P values)

  y is stored as bf16 (the contract's storage point for a mixer output, like the
  attention output).

The GPU evaluates this in fixed chunks of positions (the SSD chunked form, an exact
rewriting of the recurrence); this oracle is the recurrence itself in float64, one
position after the other, so it shares nothing with that evaluation.

Pinned by (tests/test_oracle_pins.py): the quadratic "masked attention" form
y = (L o C B^T)(dt x) + D x with L[t, s] = prod_{s < r <= t} a_r written out as explicit
matrices; the state written as an explicit sum over past positions (brute force on tiny
sizes); the closed forms of a single position and of an infinitely fast decay; the
cumulative form without decay; splitting a sequence and carrying the state; planted
mistakes (a dropped dt, a decay shifted by one position, B and C swapped, a dropped D).
"""

from __future__ import annotations

import numpy as np

from .numerics import bf16, widen


def ssd_scan(x, B, C, dt, A, D, state=None):
    """The recurrence over one sequence.

    x [T, H, P], B [T, G, N], C [T, G, N], dt [T, H] (positive), A [H] (negative), D [H];
    state: the [H, N, P] state before position 0 (zeros if None).
    Returns (y [T, H, P] float64 unrounded, the state after the last position)."""
    x, B, C = widen(x), widen(B), widen(C)
    dt, A, D = (np.asarray(v, dtype=np.float64) for v in (dt, A, D))
    T, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    grp = np.arange(H) // (H // G)
    S = np.zeros((H, N, P)) if state is None else np.array(state, dtype=np.float64)
    y = np.empty((T, H, P))
    for t in range(T):
        a = np.exp(dt[t] * A)                                   # [H]
        Bt, Ct = B[t][grp], C[t][grp]                           # [H, N]
        S = a[:, None, None] * S + (dt[t][:, None, None] * Bt[:, :, None]) * x[t][:, None, :]
        y[t] = np.einsum("hn,hnp->hp", Ct, S) + D[:, None] * x[t]
    return y, S


def ssd_outputs(x, B, C, dt, A, D) -> np.ndarray:
    """bf16 y [T, H, P] of one sequence from position 0."""
    return bf16(ssd_scan(x, B, C, dt, A, D)[0])
