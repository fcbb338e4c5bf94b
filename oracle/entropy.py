"""Decoded-token entropy, the max over decoded tokens, the threshold decision and
the unmask choice (test infrastructure only).

EntropyCache (zh) §2.2: after each denoising step new tokens are decoded from
the logits; E_{t+1} is the largest softmax entropy -sum_j p_ij log p_ij over the
tokens i decoded at that step; E_{t+1} > tau makes the next step a full
forward, E_{t+1} <= tau a partial one.  EntropyCache (pt) §2 states the same
rule (strict ">" for the full pass).  Readings where the pages are silent:
  * log is the natural log (entropies and tau in nats);
  * p is the plain softmax of the stored logits over the whole vocabulary
    (temperature 1);
  * 0 log 0 = 0, so -inf logits contribute nothing;
  * a row holding NaN or +inf has undefined entropy (NaN), and a NaN maximum
    forces a full step;
  * an empty decoded set gives E = -inf (so a partial step);
  * the decode rule: each candidate decodes to its argmax (lowest vocabulary
    id among equal maxima), and the n candidates with the largest top-1
    probability are unmasked (ties to the lower position), ranked in float64.
"""
from __future__ import annotations

import math
from typing import Iterable, Sequence, Tuple

import numpy as np


def softmax_entropy(z) -> Tuple[float, int, float]:
    """(H in nats, argmax, top-1 probability) of one logit row, by definition.

    p = softmax(z) over all entries; H = -sum_j p_j log p_j; p1 = max_j p_j.
    """
    z = np.asarray(z, dtype=np.float64).ravel()
    nan = np.isnan(z)
    if nan.all():
        amax = 0
    else:
        amax = int(np.nanargmax(z))          # first index of the maximum, NaN never wins
    if nan.any() or np.isposinf(z).any() or np.isneginf(z).all():
        return math.nan, amax, math.nan
    p = np.exp(z - z.max())                  # softmax is shift invariant
    p /= p.sum()
    nz = p > 0.0
    H = float(-np.sum(p[nz] * np.log(p[nz])))
    return H, amax, float(p.max())


def row_stats(logits) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Per-row (H, argmax, p1) of a [rows, V] logit matrix."""
    logits = np.asarray(logits)
    n = logits.shape[0]
    H = np.empty(n, dtype=np.float64)
    A = np.empty(n, dtype=np.int64)
    P = np.empty(n, dtype=np.float64)
    for i in range(n):
        H[i], A[i], P[i] = softmax_entropy(logits[i])
    return H, A, P


def max_entropy(H, decoded: Iterable[int]) -> float:
    """E = max over the decoded rows of H (-inf if none; NaN if any is NaN)."""
    H = np.asarray(H, dtype=np.float64)
    idx = np.asarray(list(decoded), dtype=np.int64)
    if idx.size == 0:
        return -math.inf
    vals = H[idx]
    if np.isnan(vals).any():
        return math.nan
    return float(vals.max())


def decide(E: float, tau: float) -> int:
    """1 = next step recomputes every row (E > tau, or E is NaN); 0 = partial."""
    if math.isnan(E):
        return 1
    return 1 if E > tau else 0


def entropy_max(logits, decoded=None, tau: float = 0.0):
    """The standalone entropy pass: per-row stats, E over `decoded`, decision.

    decoded=None means every row counts as decoded.
    """
    H, A, P = row_stats(logits)
    D = range(H.shape[0]) if decoded is None else decoded
    E = max_entropy(H, D)
    return {"H": H, "argmax": A, "p1": P, "E": E, "flag": decide(E, tau)}


def choose(cand_positions: Sequence[int], p1: Sequence[float], n: int) -> np.ndarray:
    """Positions to unmask: the n candidates of largest p1, ties to the lower
    position, NaN p1 last; returned in ascending position order."""
    cand = [int(c) for c in cand_positions]
    p1 = [float(v) for v in p1]
    order = sorted(range(len(cand)),
                   key=lambda i: (math.isnan(p1[i]), -p1[i] if not math.isnan(p1[i]) else 0.0, cand[i]))
    take = [cand[i] for i in order[: max(0, min(n, len(cand)))]]
    return np.array(sorted(take), dtype=np.int64)
