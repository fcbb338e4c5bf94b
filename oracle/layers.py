"""Projections, selective KV refresh, bidirectional attention, RMSNorm and the
SwiGLU FFN, in float64 (test infrastructure only).

EntropyCache (pt) §1 and (zh) §1: diffusion LMs use bidirectional attention, so
every position attends to every position (no causal mask).  (zh) §2.2: a
partial step recomputes K/V only for the selected rows and reads the rest from
the cache.  The pages give no layer internals; the readings used here: weights
stored [out, in] (y = x W^T), no biases, no rotary embedding, scale 1/sqrt(dh),
query head h reads KV head floor(h / (Hq / Hkv)), RMSNorm with eps 1e-5.
"""
from __future__ import annotations

import numpy as np

from .rounding import to_storage


def linear(x, W) -> np.ndarray:
    """y = x W^T with W stored [out_features, in_features]."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(W, dtype=np.float64).T


def kv_refresh(a, rows, w_qkv, K, V, n_q: int, n_kv: int, dh: int, dtype: str) -> np.ndarray:
    """Recompute Q/K/V for the selected rows and scatter K/V into the caches.

    a:     [n, d] layer input (after the pre-norm, if any) of the selected rows
    rows:  [n] cache positions of those rows
    w_qkv: [(Hq + 2 Hkv) * dh, d], output columns ordered Q heads, K heads, V heads
    K, V:  [Hkv, L, dh] caches, updated in place at `rows` only
    Returns Q [n, Hq, dh] in storage precision.
    """
    n = len(rows)
    y = linear(a, w_qkv)
    qc, kc = n_q * dh, (n_q + n_kv) * dh
    q = to_storage(y[:, :qc], dtype).reshape(n, n_q, dh)
    k = to_storage(y[:, qc:kc], dtype).reshape(n, n_kv, dh)
    v = to_storage(y[:, kc:], dtype).reshape(n, n_kv, dh)
    rows = np.asarray(rows, dtype=np.int64)
    K[:, rows, :] = k.transpose(1, 0, 2)
    V[:, rows, :] = v.transpose(1, 0, 2)
    return q


def bidir_attention(q, K, V, scale: float) -> np.ndarray:
    """O[r, h] = softmax(q[r, h] . K[g(h)]^T * scale) V[g(h)] over every cache row.

    q: [n, Hq, dh]; K, V: [Hkv, L, dh]; g(h) = h // (Hq // Hkv).  Returns float64.
    """
    q = np.asarray(q, dtype=np.float64)
    n, n_q, dh = q.shape
    n_kv = K.shape[0]
    group = n_q // n_kv
    out = np.empty((n, n_q, dh), dtype=np.float64)
    for h in range(n_q):
        g = h // group
        s = (q[:, h, :] @ K[g].T) * scale          # [n, L]
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ V[g]
    return out


def rmsnorm(x, gain, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * gain, per row."""
    x = np.asarray(x, dtype=np.float64)
    r = np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return x / r * np.asarray(gain, dtype=np.float64)


def swiglu(a, w_gate, w_up) -> np.ndarray:
    """silu(a W_gate^T) * (a W_up^T), silu(g) = g / (1 + exp(-g))."""
    g = linear(a, w_gate)
    u = linear(a, w_up)
    return g / (1.0 + np.exp(-g)) * u
