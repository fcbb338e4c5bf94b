"""KV drift of a full recompute: how far the reused Value vectors had moved
(test infrastructure only).

EntropyCache (zh) §2.1, first observation, and (pt) §2 ("entropy predicts the
cache drift"): the entropy of a newly decoded token correlates with the drift
of the KV cache, measured on the Value vectors as a cosine distance.  The pages
give no aggregation; the readings used here:
  * the Value vector of position p in one layer is the concatenation over the
    KV heads of V[g, p, :] (Hkv * dh values);
  * on a full step, every position's stale vector (the cache before the step)
    is compared with its recomputed one: d_p = 1 - cos(stale_p, fresh_p);
  * positions where either vector is all zero (never computed) are left out;
  * per layer the step reports the mean and the maximum of d_p over the
    positions kept (NaN for both when none is kept).
"""
from __future__ import annotations

import numpy as np


def cosine_distance(a, b) -> np.ndarray:
    """1 - cos between corresponding rows of a and b ([n, m]); NaN where either
    row is all zero."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    na = np.sqrt(np.sum(a * a, axis=1))
    nb = np.sqrt(np.sum(b * b, axis=1))
    ok = (na > 0) & (nb > 0)
    out = np.full(a.shape[0], np.nan)
    out[ok] = 1.0 - np.sum(a[ok] * b[ok], axis=1) / (na[ok] * nb[ok])
    return out


def value_drift(V_stale, V_fresh) -> np.ndarray:
    """(mean, max) over positions of 1 - cos(stale, fresh) for one layer's Value
    caches [Hkv, L, dh]; positions with a zero vector are left out."""
    Vs = np.asarray(V_stale, dtype=np.float64)
    Vf = np.asarray(V_fresh, dtype=np.float64)
    L = Vs.shape[1]
    a = Vs.transpose(1, 0, 2).reshape(L, -1)
    b = Vf.transpose(1, 0, 2).reshape(L, -1)
    d = cosine_distance(a, b)
    d = d[~np.isnan(d)]
    if d.size == 0:
        return np.array([np.nan, np.nan])
    return np.array([d.mean(), d.max()])
