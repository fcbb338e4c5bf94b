"""Pins for the oracle's KV refresh, attention, RMSNorm and SwiGLU.

KV refresh: brute-force triple loops on tiny shapes; identity weights give
K = X; unselected cache rows stay bitwise unchanged.  Attention: torch's
scaled_dot_product_attention in float64 (library routine, non-causal, GQA by
repeating KV heads), plus closed cases (L = 1 gives V; equal scores give the
mean of V; one dominant key gives its V row).  RMSNorm: torch.nn.functional.
rms_norm.  SwiGLU: torch.nn.functional.silu.
"""
import math

import numpy as np
import torch
import torch.nn.functional as F

from oracle.layers import bidir_attention, kv_refresh, linear, rmsnorm, swiglu


def test_kv_refresh_brute_force_loops():
    g = np.random.default_rng(0)
    n_q, n_kv, dh, d, L = 4, 2, 3, 5, 9
    a = g.standard_normal((3, d))
    W = g.standard_normal(((n_q + 2 * n_kv) * dh, d))
    rows = [1, 4, 8]
    K = g.standard_normal((n_kv, L, dh))
    V = g.standard_normal((n_kv, L, dh))
    K0, V0 = K.copy(), V.copy()
    q = kv_refresh(a, rows, W, K, V, n_q, n_kv, dh, "f64")
    for r, pos in enumerate(rows):
        for c in range(W.shape[0]):
            acc = 0.0
            for j in range(d):
                acc += a[r, j] * W[c, j]
            if c < n_q * dh:
                assert abs(q[r, c // dh, c % dh] - acc) < 1e-12
            elif c < (n_q + n_kv) * dh:
                cc = c - n_q * dh
                assert abs(K[cc // dh, pos, cc % dh] - acc) < 1e-12
            else:
                cc = c - (n_q + n_kv) * dh
                assert abs(V[cc // dh, pos, cc % dh] - acc) < 1e-12
    others = [p for p in range(L) if p not in rows]
    assert np.array_equal(K[:, others], K0[:, others]) and np.array_equal(V[:, others], V0[:, others])


def test_kv_refresh_identity_weights():
    n_kv, dh = 2, 4
    d = n_kv * dh
    W = np.concatenate([np.eye(d)] * 3)        # Hq = Hkv here: Q = K = V = a
    a = np.arange(2 * d, dtype=float).reshape(2, d)
    K = np.zeros((n_kv, 5, dh))
    V = np.zeros((n_kv, 5, dh))
    q = kv_refresh(a, [0, 3], W, K, V, n_kv, n_kv, dh, "f64")
    np.testing.assert_array_equal(q.reshape(2, d), a)
    np.testing.assert_array_equal(K[:, [0, 3]].transpose(1, 0, 2).reshape(2, d), a)
    np.testing.assert_array_equal(V[:, [0, 3]].transpose(1, 0, 2).reshape(2, d), a)


def _sdpa(q, K, V, scale):
    n_q, n_kv = q.shape[1], K.shape[0]
    qt = torch.from_numpy(q).permute(1, 0, 2)                       # [Hq, n, dh]
    kt = torch.from_numpy(K).repeat_interleave(n_q // n_kv, dim=0)  # [Hq, L, dh]
    vt = torch.from_numpy(V).repeat_interleave(n_q // n_kv, dim=0)
    o = F.scaled_dot_product_attention(qt, kt, vt, is_causal=False, scale=scale)
    return o.permute(1, 0, 2).numpy()


def test_attention_matches_torch_sdpa_mha_and_gqa():
    g = np.random.default_rng(1)
    for n_q, n_kv, n, L, dh in [(4, 4, 5, 17, 8), (28, 4, 3, 33, 16), (6, 2, 7, 64, 32), (3, 1, 1, 2, 4)]:
        q = g.standard_normal((n, n_q, dh))
        K = g.standard_normal((n_kv, L, dh))
        V = g.standard_normal((n_kv, L, dh))
        s = 1 / math.sqrt(dh)
        np.testing.assert_allclose(bidir_attention(q, K, V, s), _sdpa(q, K, V, s), rtol=1e-12, atol=1e-12)


def test_attention_closed_cases():
    g = np.random.default_rng(2)
    q = g.standard_normal((3, 2, 4))
    K = g.standard_normal((1, 1, 4))
    V = g.standard_normal((1, 1, 4))
    np.testing.assert_allclose(bidir_attention(q, K, V, 0.5), np.broadcast_to(V[0, 0], (3, 2, 4)))
    K = np.zeros((1, 9, 4))
    V = g.standard_normal((1, 9, 4))
    np.testing.assert_allclose(bidir_attention(q, K, V, 0.5), np.broadcast_to(V[0].mean(0), (3, 2, 4)),
                               atol=1e-15)
    K = np.zeros((1, 9, 4))
    K[0, 6] = 1000 * q[0, 0]                    # one key dominates for query (0, 0)
    out = bidir_attention(q[:1, :1], K, V, 1.0)
    np.testing.assert_allclose(out[0, 0], V[0, 6], atol=1e-12)


def test_rmsnorm_and_swiglu_match_torch():
    g = np.random.default_rng(3)
    x = g.standard_normal((5, 64)) * 3
    gain = g.standard_normal(64)
    want = F.rms_norm(torch.from_numpy(x), (64,), weight=torch.from_numpy(gain), eps=1e-5).numpy()
    np.testing.assert_allclose(rmsnorm(x, gain, 1e-5), want, rtol=1e-12, atol=1e-12)
    wg = g.standard_normal((32, 64))
    wu = g.standard_normal((32, 64))
    xt = torch.from_numpy(x)
    want = (F.silu(F.linear(xt, torch.from_numpy(wg))) * F.linear(xt, torch.from_numpy(wu))).numpy()
    np.testing.assert_allclose(swiglu(x, wg, wu), want, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(linear(x, wg), F.linear(xt, torch.from_numpy(wg)).numpy(), rtol=1e-13)
