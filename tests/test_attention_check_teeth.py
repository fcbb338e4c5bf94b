"""The long-context attention parity check can fail (CPU only).

tests/test_gpu_attention.py compares every output of the 96-row, 28/4-head
attention over 8224 and 32800 keys with the oracle, elementwise within 2e-2
absolute + 2e-2 relative.  Here the same seeded inputs are run through the
oracle and the same comparison is applied to outputs with a planted mistake:
* the whole output scaled by 0.5;
* the log-sum-exp merge of a kv-split computation that leaves out one split
  (every split in turn, for splits of 256, 448 and 1600 keys; the kernel's
  own split size lies among these for both lengths at 256 CUs);
* one split's partial output halved before the merge (every split in turn).
Each planted mistake must be rejected, while the exact merge of all splits
must pass.  Splitting the kv range into partitions whose partial softmax
statistics are merged by log-sum-exp is the split-KV scheme of the
Prefilling-dLLM page (attention-kernel section); the merged result equals the
plain softmax attention, which is what the exact merge checks.
"""
import math

import numpy as np
import pytest

import oracle as O
from synth import generators as G
from tests.gpu_helpers import TOL

N, HQ, HKV, DH = 96, 28, 4, 128


def rejects(got, want):
    tol = TOL["bf16"]
    return bool((np.abs(got - want) > tol + tol * np.abs(want)).any())


def inputs(Lq):
    # the same draws as run_attn() of the GPU test (seed 11 + L, q_std 3)
    seed = 11 + Lq
    q = G.random_matrix(seed, (3,), (N, HQ, DH), 3.0, "bf16").astype(np.float64)
    K = G.random_matrix(seed, (4,), (HKV, Lq, DH), 1.0, "bf16").astype(np.float64)
    V = G.random_matrix(seed, (5,), (HKV, Lq, DH), 1.0, "bf16").astype(np.float64)
    return q, K, V


def split_stats(q, K, V, per):
    """Per head: the unnormalised partial output and weight sum of each split
    of `per` keys, against a common reference maximum (exact in float64)."""
    n, Hq, dh = q.shape
    Lq = K.shape[1]
    G_ = Hq // K.shape[0]
    bounds = list(range(0, Lq, per)) + [Lq]
    S = len(bounds) - 1
    num = np.empty((S, n, Hq, dh))
    den = np.empty((S, n, Hq))
    for h in range(Hq):
        g = h // G_
        s = (q[:, h, :] @ K[g].T) / math.sqrt(dh)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        for j in range(S):
            a, b = bounds[j], bounds[j + 1]
            num[j, :, h] = p[:, a:b] @ V[g, a:b]
            den[j, :, h] = p[:, a:b].sum(axis=1)
    return num, den


@pytest.mark.parametrize("Lq", [8224, 32800])
def test_check_rejects_planted_attention_mistakes(Lq):
    q, K, V = inputs(Lq)
    want = O.bidir_attention(q, K, V, 1 / math.sqrt(DH))
    assert np.abs(want).mean() > 0.1
    assert rejects(0.5 * want, want)
    for per in (256, 448, 1600):
        num, den = split_stats(q, K, V, per)
        tot_n, tot_d = num.sum(axis=0), den.sum(axis=0)
        merged = tot_n / tot_d[..., None]
        assert not rejects(merged, want)                    # the exact merge passes
        for j in range(num.shape[0]):
            dropped = (tot_n - num[j]) / (tot_d - den[j])[..., None]
            assert rejects(dropped, want), (Lq, per, j, "dropped split")
            halved = (tot_n - 0.5 * num[j]) / tot_d[..., None]
            assert rejects(halved, want), (Lq, per, j, "halved split output")
