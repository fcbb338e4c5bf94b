"""GPU parity of bidirectional attention (ec_bidir_attention) against the oracle.

Output within 2e-3 (fp32) / 2e-2 (bf16) abs and rel.  Covers MHA and GQA,
row counts on both sides of the split-KV / unsplit boundary (128 rows), cache
lengths that are not multiples of the 64-row kv tile, L < L_cap, and the
Dream-shaped long context (L = 32800, 28/4 heads) at full size on sampled
(row, head) pairs computed one by one by the oracle.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
from entropy_gated_kv_amd import lib as L
from synth import generators as G
from tests.gpu_helpers import assert_close, dev, host, i32

pytestmark = pytest.mark.gpu


def run_attn(dtype, n, Hq, Hkv, dh, Lq, Lc, seed):
    q = G.random_matrix(seed, (3,), (n, Hq, dh), 1.0, dtype)
    K = G.random_matrix(seed, (4,), (Hkv, Lc, dh), 1.0, dtype)
    V = G.random_matrix(seed, (5,), (Hkv, Lc, dh), 1.0, dtype)
    qd, Kd = dev(q, dtype), dev(K, dtype)
    Vt = dev(np.ascontiguousarray(V.transpose(0, 2, 1)), dtype)
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    out = torch.zeros((n, Hq, dh), dtype=td, device="cuda")
    nb = L.ec_attention_workspace_bytes(n, Lq, Hq, Hkv, dh)
    ws = torch.zeros(max(nb, 1), dtype=torch.uint8, device="cuda")
    L.ec_bidir_attention(qd, i32([n]), Kd, Vt, Lq, out, ws)
    torch.cuda.synchronize()
    return q, K, V, host(out)


@pytest.mark.parametrize("n,Lq", [(1, 1), (5, 37), (64, 256), (256, 256)])
def test_fp32_mha_tiny(n, Lq):
    q, K, V, got = run_attn("f32", n, 4, 4, 32, Lq, 256, seed=n + Lq)
    want = O.bidir_attention(q.astype(np.float64), K[:, :Lq].astype(np.float64),
                             V[:, :Lq].astype(np.float64), 1 / math.sqrt(32))
    assert_close(got, want, "f32", "attention")


@pytest.mark.parametrize("n", [1, 3, 96, 128, 129, 200])
@pytest.mark.parametrize("Hq,Hkv,dh", [(8, 8, 128), (28, 4, 128), (6, 2, 64), (4, 1, 32)])
def test_bf16_shapes(n, Hq, Hkv, dh):
    Lq, Lc = 1000, 1032
    q, K, V, got = run_attn("bf16", n, Hq, Hkv, dh, Lq, Lc, seed=n * 7 + Hq)
    want = O.bidir_attention(q.astype(np.float64), K[:, :Lq].astype(np.float64),
                             V[:, :Lq].astype(np.float64), 1 / math.sqrt(dh))
    assert_close(got, want, "bf16", "attention")


def test_dream_long_context_sampled():
    n, Hq, Hkv, dh, Lq = 96, 28, 4, 128, 32800
    q, K, V, got = run_attn("bf16", n, Hq, Hkv, dh, Lq, Lq, seed=11)
    rng = np.random.default_rng(0)
    for r, h in zip(rng.integers(0, n, 12), rng.integers(0, Hq, 12)):
        g = h // (Hq // Hkv)
        want = O.bidir_attention(q[r:r + 1, h:h + 1].astype(np.float64),
                                 K[g:g + 1].astype(np.float64), V[g:g + 1].astype(np.float64),
                                 1 / math.sqrt(dh))
        assert_close(got[r, h], want[0, 0], "bf16", f"attention row {r} head {h}")


def test_dream_long_context_full_step_sampled():
    """Every row of the 32800-row cache as a query (the full-step launch, whose
    last packed-row tile is ragged), checked on sampled (row, head) pairs."""
    n, Hq, Hkv, dh, Lq = 32800, 28, 4, 128, 32800
    q, K, V, got = run_attn("bf16", n, Hq, Hkv, dh, Lq, Lq, seed=12)
    rng = np.random.default_rng(1)
    rows = list(rng.integers(0, n, 10)) + [0, n - 1, n - 2]
    heads = list(rng.integers(0, Hq, 10)) + [0, Hq - 1, 13]
    for r, h in zip(rows, heads):
        g = h // (Hq // Hkv)
        want = O.bidir_attention(q[r:r + 1, h:h + 1].astype(np.float64),
                                 K[g:g + 1].astype(np.float64), V[g:g + 1].astype(np.float64),
                                 1 / math.sqrt(dh))
        assert_close(got[r, h], want[0, 0], "bf16", f"attention row {r} head {h}")
