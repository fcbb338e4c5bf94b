"""Determinism: each entry point run twice on the same inputs gives the same
bits (no atomics in any reduction; split-K and split-KV partial results are
summed in a fixed order), and the KV refresh leaves the same cache bytes.
Shapes take the split paths: a 96-row refresh splits K, a 96-row attention
over 8224 cache rows splits the keys, a 1024-row attention runs unsplit."""
import numpy as np
import pytest
import torch

from entropy_gated_kv_amd import lib as L
from synth import generators as G
from tests.gpu_helpers import dev, i32

pytestmark = pytest.mark.gpu


def twice(fn):
    a = fn()
    b = fn()
    torch.cuda.synchronize()
    return a, b


@pytest.mark.parametrize("n", [96, 300])
def test_refresh_is_deterministic(n):
    d, Hq, Hkv, dh, Lc = 3584, 28, 4, 128, 1024
    x = dev(G.random_matrix(70 + n, (1, n, d), (n, d), 1.0, "bf16"), "bf16")
    W = dev(G.random_matrix(71, (2, d), ((Hq + 2 * Hkv) * dh, d), 0.02, "bf16"), "bf16")
    rows = i32(np.sort(np.random.default_rng(n).choice(Lc, n, replace=False)))
    ws = torch.zeros(max(L.ec_kv_refresh_workspace_bytes(n, d, Hq, Hkv, dh, L.EC_BF16), 1),
                     dtype=torch.uint8, device="cuda")

    def run():
        K = torch.zeros((Hkv, Lc, dh), dtype=torch.bfloat16, device="cuda")
        Vt = torch.zeros((Hkv, dh, Lc), dtype=torch.bfloat16, device="cuda")
        q = torch.zeros((n, Hq, dh), dtype=torch.bfloat16, device="cuda")
        L.ec_kv_refresh(x, rows, i32([n]), W, Hq, Hkv, dh, q, K, Vt, ws)
        return q, K, Vt

    a, b = twice(run)
    for u, v in zip(a, b):
        assert torch.equal(u.view(torch.int16), v.view(torch.int16))


@pytest.mark.parametrize("n, Lq", [(96, 8224), (1024, 1024)])
def test_attention_is_deterministic(n, Lq):
    Hq, Hkv, dh = 28, 4, 128
    q = dev(G.random_matrix(80, (1, n), (n, Hq, dh), 1.0, "bf16"), "bf16")
    K = dev(G.random_matrix(81, (2, Lq), (Hkv, Lq, dh), 1.0, "bf16"), "bf16")
    Vt = dev(G.random_matrix(82, (3, Lq), (Hkv, dh, Lq), 1.0, "bf16"), "bf16")
    ws = torch.zeros(max(L.ec_attention_workspace_bytes(n, Lq, Hq, Hkv, dh), 1), dtype=torch.uint8,
                     device="cuda")

    def run():
        out = torch.zeros((n, Hq, dh), dtype=torch.bfloat16, device="cuda")
        L.ec_bidir_attention(q, i32([n]), K, Vt, Lq, out, ws)
        return out

    a, b = twice(run)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
