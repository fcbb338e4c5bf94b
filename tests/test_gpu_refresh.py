"""GPU parity of the selective KV refresh (ec_kv_refresh) against the oracle.

Q and the refreshed cache rows within 2e-3 (fp32) / 2e-2 (bf16) abs and rel;
cache rows not selected must be bitwise unchanged (sentinel-filled caches).
Row counts cover 1..4 row blocks of the skinny kernel (each row-bound
instance), the 128-row boundary, split-K over a non-power-of-two count,
the tiled kernel with a ragged last tile (in each of its tile
configurations), and the LLaDA- and Dream-shaped full sizes (every row of the
partial-step shapes; 64 rows of the 1024-row full step, all tile edges
among them).
"""
import numpy as np
import pytest
import torch

import oracle as O
from entropy_gated_kv_amd import lib as L
from synth import generators as G
from tests.gpu_helpers import assert_close, dev, host, i32

pytestmark = pytest.mark.gpu


def run_case(dtype, d, Hq, Hkv, dh, Lc, rows, seed, sample=None):
    n = len(rows)
    x = G.random_matrix(seed, (1, n, d), (n, d), 1.0, dtype)
    W = G.random_matrix(seed, (2, d), ((Hq + 2 * Hkv) * dh, d), 0.02, dtype)
    xd, Wd = dev(x, dtype), dev(W, dtype)
    sentinel = 7.0
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    K = torch.full((Hkv, Lc, dh), sentinel, dtype=td, device="cuda")
    Vt = torch.full((Hkv, dh, Lc), -sentinel, dtype=td, device="cuda")
    q = torch.zeros((n, Hq, dh), dtype=td, device="cuda")
    ws_n = L.ec_kv_refresh_workspace_bytes(n, d, Hq, Hkv, dh, L.EC_BF16 if dtype == "bf16" else L.EC_F32)
    ws = torch.zeros(max(ws_n, 1), dtype=torch.uint8, device="cuda")
    L.ec_kv_refresh(xd, i32(rows), i32([n]), Wd, Hq, Hkv, dh, q, K, Vt, ws)
    torch.cuda.synchronize()
    pick = np.arange(n) if sample is None else np.asarray(sample)
    Ko = np.zeros((Hkv, Lc, dh))
    Vo = np.zeros((Hkv, Lc, dh))
    qo = O.kv_refresh(x[pick].astype(np.float64), np.asarray(rows)[pick], W.astype(np.float64),
                      Ko, Vo, Hq, Hkv, dh, dtype)
    Kg, Vg = host(K), host(Vt).transpose(0, 2, 1)
    sel = np.asarray(rows)[pick]
    assert_close(host(q)[pick], qo, dtype, "Q")
    assert_close(Kg[:, sel], Ko[:, sel], dtype, "K cache")
    assert_close(Vg[:, sel], Vo[:, sel], dtype, "V cache")
    keep = np.setdiff1d(np.arange(Lc), rows)
    assert np.all(Kg[:, keep] == sentinel) and np.all(Vg[:, keep] == -sentinel), "unselected rows changed"


@pytest.mark.parametrize("n", [1, 96, 128, 129, 300])
def test_device_row_count_below_the_buffer_bound(n):
    """A 300-row activation buffer with the row count on the device: the
    small-row kernel runs up to 128 rows and the tiled one above, each
    launched with the buffer's bound; only the first n rows are refreshed and
    only their cache positions and Q rows change."""
    d, Hq, Hkv, dh, Lc, cap = 512, 8, 2, 128, 644, 300
    rows_all = np.sort(np.random.default_rng(n).choice(Lc, cap, replace=False))
    x = G.random_matrix(n, (1, cap, d), (cap, d), 1.0, "bf16")
    W = G.random_matrix(n, (2, d), ((Hq + 2 * Hkv) * dh, d), 0.02, "bf16")
    K = torch.full((Hkv, Lc, dh), 7.0, dtype=torch.bfloat16, device="cuda")
    Vt = torch.full((Hkv, dh, Lc), -7.0, dtype=torch.bfloat16, device="cuda")
    q = torch.full((cap, Hq, dh), 3.0, dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(max(L.ec_kv_refresh_workspace_bytes(cap, d, Hq, Hkv, dh, L.EC_BF16), 1),
                     dtype=torch.uint8, device="cuda")
    L.ec_kv_refresh(dev(x, "bf16"), i32(rows_all), i32([n]), dev(W, "bf16"), Hq, Hkv, dh, q, K, Vt, ws)
    torch.cuda.synchronize()
    rows = rows_all[:n]
    Ko, Vo = np.zeros((Hkv, Lc, dh)), np.zeros((Hkv, Lc, dh))
    qo = O.kv_refresh(x[:n].astype(np.float64), rows, W.astype(np.float64), Ko, Vo, Hq, Hkv, dh, "bf16")
    Kg, Vg, qg = host(K), host(Vt).transpose(0, 2, 1), host(q)
    assert_close(qg[:n], qo, "bf16", "Q")
    assert_close(Kg[:, rows], Ko[:, rows], "bf16", "K cache")
    assert_close(Vg[:, rows], Vo[:, rows], "bf16", "V cache")
    keep = np.setdiff1d(np.arange(Lc), rows)
    assert np.all(Kg[:, keep] == 7.0) and np.all(Vg[:, keep] == -7.0), "unselected rows changed"
    assert np.all(qg[n:] == 3.0), "Q rows past the count changed"


@pytest.mark.parametrize("n", [1, 20, 64, 256])
def test_tiny_fp32_shapes(n):
    rows = np.sort(np.random.default_rng(n).choice(256, n, replace=False))
    run_case("f32", 128, 4, 4, 32, 256, rows, seed=n)


@pytest.mark.parametrize("n", [1, 7, 33, 96, 128, 129, 300])
@pytest.mark.parametrize("dh", [64, 128])
def test_bf16_gqa_shapes(n, dh):
    Lc = 520
    rows = np.sort(np.random.default_rng(n + dh).choice(Lc, n, replace=False))
    run_case("bf16", 512, 8, 2, dh, Lc, rows, seed=n + dh)


@pytest.mark.parametrize("consecutive", [True, False], ids=["full", "scattered"])
@pytest.mark.parametrize("tile", ["0", "1", "2", "3", "4"])
def test_bf16_every_tile_config(tile, consecutive, monkeypatch):
    """Each tile configuration of the tiled kernel (forced), with a ragged
    last row tile and column tile; consecutive rows take the packed
    transposed-V stores."""
    monkeypatch.setenv("EC_GEMM_TILE", tile)
    Lc, n = 644, 600
    rows = np.arange(n) + 4 if consecutive else np.sort(np.random.default_rng(9).choice(Lc, n, replace=False))
    run_case("bf16", 512, 8, 2, 128, Lc, rows, seed=int(tile) + 40)


def tile_edge_sample(n, tile, count, seed):
    """Rows at both edges of every `tile`-row tile, the last row, and random
    rows up to `count`."""
    edges = sorted({r for t in range(0, n, tile) for r in (t, t + 1, min(n, t + tile) - 1)})
    rest = np.setdiff1d(np.arange(n), edges)
    extra = np.random.default_rng(seed).choice(rest, max(0, count - len(edges)), replace=False)
    return np.sort(np.concatenate([edges, extra]).astype(np.int64))


def test_llada_full_size_partial_every_row():
    """The LLaDA-shaped refresh of a partial step (96 scattered rows of 1024,
    d 4096, 32 x 128 heads): every row of Q, K and V against the oracle."""
    Lc, n = 1024, 96
    rows = np.sort(np.random.default_rng(3).choice(Lc, n, replace=False))
    run_case("bf16", 4096, 32, 32, 128, Lc, rows, seed=5)


def test_llada_full_size_full_step_sampled():
    """A full step (all 1024 rows, the tiled kernel): 64 rows checked, among
    them both edges of every 256-row tile."""
    Lc = n = 1024
    run_case("bf16", 4096, 32, 32, 128, Lc, np.arange(Lc), seed=5,
             sample=tile_edge_sample(n, 256, 64, 7))


@pytest.mark.parametrize("n", [40, 96])
def test_dream_shape_split_k_every_row(n):
    """Dream-shaped refresh (d = 3584, 28/4 heads of 128): 28 k-iterations
    split seven ways, with the four- and six-block row instances; every row."""
    Lc = 1024
    rows = np.sort(np.random.default_rng(11 + n).choice(Lc, n, replace=False))
    run_case("bf16", 3584, 28, 4, 128, Lc, rows, seed=60 + n)
