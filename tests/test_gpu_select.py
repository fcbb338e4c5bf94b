"""GPU parity of row selection (ec_select_rows) against the oracle: bit-exact."""
import numpy as np
import pytest
import torch

import oracle as O
from entropy_gated_kv_amd import lib as L
from synth import generators as G

pytestmark = pytest.mark.gpu


def gpu_select(full, masked, bs, bl, hist, k, cap, causal=False):
    Lq = len(masked)
    ring = np.full(cap, -1, dtype=np.int32)
    for i, p in enumerate(hist):
        ring[i % cap] = p
    t = lambda a, dt=torch.int32: torch.tensor(np.asarray(a), dtype=dt, device="cuda")  # noqa: E731
    rows = torch.full((Lq,), -1, dtype=torch.int32, device="cuda")
    n = torch.zeros(1, dtype=torch.int32, device="cuda")
    L.ec_select_rows(t([full]), t(masked, torch.uint8), bs, bl, t(ring), t([len(hist)]), k, rows, n,
                     block_causal=int(causal))
    torch.cuda.synchronize()
    return rows.cpu().numpy()[: int(n.item())]


@pytest.mark.parametrize("L_", [1, 31, 64, 1000, 8224, 32800])
def test_selection_matches_oracle(L_):
    for seed in range(6):
        bl = min(32, L_)
        bs = max(0, L_ - 2 * bl) if L_ > bl else 0
        masked = np.zeros(L_, dtype=np.uint8)
        masked[bs:] = G.random_mask(seed, L_, 0.5)[bs:]
        masked[min(L_, bs + bl):] = 1
        decoded = np.flatnonzero((masked == 0) & (np.arange(L_) >= bs))
        prefix = np.arange(0, bs)
        hist = list(G.random_history(seed, prefix, min(len(prefix), 70))) + \
            list(G.random_history(seed + 9, decoded, len(decoded)))
        for k in (0, 1, 16, 64):
            cap = max(k, 1) + seed * 7
            want = O.select_rows(0, masked, bs, bl, hist, k)
            got = gpu_select(0, masked, bs, bl, hist, k, cap)
            np.testing.assert_array_equal(got, want, err_msg=f"L={L_} seed={seed} k={k}")
        got = gpu_select(1, masked, bs, bl, hist, 16, 16)
        np.testing.assert_array_equal(got, np.arange(L_))


def test_history_ring_wraps():
    L_ = 300
    masked = np.zeros(L_, dtype=np.uint8)
    masked[280:] = 1
    hist = list(range(0, 200, 3))          # 67 decoded positions, ring of 20 keeps the last 20
    want = O.select_rows(0, masked, 272, 16, hist, 20)
    got = gpu_select(0, masked, 272, 16, hist, 20, 20)
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("L_", [40, 1000, 8224, 32800])
def test_block_causal_selection_matches_oracle(L_):
    """Block diffusion: full steps take the block, partial steps its masked
    positions and the history entries inside it; history entries before the
    block (earlier blocks) and past it are left out."""
    for seed in range(6):
        bl = 32
        bs = (L_ // 2) // bl * bl if L_ > 2 * bl else 0
        masked = np.zeros(L_, dtype=np.uint8)
        masked[bs:bs + bl] = G.random_mask(seed, L_, 0.5)[bs:bs + bl]
        masked[bs + bl:] = 1
        inside = np.flatnonzero(masked[bs:bs + bl] == 0) + bs
        before = np.arange(0, bs)
        hist = list(G.random_history(seed, before, min(len(before), 50))) + \
            list(G.random_history(seed + 3, inside, len(inside)))
        if bs + bl < L_:
            hist.insert(len(hist) // 2, bs + bl)        # a position past the block
        for k in (0, 1, 8, 64):
            cap = max(k, 1) + seed * 5
            want = O.select_rows(0, masked, bs, bl, hist, k, block_causal=True)
            got = gpu_select(0, masked, bs, bl, hist, k, cap, causal=True)
            np.testing.assert_array_equal(got, want, err_msg=f"L={L_} seed={seed} k={k}")
        got = gpu_select(1, masked, bs, bl, hist, 8, 16, causal=True)
        np.testing.assert_array_equal(got, np.arange(bs, bs + bl))


@pytest.mark.parametrize("L_", [1, 77, 1000, 32800])
def test_sliding_window_matches_oracle(L_):
    """block_start = -1: the block is the block_len positions from the first
    masked one (found on the device), clipped at L; nothing masked: no block."""
    for seed in range(5):
        masked = G.random_mask(seed, L_, 0.3).astype(np.uint8)
        if seed == 0:
            masked[:] = 0                              # nothing masked
        elif seed == 1:
            masked[:] = 0
            masked[-1] = 1                             # window clipped at L
        decoded = np.flatnonzero(masked == 0)
        hist = list(G.random_history(seed, decoded, min(len(decoded), 40)))
        for bl in (1, 32):
            bl = min(bl, L_)
            bs, bl_eff = O.sliding_window(masked, bl)
            want = O.select_rows(0, masked, bs, bl_eff, hist, 16)
            got = gpu_select(0, masked, -1, bl, hist, 16, 64)
            np.testing.assert_array_equal(got, want, err_msg=f"L={L_} seed={seed} bl={bl}")
