"""Pins for the oracle's row selection: hand-worked cases and invariants.

EntropyCache (zh) §2.2 / (pt) §2: full step -> every row; partial step -> the
current masked tokens plus the k most recently decoded tokens.
"""
import numpy as np

from oracle.selection import candidates, select_rows
from synth.generators import random_history, random_mask


def test_full_step_selects_every_row():
    np.testing.assert_array_equal(select_rows(1, np.ones(9), 3, 3, [1, 2], 5), np.arange(9))


def test_hand_worked_partial_cases():
    L = 12
    masked = np.zeros(L, dtype=np.uint8)
    masked[[5, 7, 8, 9, 10, 11]] = 1          # block [4, 8) holds 5 and 7; 8.. are later blocks
    hist = [6, 4]                            # 6 decoded first, then 4
    np.testing.assert_array_equal(candidates(masked, 4, 4), [5, 7])
    np.testing.assert_array_equal(select_rows(0, masked, 4, 4, hist, 0), [5, 7])
    np.testing.assert_array_equal(select_rows(0, masked, 4, 4, hist, 1), [4, 5, 7])
    np.testing.assert_array_equal(select_rows(0, masked, 4, 4, hist, 2), [4, 5, 6, 7])
    np.testing.assert_array_equal(select_rows(0, masked, 4, 4, hist, 50), [4, 5, 6, 7])
    # history from an earlier block, decoded in order 1, 3, 2
    np.testing.assert_array_equal(select_rows(0, masked, 4, 4, [1, 3, 2, 6, 4], 4), [2, 3, 4, 5, 6, 7])


def test_invariants_on_random_states():
    for seed in range(40):
        L = 64
        bs, bl = 32, 16
        masked = np.zeros(L, dtype=np.uint8)
        masked[bs:] = random_mask(seed, L, 0.6)[bs:]
        masked[bs + bl:] = 1
        decoded = [p for p in range(bs, bs + bl) if not masked[p]]
        hist = list(random_history(seed, np.arange(0, bs), 10)) + list(random_history(seed + 1, decoded, len(decoded)))
        for k in (0, 1, 5, 64):
            rows = select_rows(0, masked, bs, bl, hist, k)
            m = int(masked[bs:bs + bl].sum())
            assert len(rows) == m + min(k, len(hist))          # masked and history are disjoint
            assert np.all(np.diff(rows) > 0)                   # ascending, no duplicates
            assert set(candidates(masked, bs, bl)) <= set(rows)
            assert not (set(rows) & set(range(bs + bl, L)))    # later blocks come from the cache


def test_sliding_window_hand_worked():
    from oracle.selection import sliding_window
    masked = np.array([0, 0, 1, 0, 1, 1, 0, 1], dtype=np.uint8)
    assert sliding_window(masked, 3) == (2, 3)                 # window [2, 5): candidates 2, 4
    np.testing.assert_array_equal(candidates(masked, *sliding_window(masked, 3)), [2, 4])
    assert sliding_window(masked, 10) == (2, 6)               # clipped at L
    assert sliding_window(np.zeros(5), 4) == (5, 0)           # nothing masked: empty block
    masked[2] = 0                                             # the leftmost is decoded: the window moves
    assert sliding_window(masked, 3) == (4, 3)
    np.testing.assert_array_equal(candidates(masked, *sliding_window(masked, 3)), [4, 5])


def test_sliding_window_step_moves_with_the_leftmost_masked_position():
    import oracle as O
    from synth import configs as C
    from synth import generators as G
    cfg = C.scaled(C.TINY, name="slide", prompt_len=40, gen_len=24, block_len=24, k=4)
    w = G.model_weights(cfg)
    model = O.Model.from_arrays(cfg.model, "f32", w)
    toks, masked = G.initial_sequence(cfg)
    st = O.init_state(model, toks, masked)
    for i in range(6):
        first = int(np.flatnonzero(st.masked)[0])
        tr = O.step(model, st, 2.0, cfg.k, -1, 8, 2)
        assert tr.cand.min() == first and tr.cand.max() < first + 8, (i, first, tr.cand)
        assert set(tr.chosen) <= set(tr.cand.tolist())
