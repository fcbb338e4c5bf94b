"""Row selection for the next forward pass (test infrastructure only).

EntropyCache (zh) §2.2 and EntropyCache (pt) §2: a full step recomputes every
position; a partial step recomputes only the tokens that are still masked plus
the k most recently decoded tokens (kept in a decode history of O(k) memory,
zh §2.3), and every other position reads its K/V from the cache.

Readings where the pages are silent:
  * "still masked" means the masked positions of the current block; masked
    positions of later blocks keep the K/V of the last full step;
  * the history holds decoded positions only (never prompt positions), in the
    order they were unmasked; within one step they are appended in ascending
    position order, so "last k" cuts at that order;
  * the history persists across blocks and across full steps.
"""
from __future__ import annotations

from typing import Sequence, Tuple

import numpy as np


def sliding_window(masked, width: int) -> Tuple[int, int]:
    """Sliding-window decoding: the current block is the `width` positions from
    the first masked position, clipped at L; (L, 0) when nothing is masked.

    EntropyCache (pt) §5 and (zh) §5 name sliding-window decoding among the
    strategies the method applies to; the pages define no window, so this is
    the plainest one: it starts at the leftmost position still to decode and
    moves as that position is decoded."""
    masked = np.asarray(masked).astype(bool)
    L = len(masked)
    idx = np.flatnonzero(masked)
    start = int(idx[0]) if idx.size else L
    return start, min(width, L - start)


def candidates(masked, block_start: int, block_len: int) -> np.ndarray:
    """Masked positions of the current block, ascending (the rows that get logits)."""
    masked = np.asarray(masked).astype(bool)
    return np.array([p for p in range(block_start, block_start + block_len) if masked[p]],
                    dtype=np.int64)


def select_rows(full: int, masked, block_start: int, block_len: int,
                history: Sequence[int], k: int, block_causal: bool = False) -> np.ndarray:
    """Ascending list of the positions whose Q/K/V are recomputed this step.

    block_causal (block diffusion, see oracle.step.step): only positions of
    the current block are ever recomputed.  A full step takes all of them; a
    partial step takes the block's masked positions and those of the last k
    decoded positions that lie inside the block (earlier blocks are final)."""
    L = len(masked)
    end = block_start + block_len
    if full:
        if block_causal:
            return np.arange(block_start, end, dtype=np.int64)
        return np.arange(L, dtype=np.int64)
    chosen = set(int(p) for p in candidates(masked, block_start, block_len))
    if k > 0:
        recent = [int(p) for p in list(history)[-k:]]
        if block_causal:
            recent = [p for p in recent if block_start <= p < end]
        chosen |= set(recent)
    return np.array(sorted(chosen), dtype=np.int64)
