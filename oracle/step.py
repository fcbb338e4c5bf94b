"""One EntropyCache denoising step and the generation loop (test infrastructure only).

EntropyCache (zh) §2.2 describes each step as three phases:
  1. forward pass, full or partial according to the previous step's flag; a
     partial pass recomputes only the current masked tokens and the k most
     recently decoded tokens and reads every other position from the KV cache;
  2. decode new tokens from the logits and take E_{t+1}, the largest entropy
     among the newly decoded tokens;
  3. decide: E_{t+1} > tau makes the next step full, otherwise partial, with
     the recompute set drawn from the decode history.
EntropyCache (pt) §2 gives the same flow.  Readings where the pages are silent
(each also stated at the function that applies it):
  * the first step is full (there is no cache yet);
  * the decision made at step t governs step t+1;
  * on a partial step every layer recomputes only the selected rows (Q/K/V,
    attention, output projection, FFN) and attends over its whole cache;
  * layer input = token embedding + additive position embedding; the MASK token
    has its own embedding row;
  * logits are produced only for the masked positions of the current block,
    optionally times a per-position scale, and stored in the storage dtype;
  * when the block has no masked position left the host moves to the next
    block (the schedule is fixed on the host).

Block diffusion (block_causal=True).  The Chinese page (§5, generality) names
block diffusion as a place where the entropy signal could drive the recompute
of a sub-block, and describes no further.  The reading taken: the sequence is
split into blocks of block_len (the prompt included); attention is
block-causal, a position attending to every position of its own and earlier
blocks; the blocks before the current one are final, their K/V computed once
by a commit pass when the block is finished.  The entropy gate then decides,
inside the current block, between recomputing all of its rows (full step) and
only its masked rows plus the last k decoded positions that lie in it
(partial step), every recomputed row attending to the keys before the block's
end.  A commit is a full step that decodes nothing (commit below).
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence, Tuple

import numpy as np

from .drift import value_drift
from .entropy import choose, decide, max_entropy, row_stats
from .layers import bidir_attention, kv_refresh, linear, rmsnorm, swiglu
from .rounding import to_storage
from .selection import candidates, select_rows, sliding_window


@dataclasses.dataclass
class Model:
    n_layers: int
    d: int
    n_q: int
    n_kv: int
    dh: int
    V: int
    d_ffn: int
    eps: float
    dtype: str
    tok_emb: np.ndarray                  # [V + 1, d] float32 (storage-exact); row V is MASK
    pos_emb: np.ndarray                  # [L, d]
    layers: List[dict]
    w_lm: Optional[np.ndarray]           # [V, d], or None (the caller decodes)
    norm_final: Optional[np.ndarray] = None
    logit_scale: Optional[np.ndarray] = None   # [L] or None

    @classmethod
    def from_arrays(cls, shape, dtype: str, w: dict) -> "Model":
        f = lambda a: None if a is None else np.asarray(a, dtype=np.float64)  # noqa: E731
        # The token table (up to ~150k x 4k) stays in float32, which holds every
        # storage value exactly; gathered rows are widened to float64.
        return cls(n_layers=shape.n_layers, d=shape.d, n_q=shape.n_q_heads, n_kv=shape.n_kv_heads,
                   dh=shape.head_dim, V=shape.vocab, d_ffn=shape.d_ffn, eps=shape.rms_eps,
                   dtype=dtype, tok_emb=np.asarray(w["tok_emb"], dtype=np.float32),
                   pos_emb=f(w["pos_emb"]),
                   layers=[{k: f(v) for k, v in lw.items()} for lw in w["layers"]],
                   w_lm=f(w.get("w_lm")), norm_final=f(w.get("norm_final")),
                   logit_scale=f(w.get("logit_scale")))


@dataclasses.dataclass
class State:
    tokens: np.ndarray                   # [L] int64
    masked: np.ndarray                   # [L] bool
    history: List[int]                   # decoded positions in unmask order
    flag: int                            # 1: this step recomputes every row
    K: List[np.ndarray]                  # per layer [Hkv, L, dh]
    V: List[np.ndarray]

    def copy(self) -> "State":
        return State(self.tokens.copy(), self.masked.copy(), list(self.history), self.flag,
                     [k.copy() for k in self.K], [v.copy() for v in self.V])


@dataclasses.dataclass
class StepTrace:
    flag_used: int
    rows: np.ndarray
    cand: np.ndarray
    logits: Optional[np.ndarray]
    H: np.ndarray
    argmax: np.ndarray
    p1: np.ndarray
    chosen: np.ndarray
    E: float
    flag_next: int
    x_cand: Optional[np.ndarray] = None   # final activations of the candidate rows
    drift: Optional[np.ndarray] = None    # full steps: per layer (mean, max) Value drift


def init_state(model: Model, tokens, masked) -> State:
    """Fresh sequence state: empty history, empty caches, first step full."""
    L = len(tokens)
    K = [np.zeros((model.n_kv, L, model.dh)) for _ in range(model.n_layers)]
    V = [np.zeros((model.n_kv, L, model.dh)) for _ in range(model.n_layers)]
    return State(np.asarray(tokens, dtype=np.int64).copy(), np.asarray(masked).astype(bool).copy(),
                 [], 1, K, V)


def forward_rows(model: Model, state: State, rows: np.ndarray,
                 drift: Optional[list] = None, attn: Optional[list] = None,
                 n_keys: Optional[int] = None) -> np.ndarray:
    """Run every layer over the selected rows, refreshing their K/V in each cache.

    Returns the final activations of those rows (after the final norm, if any).
    When `drift` is a list, each layer's (mean, max) Value drift between the
    cache before and after its refresh is appended to it (oracle.drift).
    When `attn` is a list, each layer's attention output of the selected rows
    ([n, Hq, dh], storage precision) is appended to it.
    n_keys: the rows attend to cache positions [0, n_keys) only (block
    diffusion: the end of the current block); None: every position.
    """
    dt = model.dtype
    n = len(rows)
    x = to_storage(model.tok_emb[state.tokens[rows]].astype(np.float64) + model.pos_emb[rows], dt)
    scale = 1.0 / math.sqrt(model.dh)
    for l, lw in enumerate(model.layers):
        a = to_storage(rmsnorm(x, lw["norm_attn"], model.eps), dt) if model.d_ffn else x
        stale = state.V[l].copy() if drift is not None else None
        q = kv_refresh(a, rows, lw["w_qkv"], state.K[l], state.V[l], model.n_q, model.n_kv,
                       model.dh, dt)
        if drift is not None:
            drift.append(value_drift(stale, state.V[l]))
        nk = state.K[l].shape[1] if n_keys is None else n_keys
        o = to_storage(bidir_attention(q, state.K[l][:, :nk], state.V[l][:, :nk], scale), dt)
        if attn is not None:
            attn.append(o)
        x = to_storage(x + linear(o.reshape(n, model.n_q * model.dh), lw["w_o"]), dt)
        if model.d_ffn:
            a2 = to_storage(rmsnorm(x, lw["norm_ffn"], model.eps), dt)
            h = to_storage(swiglu(a2, lw["w_gate"], lw["w_up"]), dt)
            x = to_storage(x + linear(h, lw["w_down"]), dt)
    if model.d_ffn:
        x = to_storage(rmsnorm(x, model.norm_final, model.eps), dt)
    return x


def step(model: Model, state: State, tau: float, k: int, block_start: int, block_len: int,
         n_unmask: int, keep_logits: bool = True, drift: bool = False,
         block_causal: bool = False) -> StepTrace:
    """One denoising step; mutates `state` and returns what the step computed.

    drift: on a full step, also report each layer's Value drift (oracle.drift).
    block_start < 0: sliding-window decoding, the block being the block_len
    positions from the first masked one (oracle.selection.sliding_window).
    block_causal: block diffusion (module docstring): rows of the current
    block only, attending to the keys before the block's end."""
    if block_start < 0:
        if block_causal:
            raise ValueError("block diffusion needs an explicit block")
        block_start, block_len = sliding_window(state.masked, block_len)
    flag_used = state.flag
    rows = select_rows(flag_used, state.masked, block_start, block_len, state.history, k,
                       block_causal)
    dl = [] if (drift and flag_used) else None
    x = forward_rows(model, state, rows, dl,
                     n_keys=(block_start + block_len) if block_causal else None)
    cand = candidates(state.masked, block_start, block_len)
    ci = np.searchsorted(rows, cand)
    z = linear(x[ci], model.w_lm)
    if model.logit_scale is not None:
        z = z * model.logit_scale[cand][:, None]
    z = to_storage(z, model.dtype)
    H, A, P = row_stats(z)
    # The unmask choice ranks candidates by their float64 top-1 probability.
    chosen = choose(cand, P, n_unmask)
    pick = np.searchsorted(cand, chosen)
    state.tokens[chosen] = A[pick]
    state.masked[chosen] = False
    state.history.extend(int(c) for c in chosen)
    E = max_entropy(H, pick)
    state.flag = decide(E, tau)
    return StepTrace(flag_used, rows, cand, z if keep_logits else None, H, A, P, chosen, E,
                     state.flag, x[ci] if keep_logits else None,
                     None if dl is None else np.array(dl))


def step_external(model: Model, state: State, tau: float, k: int, block_start: int,
                  block_len: int, decoded_logits) -> StepTrace:
    """A step whose decoding happens outside the layer stack.

    The forward pass is the same as in `step` (selected rows, caches refreshed);
    the caller supplies the logits of the rows it decoded this step, and the
    decision is taken from them alone: E = the largest entropy among those rows
    (EntropyCache (zh) §2.2), the next step is full iff E > tau.  Tokens, mask
    and history are left to the caller; the steady-state long-context step is
    this case (its decoded rows are synthetic).
    """
    if block_start < 0:
        block_start, block_len = sliding_window(state.masked, block_len)
    flag_used = state.flag
    rows = select_rows(flag_used, state.masked, block_start, block_len, state.history, k)
    forward_rows(model, state, rows)
    z = np.asarray(decoded_logits, dtype=np.float64)
    H, A, P = row_stats(z)
    E = max_entropy(H, range(z.shape[0]))
    state.flag = decide(E, tau)
    cand = candidates(state.masked, block_start, block_len)
    return StepTrace(flag_used, rows, cand, z, H, A, P, np.zeros(0, dtype=np.int64), E, state.flag)


def generate(model: Model, state: State, schedule: Sequence[Tuple[int, int, int]], tau: float,
             k: int, keep_logits: bool = False, n_steps: Optional[int] = None) -> List[StepTrace]:
    """Run the schedule [(block_start, block_len, n_unmask), ...] from `state`."""
    out = []
    for i, (bs, bl, n) in enumerate(schedule):
        if n_steps is not None and i >= n_steps:
            break
        out.append(step(model, state, tau, k, bs, bl, n, keep_logits))
    return out


def commit(model: Model, state: State, block_start: int, block_len: int, k: int) -> StepTrace:
    """Block diffusion: make a finished block's K/V final.

    A full step over the block's rows (keys before its end) that decodes
    nothing: with no decoded row E = -inf, so the flag it leaves is 0."""
    state.flag = 1
    return step(model, state, 0.0, k, block_start, block_len, 0, block_causal=True)


def generate_block_diffusion(model: Model, state: State, prompt_len: int,
                             schedule: Sequence[Tuple[int, int, int]], tau: float, k: int,
                             keep_logits: bool = False) -> List[StepTrace]:
    """Block diffusion with the entropy gate inside the current block.

    The prompt is committed block by block (blocks of the schedule's length),
    then each generated block runs its denoising steps (block_causal) and is
    committed once its last token is decoded."""
    out = []
    bl0 = schedule[0][1]
    for bs in range(0, prompt_len, bl0):
        out.append(commit(model, state, bs, min(bl0, prompt_len - bs), k))
    for i, (bs, bl, n) in enumerate(schedule):
        out.append(step(model, state, tau, k, bs, bl, n, keep_logits, block_causal=True))
        if i + 1 == len(schedule) or schedule[i + 1][0] != bs:
            out.append(commit(model, state, bs, bl, k))
    return out
