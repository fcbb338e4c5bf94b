"""Seeded synthetic inputs shared by the oracle's tests and the GPU path.

Only data lives here: random weights, embeddings, prompts, per-position logit
scales and synthetic logit rows.  None of the method's arithmetic (softmax,
entropy, selection, projections, attention) is in this module.

Every draw is Philox keyed by a SeedSequence (config seed, stream, tensor,
chunk), so any block of rows of any tensor can be regenerated on its own and
large tensors are drawn in parallel without changing the values.  Values are
drawn in float32; for bfloat16 workloads they are then rounded to the nearest
bfloat16 (ties to even), so every array returned here holds values exactly
representable in the workload's storage dtype.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os
from typing import Dict, Iterable, List, Optional, Tuple

import numpy as np

from .configs import BF16, F32, EntropyOnlyConfig, LongContextConfig, ModelShape, StepConfig

# Streams of the per-config SeedSequence, in a fixed order.
S_WEIGHTS, S_TOK_EMB, S_POS_EMB, S_PROMPT, S_LOGIT_SCALE, S_LOGITS = range(6)

# Tensor ids inside the weight stream.
T_QKV, T_O, T_GATE, T_UP, T_DOWN, T_LM = range(6)

CHUNK_ELEMS = 1 << 22          # elements per independently seeded chunk
WEIGHT_STD = 0.02
EMB_STD = 1.0


def _rng(seed: int, key: Tuple[int, ...]) -> np.random.Generator:
    ss = np.random.SeedSequence(entropy=seed, spawn_key=key)
    return np.random.Generator(np.random.Philox(ss))


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """float32 array -> float32 array of the nearest bfloat16 values (ties to even).

    Used only to put generated data into the storage format; inputs are finite.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).copy()             # finite inputs: the sums below stay < 2^32
    t = u >> 16
    t &= 1
    t += 0x7FFF
    u += t
    u &= np.uint32(0xFFFF0000)
    return u.view(np.float32).reshape(a.shape)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """The bfloat16 bit patterns (uint16) of a float32 array of bf16-exact values."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("array holds values that are not bfloat16-exact")
    return (u >> 16).astype(np.uint16).reshape(a.shape)


def _store(a: np.ndarray, dtype: str) -> np.ndarray:
    return round_to_bf16(a) if dtype == BF16 else np.asarray(a, dtype=np.float32)


def _chunked_rows(rows: int, cols: int) -> int:
    return max(1, CHUNK_ELEMS // max(1, cols))


def normal_matrix(seed: int, key: Tuple[int, ...], rows: int, cols: int, std: float,
                  dtype: str, row_lo: int = 0, row_hi: Optional[int] = None) -> np.ndarray:
    """Rows [row_lo, row_hi) of a rows x cols N(0, std^2) matrix, in storage precision."""
    row_hi = rows if row_hi is None else row_hi
    assert 0 <= row_lo <= row_hi <= rows
    out = np.empty((row_hi - row_lo, cols), dtype=np.float32)
    cr = _chunked_rows(rows, cols)
    chunks = list(range(row_lo // cr, (row_hi + cr - 1) // cr)) if row_hi > row_lo else []

    def work(c: int) -> None:
        r0, r1 = c * cr, min(rows, (c + 1) * cr)
        g = _rng(seed, key + (c,))
        blk = g.standard_normal((r1 - r0, cols), dtype=np.float32)
        blk *= np.float32(std)
        lo, hi = max(r0, row_lo), min(r1, row_hi)
        out[lo - row_lo:hi - row_lo] = _store(blk[lo - r0:hi - r0], dtype)

    if len(chunks) > 1:
        with _cf.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, chunks))
    else:
        for c in chunks:
            work(c)
    return out


# -- model weights and sequence inputs ----------------------------------------

def weight_shape(m: ModelShape, name: str) -> Tuple[int, int]:
    """Weights are stored [out_features, in_features] (y = x W^T)."""
    return {
        "w_qkv": (m.qkv_out, m.d),
        "w_o": (m.d, m.n_q_heads * m.head_dim),
        "w_gate": (m.d_ffn, m.d),
        "w_up": (m.d_ffn, m.d),
        "w_down": (m.d, m.d_ffn),
        "w_lm": (m.vocab, m.d),
    }[name]


_TID = {"w_qkv": T_QKV, "w_o": T_O, "w_gate": T_GATE, "w_up": T_UP, "w_down": T_DOWN, "w_lm": T_LM}


def layer_weight(cfg, layer: int, name: str, row_lo: int = 0, row_hi: Optional[int] = None) -> np.ndarray:
    m = cfg.model
    r, c = weight_shape(m, name)
    lid = 0 if name == "w_lm" else layer
    return normal_matrix(cfg.seed, (S_WEIGHTS, lid, _TID[name]), r, c, WEIGHT_STD, cfg.dtype, row_lo, row_hi)


def tok_emb(cfg, row_lo: int = 0, row_hi: Optional[int] = None) -> np.ndarray:
    """[vocab + 1, d]; the last row is the MASK embedding."""
    m = cfg.model
    return normal_matrix(cfg.seed, (S_TOK_EMB,), m.vocab + 1, m.d, EMB_STD, cfg.dtype, row_lo, row_hi)


def pos_emb(cfg, L: Optional[int] = None) -> np.ndarray:
    """[L, d] additive position table."""
    L = cfg.L if L is None else L
    return normal_matrix(cfg.seed, (S_POS_EMB,), L, cfg.model.d, EMB_STD, cfg.dtype)


def norm_gain(cfg) -> np.ndarray:
    """RMSNorm gains are initialised to one (exact in every storage dtype)."""
    return np.ones(cfg.model.d, dtype=np.float32)


def prompt_tokens(cfg, n: Optional[int] = None) -> np.ndarray:
    n = cfg.prompt_len if n is None else n
    g = _rng(cfg.seed, (S_PROMPT,))
    return g.integers(0, cfg.model.vocab, size=n, dtype=np.int64).astype(np.int32)


def logit_scale(cfg, L: Optional[int] = None) -> Optional[np.ndarray]:
    """Per-position LM-head scale s_p ~ LogUniform(lo, hi) in float32, or None."""
    rng_lohi = getattr(cfg, "logit_scale", None)
    if rng_lohi is None:
        return None
    L = cfg.L if L is None else L
    lo, hi = rng_lohi
    g = _rng(cfg.seed, (S_LOGIT_SCALE,))
    u = g.random(L, dtype=np.float64)
    return np.exp(np.log(lo) + u * (np.log(hi) - np.log(lo))).astype(np.float32)


def initial_sequence(cfg) -> Tuple[np.ndarray, np.ndarray]:
    """(tokens [L] int32, masked [L] uint8): prompt tokens, then MASK positions."""
    toks = np.full(cfg.L, cfg.model.mask_id, dtype=np.int32)
    toks[: cfg.prompt_len] = prompt_tokens(cfg)
    masked = np.zeros(cfg.L, dtype=np.uint8)
    masked[cfg.prompt_len:] = 1
    return toks, masked


def model_weights(cfg, layers: Optional[Iterable[int]] = None,
                  tok_table: Optional[np.ndarray] = None) -> Dict[str, object]:
    """All weights of a model as float32 arrays of storage-exact values.

    `tok_table`: an already generated tok_emb(cfg) to reuse (it depends only on
    the seed, vocabulary and width)."""
    m = cfg.model
    layers = range(m.n_layers) if layers is None else layers
    if tok_table is not None and tok_table.shape != (m.vocab + 1, m.d):
        raise ValueError("tok_table has the wrong shape")
    out: Dict[str, object] = {
        "tok_emb": tok_emb(cfg) if tok_table is None else tok_table,
        "pos_emb": pos_emb(cfg),
        "w_lm": layer_weight(cfg, 0, "w_lm") if getattr(cfg, "lm_head", True) else None,
        "logit_scale": logit_scale(cfg),
        "layers": [],
    }
    if m.d_ffn:
        out["norm_final"] = norm_gain(cfg)
    for l in layers:
        lw = {"w_qkv": layer_weight(cfg, l, "w_qkv"), "w_o": layer_weight(cfg, l, "w_o")}
        if m.d_ffn:
            lw.update(
                norm_attn=norm_gain(cfg), norm_ffn=norm_gain(cfg),
                w_gate=layer_weight(cfg, l, "w_gate"), w_up=layer_weight(cfg, l, "w_up"),
                w_down=layer_weight(cfg, l, "w_down"))
        out["layers"].append(lw)
    return out


def model_weights_streamed(cfg, tok_table: Optional[np.ndarray] = None) -> Dict[str, object]:
    """model_weights(cfg) with "layers" as a generator: each layer's arrays are
    drawn only when the consumer asks for them, so a large stack can be
    uploaded layer by layer (values identical to model_weights)."""
    m = cfg.model

    def layers():
        for l in range(m.n_layers):
            lw = {"w_qkv": layer_weight(cfg, l, "w_qkv"), "w_o": layer_weight(cfg, l, "w_o")}
            if m.d_ffn:
                lw.update(
                    norm_attn=norm_gain(cfg), norm_ffn=norm_gain(cfg),
                    w_gate=layer_weight(cfg, l, "w_gate"), w_up=layer_weight(cfg, l, "w_up"),
                    w_down=layer_weight(cfg, l, "w_down"))
            yield lw

    out: Dict[str, object] = {
        "tok_emb": tok_emb(cfg) if tok_table is None else tok_table,
        "pos_emb": pos_emb(cfg),
        "w_lm": layer_weight(cfg, 0, "w_lm") if getattr(cfg, "lm_head", True) else None,
        "logit_scale": logit_scale(cfg),
        "layers": layers(),
    }
    if m.d_ffn:
        out["norm_final"] = norm_gain(cfg)
    return out


# -- synthetic logits (entropy-only workload and long-context decision rows) ---

def entropy_row_scales(cfg: EntropyOnlyConfig) -> np.ndarray:
    g = _rng(cfg.seed, (S_LOGIT_SCALE,))
    lo, hi = cfg.scale_range
    u = g.random(cfg.rows, dtype=np.float64)
    return np.exp(np.log(lo) + u * (np.log(hi) - np.log(lo))).astype(np.float32)


def entropy_boosts(cfg: EntropyOnlyConfig) -> Dict[int, int]:
    """row -> boosted column, for the first n_boosted rows of a seeded permutation."""
    g = _rng(cfg.seed, (S_LOGITS, 1))
    rows = g.permutation(cfg.rows)[: cfg.n_boosted]
    cols = g.integers(0, cfg.vocab, size=cfg.n_boosted)
    return {int(r): int(c) for r, c in zip(rows, cols)}


def entropy_logits(cfg: EntropyOnlyConfig, row_lo: int = 0, row_hi: Optional[int] = None) -> np.ndarray:
    """Rows [row_lo, row_hi) of the [rows, vocab] synthetic logit matrix.

    Row i is s_i * N(0, 1) with s_i ~ LogUniform(scale_range); a seeded tenth
    of the rows get +boost at one seeded column (near one-hot rows).
    """
    row_hi = cfg.rows if row_hi is None else row_hi
    V = cfg.vocab
    scales = entropy_row_scales(cfg)
    boosts = entropy_boosts(cfg)
    out = np.empty((row_hi - row_lo, V), dtype=np.float32)
    per = max(1, CHUNK_ELEMS // V)
    chunks = list(range(row_lo // per, (row_hi + per - 1) // per)) if row_hi > row_lo else []

    def work(c: int) -> None:
        r0, r1 = c * per, min(cfg.rows, (c + 1) * per)
        g = _rng(cfg.seed, (S_LOGITS, 0, c))
        blk = g.standard_normal((r1 - r0, V), dtype=np.float32)
        blk *= scales[r0:r1, None]
        for r in range(r0, r1):
            if r in boosts:
                blk[r - r0, boosts[r]] += np.float32(cfg.boost)
        lo, hi = max(r0, row_lo), min(r1, row_hi)
        out[lo - row_lo:hi - row_lo] = _store(blk[lo - r0:hi - r0], cfg.dtype)

    if len(chunks) > 1:
        with _cf.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, chunks))
    else:
        for c in chunks:
            work(c)
    return out


def decision_logits(cfg: LongContextConfig, step: int) -> np.ndarray:
    """[decision_rows, vocab] synthetic decoded-token logits for one steady-state step.

    Every `full_every`-th step uses the small scale (flat rows, high entropy);
    the other steps use the large scale (peaked rows, low entropy).
    """
    s_full, s_other = cfg.decision_scales
    s = s_full if (step % cfg.full_every) == cfg.full_every - 1 else s_other
    g = _rng(cfg.seed, (S_LOGITS, 2, step))
    z = g.standard_normal((cfg.decision_rows, cfg.model.vocab), dtype=np.float32) * np.float32(s)
    return _store(z, cfg.dtype)


def long_context_history(cfg: LongContextConfig) -> np.ndarray:
    """The steady-state decode history: the k prefix positions just before the
    masked block, oldest first."""
    return np.arange(cfg.prefix_len - cfg.k, cfg.prefix_len, dtype=np.int32)


def random_logits(seed: int, rows: int, V: int, dtype: str, scale_lo: float = 0.1,
                  scale_hi: float = 20.0) -> np.ndarray:
    """Small generic logit matrix for tests: LogUniform row scales times N(0, 1)."""
    g = _rng(seed, (S_LOGITS, 3, rows, V))
    s = np.exp(np.log(scale_lo) + g.random(rows) * (np.log(scale_hi) - np.log(scale_lo)))
    z = g.standard_normal((rows, V), dtype=np.float32) * s[:, None].astype(np.float32)
    return _store(z, dtype)


def random_matrix(seed: int, key: Tuple[int, ...], shape: Tuple[int, ...], std: float,
                  dtype: str) -> np.ndarray:
    """Small generic N(0, std^2) tensor for kernel-level tests."""
    g = _rng(seed, (S_WEIGHTS, 99) + tuple(key))
    return _store(g.standard_normal(shape, dtype=np.float32) * np.float32(std), dtype)


def random_history(seed: int, positions: np.ndarray, n: int) -> np.ndarray:
    """A seeded decode order over `n` of the given positions (for selection tests)."""
    g = _rng(seed, (S_PROMPT, 7, n))
    return g.permutation(np.asarray(positions, dtype=np.int64))[:n].astype(np.int32)


def random_mask(seed: int, L: int, p: float) -> np.ndarray:
    g = _rng(seed, (S_PROMPT, 8, L))
    return (g.random(L) < p).astype(np.uint8)
