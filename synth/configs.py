"""Workload shapes for the EntropyCache denoising step.

Each config names a synthetic workload: the model shape, the sequence layout
(prompt, generated blocks), the decode schedule, k and tau.  Nothing here does
any of the method's arithmetic; it only describes sizes and schedules.

Citations: "EntropyCache (zh) §2.2" is the Chinese-language summary page of the
paper "EntropyCache: Decoded Token Entropy Guided KV Caching for Diffusion
Language Models" (gist.science/zh/paper/2603.18489), technical summary section
2.2 (algorithm workflow).  "EntropyCache (pt) §2" is the Portuguese-language
page on the same paper (gist.science/pt/paper/2603.18489), technical summary
section 2 (methodology).
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Tuple


F32 = "f32"
BF16 = "bf16"


@dataclasses.dataclass(frozen=True)
class ModelShape:
    n_layers: int
    d: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    vocab: int
    d_ffn: int = 0          # 0: no norms and no FFN (attention-only layer)
    rms_eps: float = 1e-5

    @property
    def qkv_out(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim

    @property
    def mask_id(self) -> int:
        # The MASK token has its own embedding row at index `vocab`; the LM head
        # has only `vocab` output columns, so MASK can never be decoded.
        return self.vocab


@dataclasses.dataclass(frozen=True)
class StepConfig:
    """A full denoising workload: model + sequence layout + decode schedule."""
    name: str
    seed: int
    dtype: str
    model: ModelShape
    prompt_len: int
    gen_len: int
    block_len: int
    k: int
    taus: Tuple[float, ...]
    schedule: str                 # "fixed:<n>" or "alternate12"
    logit_scale: Optional[Tuple[float, float]] = None  # LogUniform(lo, hi) per position

    @property
    def L(self) -> int:
        return self.prompt_len + self.gen_len

    @property
    def n_blocks(self) -> int:
        return self.gen_len // self.block_len


def unmask_schedule(cfg: StepConfig) -> List[Tuple[int, int, int]]:
    """Host-side schedule: one (block_start, block_len, n_unmask) per step.

    The count of still-masked positions in the current block is known on the
    host at every step (each step unmasks exactly min(n_unmask, remaining)), so
    the whole schedule is fixed before the first step.  "alternate12" unmasks
    1, 2, 1, 2, ... tokens per step within each block.
    """
    out = []
    for b in range(cfg.n_blocks):
        start = cfg.prompt_len + b * cfg.block_len
        remaining = cfg.block_len
        s = 0
        while remaining > 0:
            if cfg.schedule == "alternate12":
                want = 1 + (s % 2)
            elif cfg.schedule.startswith("fixed:"):
                want = int(cfg.schedule.split(":")[1])
            else:
                raise ValueError(cfg.schedule)
            n = min(want, remaining)
            out.append((start, cfg.block_len, n))
            remaining -= n
            s += 1
    return out


# -- the five workloads ------------------------------------------------------

TINY = StepConfig(
    name="tiny_fp32_L256",
    seed=1,
    dtype=F32,
    model=ModelShape(n_layers=1, d=128, n_q_heads=4, n_kv_heads=4, head_dim=32, vocab=1024),
    prompt_len=192, gen_len=64, block_len=64, k=16,
    taus=(1.5,), schedule="fixed:4",
)


@dataclasses.dataclass(frozen=True)
class EntropyOnlyConfig:
    name: str
    seed: int
    dtype: str
    rows: int
    vocab: int
    scale_range: Tuple[float, float]   # LogUniform per-row scale
    boost_frac: float                  # fraction of rows with one logit boosted
    boost: float
    tau: float

    @property
    def n_boosted(self) -> int:
        return int(math.ceil(self.boost_frac * self.rows - 1e-9))


ENTROPY_ONLY = EntropyOnlyConfig(
    name="entropy_4096x126464_bf16", seed=2, dtype=BF16, rows=4096, vocab=126464,
    scale_range=(0.1, 20.0), boost_frac=0.1, boost=15.0, tau=2.0,
)

LLADA_LAYER = StepConfig(
    name="llada8b_layer_L1024",
    seed=3,
    dtype=BF16,
    model=ModelShape(n_layers=1, d=4096, n_q_heads=32, n_kv_heads=32, head_dim=128, vocab=126464),
    prompt_len=512, gen_len=512, block_len=32, k=64,
    taus=(0.5, 1.0, 2.0), schedule="alternate12", logit_scale=(2.0, 100.0),
)


@dataclasses.dataclass(frozen=True)
class LongContextConfig:
    """Steady-state long-context layer: fixed 96 selected rows per partial step.

    Rows on a partial step are the 32 positions of the masked block plus the 64
    prefix positions just before it (standing in for the decode history).  The
    decision comes from two synthetic decoded rows per step (no LM head).
    """
    name: str
    seed: int
    dtype: str
    model: ModelShape
    prefix_len: int
    block_len: int
    k: int
    tau: float
    full_every: int
    decision_rows: int
    decision_scales: Tuple[float, float]   # (scale on forced-full steps, otherwise)

    @property
    def L(self) -> int:
        return self.prefix_len + self.block_len

    # the sequence helpers shared with StepConfig: prefix = prompt, block = gen
    @property
    def prompt_len(self) -> int:
        return self.prefix_len

    @property
    def gen_len(self) -> int:
        return self.block_len

    lm_head = False


def _dream(prefix: int) -> LongContextConfig:
    return LongContextConfig(
        name=f"dream7b_layer_L{prefix + 32}",
        seed=4,
        dtype=BF16,
        model=ModelShape(n_layers=1, d=3584, n_q_heads=28, n_kv_heads=4, head_dim=128, vocab=152064),
        prefix_len=prefix, block_len=32, k=64, tau=2.0, full_every=8,
        decision_rows=2, decision_scales=(0.1, 20.0),
    )


DREAM_8K = _dream(8192)
DREAM_32K = _dream(32768)

LLADA_STACK = StepConfig(
    name="llada8b_stack32_L2048",
    seed=5,
    dtype=BF16,
    model=ModelShape(n_layers=32, d=4096, n_q_heads=32, n_kv_heads=32, head_dim=128,
                     vocab=126464, d_ffn=12288),
    prompt_len=1792, gen_len=256, block_len=32, k=64,
    taus=(1.0,), schedule="alternate12", logit_scale=(2.0, 100.0),
)


def scaled(cfg: StepConfig, **kw) -> StepConfig:
    """A copy of a step config with some fields replaced (used for small test cases)."""
    model_kw = {k[6:]: v for k, v in kw.items() if k.startswith("model_")}
    rest = {k: v for k, v in kw.items() if not k.startswith("model_")}
    model = dataclasses.replace(cfg.model, **model_kw) if model_kw else cfg.model
    return dataclasses.replace(cfg, model=model, **rest)
