"""Seeded synthetic workloads for the EntropyCache denoising step (data only)."""
from . import configs, generators  # noqa: F401
from .configs import (BF16, DREAM_32K, DREAM_8K, ENTROPY_ONLY, F32, LLADA_LAYER,  # noqa: F401
                      LLADA_STACK, TINY, unmask_schedule)
