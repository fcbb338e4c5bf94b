"""CPU oracle for the EntropyCache denoising step.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously correct
float64 NumPy statement of what one EntropyCache denoising step computes.  Only
the test suite, the smoke check and the benchmark's CPU-baseline leg import it;
the GPU library never calls, links or loads anything here, and nothing here
imports the GPU library.  Inputs come from the shared seeded generators in the
`synth` package (data only).

Sources (cited by section, never by line):
  * "EntropyCache (zh)": the Chinese-language summary page of the paper
    "EntropyCache: Decoded Token Entropy Guided KV Caching for Diffusion
    Language Models" (gist.science/zh/paper/2603.18489).  Its technical summary
    §2.2 ("algorithm workflow") gives the three phases of a step, the
    max-entropy equation E_{t+1}, the threshold rule and the partial-recompute
    row set; §2.3 gives the O(V) / O(k) cost of the decision.
  * "EntropyCache (pt)": the Portuguese-language page on the same paper
    (gist.science/pt/paper/2603.18489).  Technical summary §1 (problem:
    bidirectional attention, full forward per step) and §2 (methodology:
    skip-or-recompute decision, decode history of the k most recent tokens,
    the observation that entropy predicts the KV drift).

Where the pages leave a step open the oracle takes one stated reading; every
reading is listed in the project's design notes and repeated at the function
that applies it.

Pinned by tests/test_oracle_*.py against closed forms, library routines (scipy
entropy, torch scaled-dot-product attention and rms_norm), brute force and the
method's invariants.  Two pins restate whole steps with torch full-sequence
forwards: the storage rounding points (a correctly rounding float64 forward),
and the multi-layer partial steps (stale caches of unselected rows propagating
through several layers: a full forward whose unselected positions take their
K/V from caches kept beside it), both bit for bit.
"""
from .rounding import to_storage, round_bf16  # noqa: F401
from .entropy import (softmax_entropy, row_stats, max_entropy, decide, entropy_max,  # noqa: F401
                      choose)
from .selection import select_rows, candidates, sliding_window  # noqa: F401
from .layers import linear, kv_refresh, bidir_attention, rmsnorm, swiglu  # noqa: F401
from .drift import cosine_distance, value_drift  # noqa: F401
from .step import (Model, State, StepTrace, step, step_external, generate, init_state,  # noqa: F401
                   forward_rows, commit, generate_block_diffusion)
