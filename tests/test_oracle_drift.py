"""Pins of the KV-drift diagnostic (oracle.drift) against closed forms, scipy's
cosine distance, and the step's invariants.

EntropyCache (zh) §2.1 and (pt) §2: the drift is measured on the Value vectors
as a cosine distance; the aggregation (per position over the concatenated KV
heads, then mean and max over positions) is the reading taken here.
"""
import numpy as np
import pytest
from scipy.spatial import distance

import oracle as O
from synth import configs as C
from synth import generators as G


def test_cosine_distance_closed_forms():
    a = np.array([[1.0, 2.0, 3.0], [1.0, 0.0, 0.0], [1.0, 2.0, 3.0], [2.0, -1.0, 0.5], [0.0, 0.0, 0.0]])
    b = np.array([[1.0, 2.0, 3.0], [0.0, 5.0, 0.0], [-1.0, -2.0, -3.0], [4.0, -2.0, 1.0], [1.0, 1.0, 1.0]])
    d = O.cosine_distance(a, b)
    np.testing.assert_allclose(d[:4], [0.0, 1.0, 2.0, 0.0], atol=1e-15)   # same, orthogonal, opposite, scaled
    assert np.isnan(d[4])                                                 # zero vector: left out


def test_cosine_distance_matches_scipy():
    rng = np.random.default_rng(0)
    a, b = rng.standard_normal((50, 37)), rng.standard_normal((50, 37))
    d = O.cosine_distance(a, b)
    ref = np.array([distance.cosine(a[i], b[i]) for i in range(50)])
    np.testing.assert_allclose(d, ref, rtol=1e-12, atol=1e-14)


def test_value_drift_concatenates_heads_per_position():
    # V caches [Hkv = 2, L = 3, dh = 4]
    rng = np.random.default_rng(1)
    Vs = rng.standard_normal((2, 3, 4))
    Vf = Vs.copy()
    Vf[1, 1] = -Vs[1, 1]                 # position 1: head 0 unchanged, head 1 negated
    Vs[:, 2] = 0.0                        # position 2: never computed
    n0, n1 = np.sum(Vs[0, 1] ** 2), np.sum(Vs[1, 1] ** 2)
    d1 = 1.0 - (n0 - n1) / (n0 + n1)      # closed form of the concatenated vector
    mean, mx = O.value_drift(Vs, Vf)
    np.testing.assert_allclose([mean, mx], [d1 / 2, d1], rtol=1e-12)
    # a per-head average would give (0 + 2) / 2 = 1 at position 1, not d1
    assert abs(d1 - 1.0) > 1e-3


def test_value_drift_empty_cache_is_nan():
    Vs = np.zeros((2, 5, 4))
    Vf = np.ones((2, 5, 4))
    assert np.all(np.isnan(O.value_drift(Vs, Vf)))


def tiny_stack():
    cfg = C.scaled(C.LLADA_STACK, name="drift", model_n_layers=2, model_d=64, model_n_q_heads=4,
                   model_n_kv_heads=2, model_head_dim=16, model_vocab=97, model_d_ffn=128,
                   prompt_len=24, gen_len=16, block_len=8, k=4)
    w = G.model_weights(cfg)
    model = O.Model.from_arrays(cfg.model, "f32", w)
    toks, masked = G.initial_sequence(cfg)
    return cfg, model, toks, masked


def test_full_recompute_of_an_unchanged_sequence_has_zero_drift():
    cfg, model, toks, masked = tiny_stack()
    st = O.init_state(model, toks, masked)
    rows = np.arange(cfg.L)
    first = []
    O.forward_rows(model, st, rows, first)
    assert np.all(np.isnan(np.array(first)))                  # empty caches before
    again = []
    O.forward_rows(model, st, rows, again)
    np.testing.assert_allclose(np.array(again), np.zeros((2, 2)), atol=1e-12)   # identical vectors


def test_step_reports_drift_on_full_steps_only():
    cfg, model, toks, masked = tiny_stack()
    st = O.init_state(model, toks, masked)
    sched = C.unmask_schedule(cfg)
    traces = [O.step(model, st, 1.5, cfg.k, bs, bl, n, drift=True) for bs, bl, n in sched[:6]]
    assert traces[0].flag_used == 1 and np.all(np.isnan(traces[0].drift))
    for t in traces[1:]:
        if t.flag_used:
            assert t.drift.shape == (2, 2)
            assert np.all((t.drift >= 0) & (t.drift <= 2)) and np.all(t.drift[:, 0] <= t.drift[:, 1])
        else:
            assert t.drift is None
    assert any(t.flag_used for t in traces[1:])               # tau 1.5 on random logits: full steps
