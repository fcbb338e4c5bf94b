"""GPU parity of the KV-drift diagnostic (ec_state.kv_drift) with the oracle.

On a full step each layer reports the mean and maximum over positions of
1 - cos(stale, fresh) of the Value vectors (oracle.drift); partial steps leave
the output unchanged.  fp32: within 1e-4 + 1e-3 |d| of the oracle (both sides'
caches agree to fp32 rounding).  bf16, teacher forced (the GPU state is the
oracle's before every step, so the stale caches are identical): within
5e-3 + 2e-2 |d|, the fresh Value vectors differing by bf16 rounding.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
from entropy_gated_kv_amd.runner import DeviceModel, DeviceSequence
from synth import configs as C
from synth import generators as G

pytestmark = pytest.mark.gpu


def setup(cfg, L_cap=None):
    w = G.model_weights(cfg)
    model = O.Model.from_arrays(cfg.model, cfg.dtype, w)
    toks, masked = G.initial_sequence(cfg)
    st = O.init_state(model, toks, masked)
    dm = DeviceModel(cfg.model, cfg.dtype, L_cap or cfg.L, w)
    ds = DeviceSequence(dm, toks, masked, history_cap=max(cfg.gen_len, cfg.k), max_block=cfg.block_len)
    ds.enable_drift()
    return model, st, ds


def check(g, ref, atol, rtol, what):
    both_nan = np.isnan(g) & np.isnan(ref)
    assert np.array_equal(np.isnan(g), np.isnan(ref)), (what, g, ref)
    ok = both_nan | (np.abs(g - ref) <= atol + rtol * np.abs(ref))
    assert ok.all(), (what, g, ref)


@pytest.mark.parametrize("tau", [1.5, math.inf])
def test_tiny_fp32_free_running(tau):
    # L = 254 (not a whole number of 16-byte vectors) in a 256-row cache
    cfg = C.scaled(C.TINY, name="tiny_drift", prompt_len=190)
    model, st, ds = setup(cfg, L_cap=256)
    n_full = 0
    prev = None
    for i, (bs, bl, n) in enumerate(C.unmask_schedule(cfg)):
        tr = O.step(model, st, tau, cfg.k, bs, bl, n, drift=True)
        ds.step(tau, cfg.k, bs, bl, n)
        torch.cuda.synchronize()
        g = ds.kv_drift.cpu().numpy().astype(np.float64)
        if tr.flag_used:
            check(g, tr.drift, 1e-4, 1e-3, f"step {i}")
            n_full += 1
        else:
            assert np.array_equal(g, prev, equal_nan=True), f"step {i}: partial step changed the drift"
        prev = g
    assert n_full == (16 if tau == 1.5 else 1)
    if tau == 1.5:
        assert np.all(np.isfinite(prev)) and np.all(prev[:, 1] > 0)


def test_bf16_two_layer_stack_teacher_forced():
    cfg = C.scaled(C.LLADA_STACK, name="stack_drift", model_n_layers=2, model_d=256,
                   model_n_q_heads=4, model_n_kv_heads=2, model_head_dim=64, model_vocab=2048,
                   model_d_ffn=512, prompt_len=96, gen_len=64, block_len=32, k=16)
    model, st, ds = setup(cfg)
    n_full = 0
    for i, (bs, bl, n) in enumerate(C.unmask_schedule(cfg)[:24]):
        ds.load_state(st.tokens, st.masked, st.history, st.flag, st.K, st.V)
        before = ds.kv_drift.cpu().numpy().astype(np.float64)
        tr = O.step(model, st, 1.0, cfg.k, bs, bl, n, drift=True)
        ds.step(1.0, cfg.k, bs, bl, n)
        torch.cuda.synchronize()
        g = ds.kv_drift.cpu().numpy().astype(np.float64)
        if tr.flag_used:
            check(g, tr.drift, 5e-3, 2e-2, f"step {i}")
            n_full += 1
        else:
            assert np.array_equal(g, before, equal_nan=True), f"step {i}: partial step changed the drift"
    assert n_full >= 2
