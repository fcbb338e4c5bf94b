"""Pins for the oracle's denoising step and generation loop.

* tau = -inf makes every step a full forward; then each step's logits must equal
  an independent float64 torch forward over all positions (F.linear,
  F.scaled_dot_product_attention with GQA, F.rms_norm, F.silu).
* Single-layer models: a position's layer-0 K/V depend only on its token and
  position, and every token that changes is in the last k decoded tokens at
  the next step (k >= tokens per step), so the partial path must reproduce
  the full path's trajectory exactly, for every tau.  With k = 0 it must not
  (the just-decoded tokens keep stale K/V), which shows the pin has teeth.
* A partial step leaves every unselected cache row bitwise unchanged.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O
from synth import configs as C
from synth import generators as G


def small_stack(n_layers=2):
    return C.scaled(C.LLADA_STACK, name="stack_small", model_n_layers=n_layers, model_d=64,
                    model_n_q_heads=4, model_n_kv_heads=2, model_head_dim=16, model_vocab=300,
                    model_d_ffn=96, prompt_len=40, gen_len=24, block_len=8, k=4)


def small_single(dtype=C.BF16):
    return C.scaled(C.LLADA_LAYER, name="layer_small", dtype=dtype, model_d=64, model_n_q_heads=4,
                    model_n_kv_heads=2, model_head_dim=16, model_vocab=500, prompt_len=48,
                    gen_len=32, block_len=16, k=4)


def build(cfg, dtype=None):
    w = G.model_weights(cfg)
    model = O.Model.from_arrays(cfg.model, dtype or cfg.dtype, w)
    toks, masked = G.initial_sequence(cfg)
    return model, O.init_state(model, toks, masked)


def torch_forward_logits(model, tokens, cand):
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))  # noqa: E731
    L = len(tokens)
    Hq, Hkv, dh, d = model.n_q, model.n_kv, model.dh, model.d
    x = t(model.tok_emb)[torch.from_numpy(np.asarray(tokens))] + t(model.pos_emb)[:L]
    for lw in model.layers:
        a = F.rms_norm(x, (d,), weight=t(lw["norm_attn"]), eps=model.eps) if model.d_ffn else x
        q, k, v = F.linear(a, t(lw["w_qkv"])).split([Hq * dh, Hkv * dh, Hkv * dh], dim=1)
        q = q.reshape(L, Hq, dh).transpose(0, 1)
        k = k.reshape(L, Hkv, dh).transpose(0, 1)
        v = v.reshape(L, Hkv, dh).transpose(0, 1)
        o = F.scaled_dot_product_attention(q, k, v, is_causal=False, enable_gqa=True)
        x = x + F.linear(o.transpose(0, 1).reshape(L, Hq * dh), t(lw["w_o"]))
        if model.d_ffn:
            a2 = F.rms_norm(x, (d,), weight=t(lw["norm_ffn"]), eps=model.eps)
            x = x + F.linear(F.silu(F.linear(a2, t(lw["w_gate"]))) * F.linear(a2, t(lw["w_up"])),
                             t(lw["w_down"]))
    if model.d_ffn:
        x = F.rms_norm(x, (d,), weight=t(model.norm_final), eps=model.eps)
    z = F.linear(x[torch.from_numpy(np.asarray(cand))], t(model.w_lm))
    if model.logit_scale is not None:
        z = z * t(model.logit_scale)[torch.from_numpy(np.asarray(cand))][:, None]
    return z.numpy()


@pytest.mark.parametrize("cfg_fn", [lambda: C.TINY, small_stack, small_single])
def test_vanilla_steps_match_torch_forward(cfg_fn):
    cfg = cfg_fn()
    model, st = build(cfg, "f64")
    sched = C.unmask_schedule(cfg)[:10]
    for bs, bl, n in sched:
        toks = st.tokens.copy()
        tr = O.step(model, st, -math.inf, cfg.k, bs, bl, n)
        assert tr.flag_used == 1 and tr.flag_next == 1
        np.testing.assert_array_equal(tr.rows, np.arange(cfg.L))
        want = torch_forward_logits(model, toks, tr.cand)
        np.testing.assert_allclose(tr.logits, want, rtol=1e-10, atol=1e-10)


def _run(cfg, dtype, tau, k, n_steps=None):
    model, st = build(cfg, dtype)
    sched = C.unmask_schedule(cfg)
    tr = O.generate(model, st, sched, tau, k, keep_logits=True, n_steps=n_steps)
    return tr, st


@pytest.mark.parametrize("cfg_fn,dtype", [(lambda: C.TINY, "f32"), (lambda: C.TINY, "f64"),
                                          (small_single, "bf16")])
def test_single_layer_trajectory_is_tau_invariant(cfg_fn, dtype):
    cfg = cfg_fn()
    full, st_full = _run(cfg, dtype, -math.inf, cfg.k)
    part, st_part = _run(cfg, dtype, math.inf, cfg.k)
    assert all(t.flag_used == 1 for t in full)
    assert part[0].flag_used == 1 and all(t.flag_used == 0 for t in part[1:])
    for a, b in zip(full, part):
        np.testing.assert_array_equal(a.chosen, b.chosen)
        np.testing.assert_array_equal(a.argmax, b.argmax)
        np.testing.assert_allclose(a.logits, b.logits, rtol=1e-12, atol=1e-12)
        assert abs(a.E - b.E) <= 1e-12
    np.testing.assert_array_equal(st_full.tokens, st_part.tokens)
    assert st_full.history == st_part.history


def test_without_history_the_partial_path_goes_stale():
    cfg = C.TINY
    _, st_full = _run(cfg, "f64", -math.inf, cfg.k, n_steps=3)
    _, st_k0 = _run(cfg, "f64", math.inf, 0, n_steps=3)
    _, st_k = _run(cfg, "f64", math.inf, cfg.k, n_steps=3)
    np.testing.assert_allclose(st_k.K[0], st_full.K[0], rtol=1e-12, atol=1e-12)
    decoded_step1 = st_full.history[:4]
    assert not np.allclose(st_k0.K[0][:, decoded_step1], st_full.K[0][:, decoded_step1])


def test_literal_tiny_config_only_takes_full_steps():
    # random N(0, 0.02) weights give near-uniform logits: E is close to log V, far above tau
    tr, st = _run(C.TINY, "f32", C.TINY.taus[0], C.TINY.k)
    assert len(tr) == 16 and all(t.flag_used == 1 for t in tr)
    assert all(t.E > 6.0 for t in tr)
    assert not st.masked.any()


def test_partial_step_keeps_unselected_rows_of_every_layer():
    cfg = small_stack()
    model, st = build(cfg, "bf16")
    sched = C.unmask_schedule(cfg)
    O.step(model, st, math.inf, cfg.k, *sched[0])
    O.step(model, st, math.inf, cfg.k, *sched[1])
    K0 = [k.copy() for k in st.K]
    V0 = [v.copy() for v in st.V]
    tr = O.step(model, st, math.inf, cfg.k, *sched[2])
    assert tr.flag_used == 0
    keep = np.setdiff1d(np.arange(cfg.L), tr.rows)
    for l in range(cfg.model.n_layers):
        assert np.array_equal(st.K[l][:, keep], K0[l][:, keep])
        assert np.array_equal(st.V[l][:, keep], V0[l][:, keep])
    assert len(tr.rows) == len(tr.cand) + min(cfg.k, 3)


def test_schedules():
    s3 = C.unmask_schedule(C.LLADA_LAYER)
    assert len(s3) == 16 * 22
    assert sum(n for _, _, n in s3) == 512
    s1 = C.unmask_schedule(C.TINY)
    assert len(s1) == 16 and all(n == 4 for _, _, n in s1)
    assert len(C.unmask_schedule(C.LLADA_STACK)) == 8 * 22


def test_history_appends_each_steps_positions_in_ascending_order():
    # Stated reading: positions unmasked in one step enter the history in
    # ascending position order, so "the k most recent" cuts at that order.
    cfg = small_single()
    model, st = build(cfg, "bf16")
    sched = C.unmask_schedule(cfg)
    seen = 0
    for bs, bl, n in sched[:8]:
        tr = O.step(model, st, math.inf, cfg.k, bs, bl, n)
        assert st.history[seen:] == sorted(int(c) for c in tr.chosen)
        seen = len(st.history)
    # k = 4 cuts inside a two-token step of this 1,2,1,2 schedule
    assert sched[6][2] == 1 and sched[5][2] == 2
    tr = O.step(model, st, math.inf, cfg.k, *sched[8])
    recent = set(st.history[-len(tr.chosen) - cfg.k:-len(tr.chosen)])
    assert recent <= set(tr.rows.tolist())


def test_external_decoding_step_agrees_with_step():
    """Handing step_external the logits that step() decoded (the chosen rows)
    must reproduce step()'s rows, caches, E and decision, and leave tokens,
    mask and history alone."""
    cfg = small_single()
    model, st = build(cfg)
    sched = C.unmask_schedule(cfg)
    for bs, bl, n in sched[:5]:
        O.step(model, st, 1.0, cfg.k, bs, bl, n)
    for bs, bl, n in sched[5:9]:
        a, b = st.copy(), st.copy()
        tr = O.step(model, a, 1.0, cfg.k, bs, bl, n)
        ext = tr.logits[np.searchsorted(tr.cand, tr.chosen)]
        te = O.step_external(model, b, 1.0, cfg.k, bs, bl, ext)
        np.testing.assert_array_equal(te.rows, tr.rows)
        for l in range(cfg.model.n_layers):
            assert np.array_equal(a.K[l], b.K[l]) and np.array_equal(a.V[l], b.V[l])
        assert te.E == tr.E and b.flag == a.flag == te.flag_next
        assert np.array_equal(b.tokens, st.tokens) and np.array_equal(b.masked, st.masked)
        assert b.history == st.history
        st = a


def small_long_context():
    return C.scaled(C.DREAM_8K, name="long_small", model_d=64, model_n_q_heads=7,
                    model_n_kv_heads=1, model_head_dim=16, model_vocab=500, prefix_len=96,
                    block_len=8, k=16)


def test_long_context_steady_state_rows_and_forced_full_steps():
    """Steady state: partial steps recompute exactly the masked block plus the
    k history positions before it; the synthetic decision rows (flat on every
    8th step, peaked otherwise) force a full step after each flat step."""
    cfg = small_long_context()
    w = G.model_weights(cfg)
    assert w["w_lm"] is None
    model = O.Model.from_arrays(cfg.model, cfg.dtype, w)
    toks, masked = G.initial_sequence(cfg)
    st = O.init_state(model, toks, masked)
    st.history = [int(p) for p in G.long_context_history(cfg)]
    steady = np.union1d(np.arange(cfg.prefix_len, cfg.L), G.long_context_history(cfg))
    assert len(steady) == cfg.block_len + cfg.k
    for t in range(0, 18):
        tr = O.step_external(model, st, cfg.tau, cfg.k, cfg.prefix_len, cfg.block_len,
                             G.decision_logits(cfg, t))
        full = t == 0 or (t - 1) % cfg.full_every == cfg.full_every - 1
        np.testing.assert_array_equal(tr.rows, np.arange(cfg.L) if full else steady, err_msg=str(t))
        flat = t % cfg.full_every == cfg.full_every - 1
        # flat rows: H close to ln V; peaked rows: H well below tau
        assert (tr.E > math.log(cfg.model.vocab) - 0.1) if flat else (tr.E < cfg.tau - 0.5), (t, tr.E)
        assert tr.flag_next == int(flat)


def test_streamed_weights_equal_model_weights():
    cfg = small_stack(3)
    a, b = G.model_weights(cfg), G.model_weights_streamed(cfg)
    la = a.pop("layers")
    lb = list(b.pop("layers"))
    assert len(la) == len(lb) == 3
    for x, y in zip(la, lb):
        assert x.keys() == y.keys() and all(np.array_equal(x[k], y[k]) for k in x)
    assert a.keys() == b.keys()
    for k in a:
        assert (a[k] is None and b[k] is None) or np.array_equal(a[k], b[k]), k
