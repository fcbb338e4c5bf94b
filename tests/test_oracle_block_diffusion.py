"""Pins for the oracle's block-diffusion mode (entropy gate inside the current block).

Reading (the Chinese page, §5, names block diffusion as a place for the
entropy signal to drive sub-block recomputation, and says no more): attention
is block-causal over blocks of block_len (the prompt included); a finished
block is committed once (a full pass over its rows with its final tokens);
inside the current block the gate chooses between recomputing every row of
the block and only its masked rows plus the last k decoded positions that lie
in it.

* tau = -inf recomputes the whole current block at every step.  Each step's
  logits must then equal an independent float64 torch forward over positions
  [0, block end) with a block-causal attention mask and no cache at all
  (earlier blocks holding their final tokens).  This pins the row selection,
  the key limit, the commits and the layer arithmetic together.
* Teeth: the same comparison fails for a bidirectional mask over all L
  positions, and for a run that skips the commits.
* Single-layer models: a row's K/V depend only on its own token, so with k at
  least the tokens decoded per step the gated path reproduces the tau = -inf
  trajectory for every tau; with k = 0 it does not.
* Rows: full and commit steps select exactly the block; partial steps select
  a subset of it; cache rows outside the block never change during its steps.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O
from synth import configs as C
from synth import generators as G


def small_stack():
    return C.scaled(C.LLADA_STACK, name="stack_small_bd", model_n_layers=2, model_d=64,
                    model_n_q_heads=4, model_n_kv_heads=2, model_head_dim=16, model_vocab=300,
                    model_d_ffn=96, prompt_len=40, gen_len=24, block_len=8, k=4)


def small_single():
    return C.scaled(C.LLADA_LAYER, name="layer_small_bd", model_d=64, model_n_q_heads=4,
                    model_n_kv_heads=2, model_head_dim=16, model_vocab=500, prompt_len=48,
                    gen_len=32, block_len=16, k=4)


def tiny():
    return C.scaled(C.TINY, name="tiny_bd", block_len=16, k=4)


def build(cfg, dtype):
    w = G.model_weights(cfg)
    model = O.Model.from_arrays(cfg.model, dtype, w)
    toks, masked = G.initial_sequence(cfg)
    return model, O.init_state(model, toks, masked)


def torch_block_causal_logits(model, tokens, n_pos, block_len, cand, causal=True):
    """Logits of the candidate positions from one forward over positions
    [0, n_pos), no cache; query i attends to key j iff j's block is not after
    i's (blocks of block_len from position 0), or to every key when not causal."""
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))  # noqa: E731
    Hq, Hkv, dh, d = model.n_q, model.n_kv, model.dh, model.d
    tok = torch.from_numpy(np.asarray(tokens[:n_pos]))
    x = t(model.tok_emb)[tok] + t(model.pos_emb)[:n_pos]
    blk = torch.arange(n_pos) // block_len
    mask = (blk[None, :] <= blk[:, None]) if causal else torch.ones(n_pos, n_pos, dtype=torch.bool)
    for lw in model.layers:
        a = F.rms_norm(x, (d,), weight=t(lw["norm_attn"]), eps=model.eps) if model.d_ffn else x
        q, k, v = F.linear(a, t(lw["w_qkv"])).split([Hq * dh, Hkv * dh, Hkv * dh], dim=1)
        q = q.reshape(n_pos, Hq, dh).transpose(0, 1)
        k = k.reshape(n_pos, Hkv, dh).transpose(0, 1)
        v = v.reshape(n_pos, Hkv, dh).transpose(0, 1)
        o = F.scaled_dot_product_attention(q, k, v, attn_mask=mask, enable_gqa=True)
        x = x + F.linear(o.transpose(0, 1).reshape(n_pos, Hq * dh), t(lw["w_o"]))
        if model.d_ffn:
            a2 = F.rms_norm(x, (d,), weight=t(lw["norm_ffn"]), eps=model.eps)
            x = x + F.linear(F.silu(F.linear(a2, t(lw["w_gate"]))) * F.linear(a2, t(lw["w_up"])),
                             t(lw["w_down"]))
    if model.d_ffn:
        x = F.rms_norm(x, (d,), weight=t(model.norm_final), eps=model.eps)
    c = torch.from_numpy(np.asarray(cand))
    z = F.linear(x[c], t(model.w_lm))
    if model.logit_scale is not None:
        z = z * t(model.logit_scale)[c][:, None]
    return z.numpy()


def run_vanilla(cfg, model, st, n_steps, commits=True):
    """tau = -inf block diffusion; yields (tokens before the step, trace) for
    each denoising step (commits are not yielded)."""
    sched = C.unmask_schedule(cfg)
    bl = cfg.block_len
    for bs in range(0, cfg.prompt_len, bl):
        O.commit(model, st, bs, bl, cfg.k)
    for i, (bs, blen, n) in enumerate(sched[:n_steps]):
        toks = st.tokens.copy()
        tr = O.step(model, st, -math.inf, cfg.k, bs, blen, n, block_causal=True)
        yield toks, bs + blen, tr
        if commits and (i + 1 == len(sched) or sched[i + 1][0] != bs):
            O.commit(model, st, bs, blen, cfg.k)


@pytest.mark.parametrize("cfg_fn", [small_single, small_stack, tiny])
def test_vanilla_block_diffusion_matches_block_causal_forward(cfg_fn):
    cfg = cfg_fn()
    assert cfg.prompt_len % cfg.block_len == 0
    model, st = build(cfg, "f64")
    n_blocks_seen = set()
    for toks, end, tr in run_vanilla(cfg, model, st, 3 * cfg.block_len):
        want = torch_block_causal_logits(model, toks, end, cfg.block_len, tr.cand)
        np.testing.assert_allclose(tr.logits, want, rtol=1e-10, atol=1e-10)
        n_blocks_seen.add(end)
    assert len(n_blocks_seen) >= 2          # the comparison crossed a commit


@pytest.mark.parametrize("cfg_fn", [small_single, small_stack])
def test_block_causal_pin_has_teeth(cfg_fn):
    cfg = cfg_fn()
    model, st = build(cfg, "f64")
    gaps_mask, gaps_commit = [], []
    for toks, end, tr in run_vanilla(cfg, model, st, 2 * cfg.block_len):
        full_mask = torch_block_causal_logits(model, toks, cfg.L, cfg.block_len, tr.cand, causal=False)
        gaps_mask.append(np.abs(full_mask - tr.logits).max())
    model, st = build(cfg, "f64")
    for toks, end, tr in run_vanilla(cfg, model, st, 2 * cfg.block_len, commits=False):
        want = torch_block_causal_logits(model, toks, end, cfg.block_len, tr.cand)
        gaps_commit.append(np.abs(want - tr.logits).max())
    assert max(gaps_mask) > 1e-3            # a bidirectional mask gives other logits
    assert max(gaps_commit) > 1e-3          # so does leaving finished blocks uncommitted


def _trajectory(cfg, dtype, tau, k):
    model, st = build(cfg, dtype)
    tr = O.generate_block_diffusion(model, st, cfg.prompt_len, C.unmask_schedule(cfg), tau, k,
                                    keep_logits=True)
    return [t for t in tr if t.cand.size], st


@pytest.mark.parametrize("cfg_fn,dtype", [(tiny, "f32"), (small_single, "bf16")])
def test_single_layer_block_diffusion_is_tau_invariant(cfg_fn, dtype):
    cfg = cfg_fn()
    full, st_full = _trajectory(cfg, dtype, -math.inf, cfg.k)
    part, st_part = _trajectory(cfg, dtype, math.inf, cfg.k)
    assert any(t.flag_used == 0 and len(t.rows) < cfg.block_len for t in part)
    for a, b in zip(full, part):
        np.testing.assert_array_equal(a.chosen, b.chosen)
        np.testing.assert_allclose(a.logits, b.logits, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(st_full.tokens, st_part.tokens)
    # k = 0: the just-decoded rows keep stale K/V inside the block
    stale, _ = _trajectory(cfg, dtype, math.inf, 0)
    assert max(np.abs(a.logits - b.logits).max() for a, b in zip(full, stale)) > 1e-6


def test_rows_stay_inside_the_block_and_other_rows_keep_their_cache():
    cfg = small_stack()
    model, st = build(cfg, "bf16")
    sched = C.unmask_schedule(cfg)
    for bs in range(0, cfg.prompt_len, cfg.block_len):
        tr = O.commit(model, st, bs, cfg.block_len, cfg.k)
        np.testing.assert_array_equal(tr.rows, np.arange(bs, bs + cfg.block_len))
        assert tr.flag_next == 0 and tr.chosen.size == 0
    for i, (bs, bl, n) in enumerate(sched):
        before = [(k.copy(), v.copy()) for k, v in zip(st.K, st.V)]
        tr = O.step(model, st, 1.0, cfg.k, bs, bl, n, block_causal=True)
        if tr.flag_used:
            np.testing.assert_array_equal(tr.rows, np.arange(bs, bs + bl))
        assert np.all((tr.rows >= bs) & (tr.rows < bs + bl))
        outside = np.r_[0:bs, bs + bl:cfg.L]
        for (k0, v0), k1, v1 in zip(before, st.K, st.V):
            assert np.array_equal(k0[:, outside], k1[:, outside])
            assert np.array_equal(v0[:, outside], v1[:, outside])
        if i + 1 == len(sched) or sched[i + 1][0] != bs:
            O.commit(model, st, bs, bl, cfg.k)


def test_block_causal_selection_hand_worked():
    masked = np.zeros(20, dtype=bool)
    masked[[9, 11, 14]] = True                 # current block [8, 16)
    history = [3, 5, 12, 8, 17, 10]            # 3, 5 earlier blocks; 17 past the block
    got = O.select_rows(0, masked, 8, 8, history, 4, block_causal=True)
    np.testing.assert_array_equal(got, [8, 9, 10, 11, 12, 14])   # 17 dropped, 3/5 outside last 4
    got = O.select_rows(0, masked, 8, 8, history, 6, block_causal=True)
    np.testing.assert_array_equal(got, [8, 9, 10, 11, 12, 14])   # 3 and 5 are in earlier blocks
    np.testing.assert_array_equal(O.select_rows(1, masked, 8, 8, history, 4, block_causal=True),
                                  np.arange(8, 16))
    # the plain mode keeps positions outside the block
    np.testing.assert_array_equal(O.select_rows(0, masked, 8, 8, history, 4),
                                  [8, 9, 10, 11, 12, 14, 17])
    with pytest.raises(ValueError):
        model, st = build(small_single(), "f64")
        O.step(model, st, 1.0, 4, -1, 16, 1, block_causal=True)
