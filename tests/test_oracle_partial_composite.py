"""Pin for the oracle's partial steps in a multi-layer stack.

On a partial step only the selected rows are recomputed (EntropyCache (zh)
§2.2); every other position is read from the KV cache, in every layer, as it
was when that position was last recomputed.  In a stack this composite has no
closed form: an unselected row's deeper-layer K/V carry the tokens of the step
that last computed them.

The pin restates it with full-sequence forwards: torch runs every layer over
all positions, and before each layer's attention overwrites the K/V of the
positions outside the step's selection with caches kept beside it (which the
selected positions then update).  Rounding follows the storage points of the
rounding-placement pin, correctly rounded, so the oracle's stored logits must
match bit for bit on a mix of full and partial steps, with tokens decoded in
between.  The selection is derived here too (all positions on a full step;
else the block's masked positions and the last k decoded ones).

Teeth: a reference without the cache override (every step a fresh forward)
and one that reads layer 0's cache at every layer both give other logits.
"""
import math

import numpy as np
import torch
import torch.nn.functional as F

import oracle as O
from synth import configs as C
from synth import generators as G
from test_oracle_rounding_placement import store


def small_stack(n_layers):
    return C.scaled(C.LLADA_STACK, name=f"stack_small_pc{n_layers}", model_n_layers=n_layers, model_d=64,
                    model_n_q_heads=4, model_n_kv_heads=2, model_head_dim=16, model_vocab=300,
                    model_d_ffn=96, prompt_len=40, gen_len=24, block_len=8, k=4)


class TorchCache:
    def __init__(self, model, L):
        self.K = [torch.zeros(L, model.n_kv, model.dh, dtype=torch.float64) for _ in model.layers]
        self.V = [torch.zeros(L, model.n_kv, model.dh, dtype=torch.float64) for _ in model.layers]


def cached_forward(model, cache, tokens, sel, cand, dtype, mode="cache"):
    """Logits of `cand`; positions in `sel` are recomputed and written to the cache.
    mode "none": no override (a fresh forward); "layer0": every layer reads layer 0's cache."""
    S = lambda v: store(v, dtype)  # noqa: E731
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))  # noqa: E731
    L = len(tokens)
    Hq, Hkv, dh, d = model.n_q, model.n_kv, model.dh, model.d
    keep = torch.ones(L, dtype=torch.bool)
    keep[torch.from_numpy(np.asarray(sel))] = False          # positions read from the cache
    x = S(t(model.tok_emb)[torch.from_numpy(np.asarray(tokens))] + t(model.pos_emb)[:L])
    for l, lw in enumerate(model.layers):
        a = S(F.rms_norm(x, (d,), weight=t(lw["norm_attn"]), eps=model.eps))
        q, k, v = S(F.linear(a, t(lw["w_qkv"]))).split([Hq * dh, Hkv * dh, Hkv * dh], dim=1)
        k = k.reshape(L, Hkv, dh).clone()
        v = v.reshape(L, Hkv, dh).clone()
        src = 0 if mode == "layer0" else l
        if mode != "none":
            k[keep] = cache.K[src][keep]
            v[keep] = cache.V[src][keep]
        cache.K[l][~keep] = k[~keep]
        cache.V[l][~keep] = v[~keep]
        o = F.scaled_dot_product_attention(q.reshape(L, Hq, dh).transpose(0, 1), k.transpose(0, 1),
                                           v.transpose(0, 1), enable_gqa=True)
        x = S(x + F.linear(S(o).transpose(0, 1).reshape(L, Hq * dh), t(lw["w_o"])))
        a2 = S(F.rms_norm(x, (d,), weight=t(lw["norm_ffn"]), eps=model.eps))
        h = S(F.silu(F.linear(a2, t(lw["w_gate"]))) * F.linear(a2, t(lw["w_up"])))
        x = S(x + F.linear(h, t(lw["w_down"])))
    x = S(F.rms_norm(x, (d,), weight=t(model.norm_final), eps=model.eps))
    c = torch.from_numpy(np.asarray(cand))
    z = F.linear(x[c], t(model.w_lm))
    if model.logit_scale is not None:
        z = z * t(model.logit_scale)[c][:, None]
    return S(z).numpy()


# full (1) / partial (0) pattern: runs of partial steps after full ones, and a
# partial step right at a block change
FLAGS = [1, 0, 0, 0, 1, 0, 0, 1, 0, 0, 0, 0, 0, 1, 0, 0]


def run(n_layers, dtype="bf16", modes=("cache",)):
    cfg = small_stack(n_layers)
    model = O.Model.from_arrays(cfg.model, dtype, G.model_weights(cfg))
    toks, masked = G.initial_sequence(cfg)
    st = O.init_state(model, toks, masked)
    caches = {m: TorchCache(model, cfg.L) for m in modes}
    gaps = {m: [] for m in modes}
    n_partial = 0
    for (bs, bl, n), flag in zip(C.unmask_schedule(cfg), FLAGS):
        st.flag = flag
        before_tokens, before_masked = st.tokens.copy(), st.masked.copy()
        hist = list(st.history)
        tr = O.step(model, st, math.inf, cfg.k, bs, bl, n)
        cand = np.flatnonzero(before_masked[bs:bs + bl]) + bs
        sel = (np.arange(cfg.L) if flag else
               np.union1d(cand, np.asarray(hist[len(hist) - min(cfg.k, len(hist)):], dtype=np.int64)))
        np.testing.assert_array_equal(tr.rows, sel)
        np.testing.assert_array_equal(tr.cand, cand)
        n_partial += (not flag) and len(sel) < cfg.L
        for m in modes:
            want = cached_forward(model, caches[m], before_tokens, sel, cand, dtype, m)
            gaps[m].append(np.abs(want - tr.logits).max())
    return gaps, n_partial


def test_partial_steps_of_a_stack_match_full_forwards_with_cached_kv():
    for n_layers in (2, 3):
        gaps, n_partial = run(n_layers)
        assert n_partial >= 8
        assert max(gaps["cache"]) == 0, gaps["cache"]


def test_fp32_storage_also_matches():
    gaps, _ = run(2, "f32")
    assert max(gaps["cache"]) == 0


def test_pin_has_teeth():
    gaps, _ = run(2, modes=("cache", "none", "layer0"))
    assert max(gaps["cache"]) == 0
    partial = [i for i, f in enumerate(FLAGS) if not f]
    assert max(gaps["none"][i] for i in partial) > 1e-2       # the stale composite is visible
    assert max(gaps["layer0"][i] for i in partial) > 1e-2
    assert all(gaps["none"][i] == 0 for i, f in enumerate(FLAGS) if f)   # full steps need no cache
