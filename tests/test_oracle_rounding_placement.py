"""Pin for where the oracle rounds to the storage dtype.

The oracle computes in float64 and rounds to the workload's storage dtype
(bf16 or fp32) at fixed points of the layer: the layer input; Q, K and V; the
attention output; x after each residual add; each normed activation; the FFN
intermediate; the logits after their scale.  The pages fix no precision; this
is the reading the whole step follows.

The pin is an independent float64 torch forward over all positions (tau = -inf
makes every oracle step a full forward) that rounds at exactly those points
with torch's own conversions.  torch converts float64 to bfloat16 through
float32, which rounds twice; the reference avoids that with round-to-odd into
float32 (the low bit of an inexact result set, after truncation), after which
torch's float32 -> bfloat16 round-to-nearest-even gives the correctly rounded
value (rounding to odd with at least two extra bits, then to nearest, equals
one rounding to nearest: Boldo and Melquiond, IEEE Trans. Computers 57(4),
2008).

* Both sides round correctly at the same points and differ only in float64
  summation order, so the stored logits must be bit-identical.
* Teeth: the same reference with any one rounding point left out gives
  different logits on the two-layer FFN/GQA stack (every point is in play).
* The helper's rounding agrees with the oracle's bf16 rounding on random values
  and on values placed just off bf16 rounding ties.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O
from oracle.rounding import round_bf16
from synth import configs as C
from synth import generators as G

POINTS = ("input", "norm", "qkv", "attn", "residual", "ffn", "logits")


def round_to_odd_f32(x: torch.Tensor) -> torch.Tensor:
    """float64 -> float32, truncated toward zero and made odd when inexact."""
    r = x.to(torch.float32)
    inexact = r.to(torch.float64) != x
    bits = r.view(torch.int32)
    past = inexact & (r.to(torch.float64).abs() > x.abs())    # rounded away from zero
    bits = torch.where(past, bits - 1, bits)                  # one ulp back toward zero
    bits = torch.where(inexact, bits | 1, bits)
    return bits.view(torch.float32)


def store(x: torch.Tensor, dtype: str) -> torch.Tensor:
    if dtype == "f64":
        return x
    if dtype == "f32":
        return x.to(torch.float32).to(torch.float64)
    if dtype == "bf16":
        return round_to_odd_f32(x).to(torch.bfloat16).to(torch.float64)
    raise ValueError(dtype)


def torch_forward_stored(model, tokens, cand, dtype, skip=()):
    """Logits of `cand` from one forward over every position, rounding at each
    storage point not named in `skip`."""
    S = lambda name, v: v if name in skip else store(v, dtype)  # noqa: E731
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))  # noqa: E731
    L = len(tokens)
    Hq, Hkv, dh, d = model.n_q, model.n_kv, model.dh, model.d
    x = S("input", t(model.tok_emb)[torch.from_numpy(np.asarray(tokens))] + t(model.pos_emb)[:L])
    for lw in model.layers:
        a = S("norm", F.rms_norm(x, (d,), weight=t(lw["norm_attn"]), eps=model.eps)) if model.d_ffn else x
        qkv = S("qkv", F.linear(a, t(lw["w_qkv"])))
        q, k, v = qkv.split([Hq * dh, Hkv * dh, Hkv * dh], dim=1)
        q = q.reshape(L, Hq, dh).transpose(0, 1)
        k = k.reshape(L, Hkv, dh).transpose(0, 1)
        v = v.reshape(L, Hkv, dh).transpose(0, 1)
        o = S("attn", F.scaled_dot_product_attention(q, k, v, enable_gqa=True))
        x = S("residual", x + F.linear(o.transpose(0, 1).reshape(L, Hq * dh), t(lw["w_o"])))
        if model.d_ffn:
            a2 = S("norm", F.rms_norm(x, (d,), weight=t(lw["norm_ffn"]), eps=model.eps))
            h = S("ffn", F.silu(F.linear(a2, t(lw["w_gate"]))) * F.linear(a2, t(lw["w_up"])))
            x = S("residual", x + F.linear(h, t(lw["w_down"])))
    if model.d_ffn:
        x = S("norm", F.rms_norm(x, (d,), weight=t(model.norm_final), eps=model.eps))
    c = torch.from_numpy(np.asarray(cand))
    z = F.linear(x[c], t(model.w_lm))
    if model.logit_scale is not None:
        z = z * t(model.logit_scale)[c][:, None]
    return S("logits", z).numpy()


def small_stack():
    return C.scaled(C.LLADA_STACK, name="stack_small_rp", model_n_layers=2, model_d=64,
                    model_n_q_heads=4, model_n_kv_heads=2, model_head_dim=16, model_vocab=300,
                    model_d_ffn=96, prompt_len=40, gen_len=24, block_len=8, k=4)


def small_single():
    return C.scaled(C.LLADA_LAYER, name="layer_small_rp", model_d=64, model_n_q_heads=4,
                    model_n_kv_heads=2, model_head_dim=16, model_vocab=500, prompt_len=48,
                    gen_len=32, block_len=16, k=4)


def vanilla_steps(cfg, dtype, n_steps):
    """(tokens before the step, step trace) for the first tau = -inf steps."""
    w = G.model_weights(cfg)
    model = O.Model.from_arrays(cfg.model, dtype, w)
    toks, masked = G.initial_sequence(cfg)
    st = O.init_state(model, toks, masked)
    out = []
    for bs, bl, n in C.unmask_schedule(cfg)[:n_steps]:
        before = st.tokens.copy()
        out.append((before, O.step(model, st, -math.inf, cfg.k, bs, bl, n)))
    return model, out


@pytest.mark.parametrize("cfg_fn,dtype", [(small_single, "bf16"), (small_stack, "bf16"),
                                          (lambda: C.TINY, "f32")])
def test_stored_logits_equal_a_torch_forward_rounding_at_the_same_points(cfg_fn, dtype):
    cfg = cfg_fn()
    model, steps = vanilla_steps(cfg, dtype, 6)
    for toks, tr in steps:
        want = torch_forward_stored(model, toks, tr.cand, dtype)
        np.testing.assert_array_equal(tr.logits, want)


def test_each_rounding_point_is_pinned():
    cfg = small_stack()
    model, steps = vanilla_steps(cfg, "bf16", 3)
    for point in POINTS:
        gaps = [np.abs(torch_forward_stored(model, toks, tr.cand, "bf16", skip=(point,)) - tr.logits).max()
                for toks, tr in steps]
        assert max(gaps) > 0, point
    # and the storage dtype matters at all: a float64 reference is far off
    toks, tr = steps[0]
    assert np.abs(torch_forward_stored(model, toks, tr.cand, "f64") - tr.logits).max() > 1e-3


def test_round_to_odd_path_rounds_like_the_oracle():
    rng = np.random.default_rng(5)
    x = rng.standard_normal(200000) * np.exp2(rng.integers(-60, 60, 200000))
    # values at and next to bf16 rounding ties: a bf16 value plus half its spacing, nudged
    base = round_bf16(rng.standard_normal(20000))
    half = np.abs(base) * 2.0 ** -9
    ties = np.concatenate([base + half, base - half, base + half * (1 + 2.0 ** -40),
                           base + half * (1 - 2.0 ** -40), base + half * (1 + 2.0 ** -30)])
    for v in (x, ties):
        got = store(torch.from_numpy(v), "bf16").numpy()
        np.testing.assert_array_equal(got, round_bf16(v))
    # plain float64 -> bfloat16 in torch rounds twice and misses some of the nudged ties
    twice = torch.from_numpy(ties).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.any(twice != round_bf16(ties))
