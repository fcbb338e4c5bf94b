"""The 32-layer LLaDA-shaped stack at full size on the GPU.

* A partial step, teacher forced: from a seeded mid-generation state (two
  blocks decoded, the third partly decoded, random K/V caches in every layer)
  the GPU and the oracle each run one step.  A partial step reads every other
  position from the caches (EntropyCache, Chinese summary page §2.2), so
  stale rows feed all 32 layers here.  Checked: rows exact; every layer's
  unselected K/V rows bitwise unchanged; layer 0's refreshed K/V rows (same
  inputs on both sides) within 2e-2; all candidates' logits within the
  propagated tolerance of the single-layer tests; entropy, argmax, unmask
  choice and flag on the GPU's stored logits as in the step tests.
  Deeper layers do not see identical inputs: the residual stream is stored in
  bf16 after every layer, and last-bit rounding differences between the
  GPU's float32 sums and the oracle's float64 sums compound layer by layer.
  Their bound comes from the oracle alone: a second oracle step whose every
  storage rounding is preceded by a random relative perturbation of +-2^-9
  (about half a bf16 unit) drifts from the plain one by what independent
  rounding differences produce.  For every layer >= 1 the GPU's refreshed K/V
  rows must deviate from the oracle by no more than that drift, in RMS and
  in maximum (plus 2e-2), and so must the logits in RMS.  The oracle streams
  the layer weights in float64 one layer at a time.
* Two steps from a fresh sequence (a full step, then a partial one) run free:
  rows equal the oracle's selection from the same state, the decisions are
  checked on the GPU's stored logits, and layer 0's refreshed K/V rows (a
  function of each row's own token and position) match the oracle on a
  sample of rows.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle as O
from entropy_gated_kv_amd.runner import DeviceModel, DeviceSequence
from synth import configs as C
from synth import generators as G
from tests.gpu_helpers import assert_close, host
from tests.step_checks import decisions_on_stored_logits
from tests.test_gpu_step import logit_tol

pytestmark = pytest.mark.gpu


class StreamedLayers:
    """The stack's layer weights in float64, regenerated one layer at a time
    each time the oracle walks the layers (about 1.7 GB per layer)."""

    def __init__(self, cfg):
        self.cfg = cfg

    def __len__(self):
        return self.cfg.model.n_layers

    def __iter__(self):
        m = self.cfg.model
        for l in range(m.n_layers):
            lw = {k: G.layer_weight(self.cfg, l, k).astype(np.float64)
                  for k in ("w_qkv", "w_o", "w_gate", "w_up", "w_down")}
            lw["norm_attn"] = G.norm_gain(self.cfg).astype(np.float64)
            lw["norm_ffn"] = G.norm_gain(self.cfg).astype(np.float64)
            yield lw


def mid_generation_state(cfg, rng):
    """Two blocks decoded, the third with 9 positions decoded; decoded
    positions hold random tokens and enter the history block by block in
    random order within a block."""
    toks, masked = G.initial_sequence(cfg)
    toks, masked = toks.astype(np.int64), masked.astype(bool)
    b0 = cfg.prompt_len
    hist = []
    for b in range(2):
        pos = b0 + b * cfg.block_len + rng.permutation(cfg.block_len)
        hist += [int(p) for p in pos]
    bs = b0 + 2 * cfg.block_len
    hist += [int(p) for p in bs + rng.choice(cfg.block_len, 9, replace=False)]
    toks[hist] = rng.integers(0, cfg.model.vocab, len(hist))
    masked[hist] = False
    return toks, masked, hist, bs


def perturbed_step(model, state, *args, eps=2.0 ** -9, seed=123):
    """The oracle's step with each storage rounding applied to x (1 + eps r),
    r = +-1 at random per element."""
    import importlib
    mod = importlib.import_module("oracle.step")
    real = mod.to_storage
    rng = np.random.default_rng(seed)

    def perturbed(x, dtype):
        x = np.asarray(x, dtype=np.float64)
        return real(x * (1.0 + eps * rng.choice([-1.0, 1.0], size=x.shape)), dtype)

    mod.to_storage = perturbed
    try:
        return O.step(model, state, *args)
    finally:
        mod.to_storage = real


def rms(a):
    return float(np.sqrt(np.mean(np.square(a))))


def test_llada_stack_full_size_partial_step_teacher_forced():
    cfg = C.LLADA_STACK
    m = cfg.model
    tau, n_unmask = cfg.taus[0], 2
    rng = np.random.default_rng(7)
    w = G.model_weights_streamed(cfg)
    dm = DeviceModel(m, cfg.dtype, cfg.L, w)            # consumes the layer generator
    toks, masked, hist, bs = mid_generation_state(cfg, rng)
    ds = DeviceSequence(dm, toks, masked, history_cap=cfg.gen_len, max_block=cfg.block_len)
    K = [G.random_matrix(cfg.seed, (31, l), (m.n_kv_heads, cfg.L, m.head_dim), 1.0, cfg.dtype)
         for l in range(m.n_layers)]
    V = [G.random_matrix(cfg.seed, (32, l), (m.n_kv_heads, cfg.L, m.head_dim), 1.0, cfg.dtype)
         for l in range(m.n_layers)]
    ds.load_state(toks, masked, hist, 0, K, V)
    print("stack: GPU state loaded", flush=True)
    ds.step(tau, cfg.k, bs, cfg.block_len, n_unmask)
    torch.cuda.synchronize()
    model = O.Model(n_layers=m.n_layers, d=m.d, n_q=m.n_q_heads, n_kv=m.n_kv_heads,
                    dh=m.head_dim, V=m.vocab, d_ffn=m.d_ffn, eps=m.rms_eps, dtype=cfg.dtype,
                    tok_emb=np.asarray(w["tok_emb"], dtype=np.float32),
                    pos_emb=np.asarray(w["pos_emb"], dtype=np.float64),
                    layers=StreamedLayers(cfg), w_lm=np.asarray(w["w_lm"], dtype=np.float64),
                    norm_final=np.asarray(w["norm_final"], dtype=np.float64),
                    logit_scale=np.asarray(w["logit_scale"], dtype=np.float64))
    def state():
        return O.State(toks.copy(), masked.copy(), list(hist), 0,
                       [k.astype(np.float64) for k in K], [v.astype(np.float64) for v in V])

    st = state()
    tr = O.step(model, st, tau, cfg.k, bs, cfg.block_len, n_unmask)
    print(f"stack: oracle step done, {len(tr.rows)} rows, {len(tr.cand)} candidates", flush=True)
    sp = state()
    tp = perturbed_step(model, sp, tau, cfg.k, bs, cfg.block_len, n_unmask)
    print("stack: perturbed oracle step done", flush=True)
    n = int(ds.n_rows.item())
    assert len(tr.rows) == 23 + cfg.k
    np.testing.assert_array_equal(ds.rows[:n].cpu().numpy(), tr.rows)
    keep = np.setdiff1d(np.arange(cfg.L), tr.rows)
    for l in range(m.n_layers):
        k, v = ds.caches(l)
        assert np.array_equal(k[:, keep], K[l][:, keep]) and np.array_equal(v[:, keep], V[l][:, keep])
        for name, got, want, pert in (("K", k, st.K[l], sp.K[l]), ("V", v, st.V[l], sp.V[l])):
            got, want, pert = got[:, tr.rows], want[:, tr.rows], pert[:, tr.rows]
            if l == 0:
                assert_close(got, want, "bf16", f"layer 0 {name} rows")
                continue
            e, d = got - want, pert - want
            print(f"stack layer {l:2d} {name}: rms {rms(e) / rms(want):.4f} (drift {rms(d) / rms(want):.4f}), "
                  f"max {np.abs(e).max():.3f} (drift {np.abs(d).max():.3f})", flush=True)
            assert rms(e) <= rms(d), (l, name, rms(e), rms(d))
            assert np.abs(e).max() <= np.abs(d).max() + 2e-2, (l, name)
    mc = len(tr.cand)
    g = {"logits": host(ds.logits[:mc]), "H": ds.row_entropy[:mc].cpu().numpy(),
         "argmax": ds.row_argmax[:mc].cpu().numpy(), "p1": ds.row_top1[:mc].cpu().numpy(),
         "chosen": ds.chosen[: int(ds.n_chosen.item())].cpu().numpy(),
         "E": float(ds.e_max.item()), "flag": int(ds.full_flag.item())}
    tol = logit_tol(model, tr)
    err = np.abs(g["logits"] - tr.logits)
    assert np.all(err <= tol), float((err / tol).max())
    assert rms(g["logits"] - tr.logits) <= rms(tp.logits - tr.logits)
    decisions_on_stored_logits(g, tr.cand, n_unmask, tau, "stack partial step")
    print(f"stack: worst logit error / tolerance {float((err / tol).max()):.3f}", flush=True)


def test_llada_stack_full_size_two_steps():
    cfg = C.LLADA_STACK
    tau = cfg.taus[0]
    w = G.model_weights_streamed(cfg)
    layer0 = {}

    def keep_first(gen):
        for i, lw in enumerate(gen):
            if i == 0:
                layer0.update(lw)
            yield lw

    w["layers"] = keep_first(w["layers"])
    dm = DeviceModel(cfg.model, cfg.dtype, cfg.L, w)
    toks, masked = G.initial_sequence(cfg)
    ds = DeviceSequence(dm, toks, masked, history_cap=cfg.gen_len, max_block=cfg.block_len)
    one = dataclasses.replace(cfg.model, n_layers=1)
    m1 = O.Model.from_arrays(one, cfg.dtype, {"tok_emb": w["tok_emb"], "pos_emb": w["pos_emb"],
                                              "w_lm": None, "norm_final": w["norm_final"],
                                              "layers": [layer0]})
    rng = np.random.default_rng(3)
    for i, (bs, bl, n) in enumerate(C.unmask_schedule(cfg)[:2]):
        tokens0 = ds.tokens.cpu().numpy().astype(np.int64)
        masked0 = ds.is_masked.cpu().numpy().astype(bool)
        hist0 = ds.history[: int(ds.history_len.item())].cpu().numpy().tolist()
        flag0 = int(ds.full_flag.item())
        ds.step(tau, cfg.k, bs, bl, n)
        torch.cuda.synchronize()
        rows = ds.rows[: int(ds.n_rows.item())].cpu().numpy()
        np.testing.assert_array_equal(rows, O.select_rows(flag0, masked0, bs, bl, hist0, cfg.k))
        cand = O.candidates(masked0, bs, bl)
        chosen = ds.chosen[: int(ds.n_chosen.item())].cpu().numpy()
        assert len(chosen) == min(n, len(cand)) and np.all(np.isin(chosen, cand))
        assert np.all(np.diff(chosen) > 0)
        pick = np.searchsorted(cand, chosen)
        H = ds.row_entropy[: len(cand)].cpu().numpy()
        A = ds.row_argmax[: len(cand)].cpu().numpy()
        tokens1 = ds.tokens.cpu().numpy()
        assert np.array_equal(tokens1[chosen], A[pick])
        assert not ds.is_masked.cpu().numpy()[chosen].any()
        hist1 = ds.history[: int(ds.history_len.item())].cpu().numpy().tolist()
        assert hist1 == hist0 + chosen.tolist()
        E = float(ds.e_max.item())
        assert math.isfinite(E)
        g = {"logits": host(ds.logits[: len(cand)]), "H": H, "argmax": A,
             "p1": ds.row_top1[: len(cand)].cpu().numpy(), "chosen": chosen, "E": E,
             "flag": int(ds.full_flag.item())}
        decisions_on_stored_logits(g, cand, n, tau, f"stack step {i}")
        # layer 0's refreshed rows, on a sample
        st = O.init_state(m1, tokens0, masked0)
        sample = np.unique(np.concatenate([rng.choice(rows, min(24, len(rows)), replace=False),
                                           [rows[0], rows[-1]]]))
        O.forward_rows(m1, st, sample)
        k, v = ds.caches(0)
        assert_close(k[:, sample], st.K[0][:, sample], "bf16", f"step {i} layer-0 K rows")
        assert_close(v[:, sample], st.V[0][:, sample], "bf16", f"step {i} layer-0 V rows")
