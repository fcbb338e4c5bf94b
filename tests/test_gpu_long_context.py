"""GPU parity of the steady-state long-context step (ec_step without LM head).

The Dream-shaped layer (d = 3584, 28 query / 4 KV heads of 128) runs the step
with external decoding: each step's decision comes from two synthetic decoded
rows of V = 152064 (flat on every 8th step, peaked otherwise), so a full step
follows each flat step and the other steps recompute the fixed 96 rows (the
masked block of 32 plus the 64 history positions before it).

* A shortened prefix (L = 1024 + 32): prefill plus 17 steps run free on the
  GPU and must match the oracle's trajectory: rows and flags exactly, E within
  1e-4 relative (both sides read the same bf16 logits), caches within 2e-2.
* Full size (L = 8224 and 32800): one partial step, teacher forced from a
  seeded cache, against the oracle (rows exact, refreshed rows within 2e-2,
  every other cache row bitwise unchanged, every one of the step's 96 x 28 x
  128 attention outputs within 2e-2, E and flag); and one full step, whose
  refreshed cache rows are checked on a sample the oracle computes one by one
  (a row's K/V depend only on its own input).  The seeded K cache has
  standard deviation 2, so with the model's queries (standard deviation about
  1.7) the scores spread by about 3.4 and the attention outputs are of order
  0.1-1, well above the tolerance floor: a wrong split merge shows.
"""
import numpy as np
import pytest
import torch

import oracle as O
from entropy_gated_kv_amd.runner import DeviceModel, DeviceSequence, to_device
from synth import configs as C
from synth import generators as G
from tests.gpu_helpers import assert_close, host

pytestmark = pytest.mark.gpu


def short_cfg():
    return C.scaled(C.DREAM_8K, name="dream_short", prefix_len=1024)


_TOK = {}


def token_table(cfg):
    """tok_emb(cfg), generated once per (seed, vocab, width): about 545M values."""
    key = (cfg.seed, cfg.model.vocab, cfg.model.d)
    if key not in _TOK:
        _TOK.clear()
        _TOK[key] = G.tok_emb(cfg)
    return _TOK[key]


def setup(cfg):
    w = G.model_weights(cfg, tok_table=token_table(cfg))
    model = O.Model.from_arrays(cfg.model, cfg.dtype, w)
    toks, masked = G.initial_sequence(cfg)
    st = O.init_state(model, toks, masked)
    st.history = [int(p) for p in G.long_context_history(cfg)]
    dm = DeviceModel(cfg.model, cfg.dtype, cfg.L, w)
    ds = DeviceSequence(dm, toks, masked, history_cap=cfg.k, max_block=cfg.block_len)
    ds.load_state(toks, masked, st.history, 1)
    return model, st, ds


def decision(cfg, t):
    z = G.decision_logits(cfg, t)
    return z, to_device(z, cfg.dtype)


def test_short_prefix_trajectory_free_running():
    cfg = short_cfg()
    model, st, ds = setup(cfg)
    for t in range(18):
        z, zd = decision(cfg, t)
        tr = O.step_external(model, st, cfg.tau, cfg.k, cfg.prefix_len, cfg.block_len, z)
        ds.step_external(cfg.tau, cfg.k, cfg.prefix_len, cfg.block_len, zd)
        torch.cuda.synchronize()
        n = int(ds.n_rows.item())
        np.testing.assert_array_equal(ds.rows[:n].cpu().numpy(), tr.rows, err_msg=f"step {t}")
        E = float(ds.e_max.item())
        assert abs(E - tr.E) <= 1e-4 * max(1.0, abs(tr.E)), (t, E, tr.E)
        assert int(ds.full_flag.item()) == tr.flag_next, t
        np.testing.assert_allclose(ds.row_entropy[:2].cpu().numpy(), tr.H, rtol=1e-4, atol=1e-5)
    k, v = ds.caches(0)
    assert_close(k, st.K[0], "bf16", "K cache")
    assert_close(v, st.V[0], "bf16", "V cache")


def seeded_caches(cfg, k_std=1.0):
    m = cfg.model
    K = G.random_matrix(cfg.seed, (21,), (m.n_kv_heads, cfg.L, m.head_dim), k_std, cfg.dtype)
    V = G.random_matrix(cfg.seed, (22,), (m.n_kv_heads, cfg.L, m.head_dim), 1.0, cfg.dtype)
    return K.astype(np.float64), V.astype(np.float64)


@pytest.mark.parametrize("cfg", [C.DREAM_8K, C.DREAM_32K], ids=["L8224", "L32800"])
def test_full_size_partial_step(cfg):
    model, st, ds = setup(cfg)
    K, V = seeded_caches(cfg, k_std=2.0)
    st.K, st.V, st.flag = [K.copy()], [V.copy()], 0
    ds.load_state(st.tokens, st.masked, st.history, 0, [K], [V])
    ds.enable_attn_out()
    z, zd = decision(cfg, 3)
    before = st.copy()
    tr = O.step_external(model, st, cfg.tau, cfg.k, cfg.prefix_len, cfg.block_len, z)
    ds.step_external(cfg.tau, cfg.k, cfg.prefix_len, cfg.block_len, zd)
    torch.cuda.synchronize()
    n = int(ds.n_rows.item())
    assert n == cfg.block_len + cfg.k
    np.testing.assert_array_equal(ds.rows[:n].cpu().numpy(), tr.rows)
    attn = []
    O.forward_rows(model, before, tr.rows, attn=attn)
    want = attn[-1]
    assert np.abs(want).mean() > 0.1
    assert_close(host(ds.attn_out[:n]), want, "bf16", "step attention output")
    k, v = ds.caches(0)
    assert_close(k[:, tr.rows], st.K[0][:, tr.rows], "bf16", "refreshed K rows")
    assert_close(v[:, tr.rows], st.V[0][:, tr.rows], "bf16", "refreshed V rows")
    keep = np.setdiff1d(np.arange(cfg.L), tr.rows)
    assert np.array_equal(k[:, keep], K[:, keep]) and np.array_equal(v[:, keep], V[:, keep])
    assert abs(float(ds.e_max.item()) - tr.E) <= 1e-4 * max(1.0, abs(tr.E))
    assert int(ds.full_flag.item()) == tr.flag_next == 0


@pytest.mark.parametrize("cfg", [C.DREAM_8K, C.DREAM_32K], ids=["L8224", "L32800"])
def test_full_size_full_step_sampled(cfg):
    model, st, ds = setup(cfg)
    z, zd = decision(cfg, 7)                     # a flat row: the next step is full again
    ds.step_external(cfg.tau, cfg.k, cfg.prefix_len, cfg.block_len, zd)
    torch.cuda.synchronize()
    n = int(ds.n_rows.item())
    assert n == cfg.L
    np.testing.assert_array_equal(ds.rows[:n].cpu().numpy(), np.arange(cfg.L))
    assert int(ds.full_flag.item()) == 1
    k, v = ds.caches(0)
    rng = np.random.default_rng(2)
    sample = np.unique(np.concatenate([rng.integers(0, cfg.L, 40), [0, cfg.L - 1],
                                       np.arange(cfg.prefix_len - 2, cfg.prefix_len + 2)]))
    O.forward_rows(model, st, sample)            # refreshes exactly these rows' K/V
    assert_close(k[:, sample], st.K[0][:, sample], "bf16", "sampled K rows")
    assert_close(v[:, sample], st.V[0][:, sample], "bf16", "sampled V rows")
