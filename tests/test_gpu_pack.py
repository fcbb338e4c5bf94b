"""The LM head's packed weight layout (ec_pack_lm_head) on the GPU.

* The packed buffer equals the layout ec.h documents, built here on the host
  from its definition: for each group of 16 rows, the d / 32 blocks of
  16 rows x 32 columns in column order, entry (row n, columns 8g .. 8g + 7)
  of a block being its 16-byte chunk 16 g + n.
* Steps whose LM head reads the packed copy give the same bits as steps that
  read w_lm (logits, entropies, decisions, tokens).
* Steps without a logits buffer, where the packed LM head writes each row's
  softmax statistics per group of column tiles and the step folds those,
  are checked against the oracle run on the logits their twin with a buffer
  stored (tests/step_checks.py: H within 1e-4 + 1e-5 H, argmax exact, p1
  within its float32 bound, unmask set, E and flag with the step tests' tie
  zones).  Their decisions must equal the twin's unless one fell in such a
  tie zone, after which the trajectories may differ and that comparison
  stops.
* Cases: the LLaDA-shaped layer at full size (V = 126464), and one-layer
  models whose vocabulary sizes reach each launch shape of the packed LM head
  on a 256-CU part: one, two, three (with a short last group that repeats a
  tile) and four column tiles per workgroup; ragged last tiles (V % 64 = 32)
  and d = 256, 512, 768 (one, two, three k-blocks).
"""
import math

import numpy as np
import pytest
import torch

import oracle as O

from entropy_gated_kv_amd import lib as L
from entropy_gated_kv_amd.runner import DeviceModel, DeviceSequence
from synth import configs as C
from synth import generators as G
from tests.step_checks import decisions_on_stored_logits

pytestmark = pytest.mark.gpu


def host_pack(w):
    """The documented layout, as int16 bit patterns ([V, d] -> flat)."""
    V, d = w.shape
    chunks = w.reshape(V // 16, 16, d // 32, 4, 8)          # [group, n, block, g, 8]
    return chunks.transpose(0, 2, 3, 1, 4).reshape(-1)      # [group, block, g, n, 8]


@pytest.mark.parametrize("V,d", [(16, 32), (256, 512), (4096, 4096)])
def test_packed_layout(V, d):
    w = torch.randint(-30000, 30000, (V, d), dtype=torch.int16, device="cuda").view(torch.bfloat16)
    out = torch.full((V, d), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    L.ec_pack_lm_head(w, out)
    torch.cuda.synchronize()
    want = host_pack(w.view(torch.int16).cpu().numpy())
    np.testing.assert_array_equal(out.view(torch.int16).cpu().numpy().reshape(-1), want)


TAU = 1.0


def step_outputs(s, logits, m):
    nc = int(s.n_chosen.item())
    return {"logits": logits[:m].float().cpu().numpy(), "H": s.row_entropy[:m].cpu().numpy(),
            "argmax": s.row_argmax[:m].cpu().numpy(), "p1": s.row_top1[:m].cpu().numpy(),
            "chosen": s.chosen[:nc].cpu().numpy(), "E": float(s.e_max.item()),
            "flag": int(s.full_flag.item())}


DECISIONS = ("tokens", "is_masked", "chosen", "n_chosen", "full_flag")


def steps_agree(cfg):
    w = G.model_weights(cfg)
    toks, masked = G.initial_sequence(cfg)
    packed = DeviceModel(cfg.model, cfg.dtype, cfg.L, w, pack_lm_head=True)
    plain = DeviceModel(cfg.model, cfg.dtype, cfg.L, w, pack_lm_head=False)
    assert packed.w_lm_packed is not None and plain.w_lm_packed is None
    mk = lambda m, keep: DeviceSequence(m, toks, masked, history_cap=cfg.gen_len, max_block=cfg.block_len,
                                        keep_logits=keep)
    a, b, f = mk(packed, True), mk(plain, True), mk(packed, False)
    assert f.logits is None
    fused_on = True
    for i, (bs, bl, n) in enumerate(C.unmask_schedule(cfg)[:6]):
        cand = bs + np.flatnonzero(a.is_masked[bs:bs + bl].cpu().numpy())   # this step's candidates
        for s in (a, b, f) if fused_on else (a, b):
            s.step(TAU, cfg.k, bs, bl, n)
        torch.cuda.synchronize()
        assert torch.equal(a.logits[:bl].view(torch.int16), b.logits[:bl].view(torch.int16)), i
        for fld in ("row_entropy", "row_top1", "row_argmax", "e_max") + DECISIONS:
            assert torch.equal(getattr(a, fld), getattr(b, fld)), (i, fld)
        ties = decisions_on_stored_logits(step_outputs(a, a.logits, len(cand)), cand, n, TAU,
                                          f"{cfg.name} packed step {i}")
        if not fused_on:
            continue
        ties += decisions_on_stored_logits(step_outputs(f, a.logits, len(cand)), cand, n, TAU,
                                           f"{cfg.name} no-logits step {i}")
        if not all(torch.equal(getattr(a, fld), getattr(f, fld)) for fld in DECISIONS):
            # the statistics' float32 sums may order a near-tie differently;
            # past it the trajectories differ
            assert ties > 0, i
            fused_on = False


def test_packed_lm_head_steps_agree():
    steps_agree(C.LLADA_LAYER)


# (V, d): column tiles of 64 and the launch shape they get
@pytest.mark.parametrize("V,d", [(40032, 256),     # 626 tiles: one per workgroup
                                 (65568, 512),     # 1025 tiles: pairs, the last pair repeats a tile
                                 (128032, 768),    # 2001 tiles: triples
                                 (160032, 256)],   # 2501 tiles: groups of four
                         ids=["single", "pairs", "triples", "quads"])
def test_packed_lm_head_launch_shapes_agree(V, d):
    heads = d // 128
    steps_agree(C.scaled(C.LLADA_LAYER, model_vocab=V, model_d=d, model_n_q_heads=heads,
                                 model_n_kv_heads=heads))


def test_packed_lm_head_stack_agrees():
    """A two-layer RMSNorm / SwiGLU stack (the LM head reads the final norm's
    output): the three twins as above."""
    steps_agree(C.scaled(C.LLADA_STACK, name="stack2_pack", model_n_layers=2, model_d=256,
                         model_n_q_heads=2, model_n_kv_heads=2, model_d_ffn=512, model_vocab=40032,
                         prompt_len=96, gen_len=64, block_len=32, k=16))


def test_no_logits_with_a_workspace_for_longer_blocks():
    """Steps without a logits buffer on a sequence whose buffers and workspace
    are sized for blocks of 64 give the same bits as on one sized for 32."""
    cfg = C.scaled(C.LLADA_LAYER, name="ws64", model_d=256, model_n_q_heads=2, model_n_kv_heads=2,
                   model_vocab=40032, prompt_len=96, gen_len=64, block_len=32, k=16)
    w = G.model_weights(cfg)
    toks, masked = G.initial_sequence(cfg)
    dm = DeviceModel(cfg.model, cfg.dtype, cfg.L, w, pack_lm_head=True)
    a, b = [DeviceSequence(dm, toks, masked, history_cap=cfg.gen_len, max_block=mb, keep_logits=False)
            for mb in (32, 64)]
    for i, (bs, bl, n) in enumerate(C.unmask_schedule(cfg)[:6]):
        for s in (a, b):
            s.step(TAU, cfg.k, bs, bl, n)
        torch.cuda.synchronize()
        for fld in ("row_entropy", "row_top1", "row_argmax", "e_max", "tokens", "is_masked", "chosen",
                    "n_chosen", "full_flag"):
            x, y = getattr(a, fld), getattr(b, fld)
            m = min(x.numel(), y.numel())
            assert torch.equal(x.flatten()[:m].view(torch.uint8) if x.dtype == torch.float32 else x.flatten()[:m],
                               y.flatten()[:m].view(torch.uint8) if y.dtype == torch.float32 else y.flatten()[:m]), (i, fld)


def test_non_finite_and_constant_rows_in_both_modes():
    """Candidate rows whose logits hold +-inf or NaN (a logit scale of +inf,
    -inf or NaN; 3e38 overflows some of a row) take the exact statistics path of the LM head's
    epilogue, and a scale of 0 gives a row of zeros with H = ln V, p1 = 1/V
    and argmax 0.  One full step decodes every candidate, with and without a
    logits buffer: H is NaN exactly where the oracle's is (rows holding NaN
    or +inf), finite rows within the step tests' bounds, argmax exact, and E
    = NaN forces the next step full."""
    cfg = C.scaled(C.LLADA_LAYER, name="non_finite", model_d=256, model_n_q_heads=2, model_n_kv_heads=2,
                   model_vocab=40032, prompt_len=96, gen_len=64, block_len=32, k=16)
    V = cfg.model.vocab
    w = G.model_weights(cfg)
    toks, masked = G.initial_sequence(cfg)
    dm = DeviceModel(cfg.model, cfg.dtype, cfg.L, w, pack_lm_head=True)
    bs, bl = cfg.prompt_len, cfg.block_len
    special = {bs + 1: 0.0, bs + 5: math.inf, bs + 9: -math.inf, bs + 13: math.nan, bs + 17: 3e38}
    for pos, v in special.items():
        dm.logit_scale[pos] = v
    a, f = [DeviceSequence(dm, toks, masked, history_cap=cfg.gen_len, max_block=bl, keep_logits=k)
            for k in (True, False)]
    cand = bs + np.flatnonzero(np.asarray(masked[bs:bs + bl], dtype=bool))
    assert len(cand) == bl
    for s in (a, f):
        s.step(TAU, cfg.k, bs, bl, bl)
    torch.cuda.synchronize()
    z = a.logits[:bl].float().cpu().numpy().astype(np.float64)
    Ho, Ao, Po = O.row_stats(z)
    iz = int(np.searchsorted(cand, bs + 1))
    assert np.all(z[iz] == 0) and Ao[iz] == 0 and abs(Ho[iz] - math.log(V)) < 1e-9
    nan = np.isnan(Ho)
    assert nan[[int(np.searchsorted(cand, p)) for p in (bs + 5, bs + 9, bs + 13)]].all()
    shift = 2.0 ** -23 * np.where(np.isfinite(z), np.abs(z), 0.0).max(axis=1) * 1.4426950408889634
    for s, name in ((a, "logits"), (f, "statistics")):
        H, A, P = (s.row_entropy[:bl].cpu().numpy(), s.row_argmax[:bl].cpu().numpy(),
                   s.row_top1[:bl].cpu().numpy())
        np.testing.assert_array_equal(np.isnan(H), nan, err_msg=name)
        assert np.all(np.abs(H[~nan] - Ho[~nan]) <= 1e-4 + 1e-5 * np.abs(Ho[~nan])), name
        np.testing.assert_array_equal(A, Ao, err_msg=name)
        np.testing.assert_array_equal(np.isnan(P), np.isnan(Po), err_msg=name)
        ok = ~np.isnan(Po)
        assert np.all(np.abs(P[ok] - Po[ok]) <= (1e-5 + shift[ok]) * Po[ok]), name
        assert abs(P[iz] - 1.0 / V) <= 1e-6 / V, name
        assert math.isnan(float(s.e_max.item())) and int(s.full_flag.item()) == 1, name
        assert int(s.n_chosen.item()) == bl, name
        np.testing.assert_array_equal(s.chosen[:bl].cpu().numpy(), cand, err_msg=name)
