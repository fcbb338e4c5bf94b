"""The LM head's packed weight layout (ec_pack_lm_head) on the GPU.

* The packed buffer equals the layout ec.h documents, built here on the host
  from its definition: for each group of 16 rows, the d / 32 blocks of
  16 rows x 32 columns in column order, entry (row n, columns 8g .. 8g + 7)
  of a block being its 16-byte chunk 16 g + n.
* Steps whose LM head reads the packed copy give the same bits as steps that
  read w_lm (logits, entropies, decisions, tokens), on the LLaDA-shaped layer
  at full size (V = 126464), and on one-layer models whose vocabulary sizes
  reach each launch shape of the packed LM head on a 256-CU part with three
  resident workgroups per CU: single tiles one per workgroup, pairs, triples
  (with a short last group that repeats a tile) and single tiles on a
  persistent grid; ragged last tiles (V % 64 = 32) and d = 256, 512, 768
  (one, two, three k-blocks).
"""
import numpy as np
import pytest
import torch

from entropy_gated_kv_amd import lib as L
from entropy_gated_kv_amd.runner import DeviceModel, DeviceSequence
from synth import configs as C
from synth import generators as G

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


def steps_bit_identical(cfg):
    w = G.model_weights(cfg)
    toks, masked = G.initial_sequence(cfg)
    packed = DeviceModel(cfg.model, cfg.dtype, cfg.L, w, pack_lm_head=True)
    plain = DeviceModel(cfg.model, cfg.dtype, cfg.L, w, pack_lm_head=False)
    assert packed.w_lm_packed is not None and plain.w_lm_packed is None
    seqs = [DeviceSequence(m, toks, masked, history_cap=cfg.gen_len, max_block=cfg.block_len)
            for m in (packed, plain)]
    for i, (bs, bl, n) in enumerate(C.unmask_schedule(cfg)[:6]):
        for s in seqs:
            s.step(1.0, cfg.k, bs, bl, n)
        torch.cuda.synchronize()
        a, b = seqs
        m = bl
        assert torch.equal(a.logits[:m].view(torch.int16), b.logits[:m].view(torch.int16)), i
        for f in ("row_entropy", "row_top1", "row_argmax", "tokens", "is_masked", "full_flag",
                  "e_max", "chosen", "n_chosen"):
            assert torch.equal(getattr(a, f), getattr(b, f)), (i, f)


def test_packed_lm_head_steps_are_bit_identical():
    steps_bit_identical(C.LLADA_LAYER)


# (V, d): column tiles of 64 and the launch shape they get
@pytest.mark.parametrize("V,d", [(40032, 256),     # 626 tiles: one per workgroup
                                 (65568, 512),     # 1025 tiles: pairs, the last pair repeats a tile
                                 (128032, 768),    # 2001 tiles: triples
                                 (160032, 256)],   # 2501 tiles: single tiles, persistent grid
                         ids=["single", "pairs", "triples", "persistent"])
def test_packed_lm_head_launch_shapes_are_bit_identical(V, d):
    heads = d // 128
    steps_bit_identical(C.scaled(C.LLADA_LAYER, model_vocab=V, model_d=d, model_n_q_heads=heads,
                                 model_n_kv_heads=heads))
