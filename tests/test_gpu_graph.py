"""ec_step under HIP graph capture: several steps captured into one graph and
replayed three times (the state restored by eager copies, with eager work and
synchronisation between replays) reproduce the eager trajectory bit for bit.
The step records no memset and never synchronises, so it captures as is.
Cases: the tiny fp32 layer, a two-layer bf16 stack, and a one-layer bf16
model stepping without a logits buffer (its packed LM head writes softmax
statistics that the step folds)."""
import numpy as np
import pytest
import torch

from entropy_gated_kv_amd.runner import DeviceModel, DeviceSequence
from synth import configs as C
from synth import generators as G

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cfg_name", ["tiny_fp32", "stack_bf16", "no_logits_bf16"])
def test_captured_steps_replay_like_eager(cfg_name):
    keep_logits = True
    if cfg_name == "tiny_fp32":
        cfg, tau = C.TINY, float("inf")
    elif cfg_name == "no_logits_bf16":
        cfg = C.scaled(C.LLADA_LAYER, name="no_logits_graph", model_d=256, model_n_q_heads=2,
                       model_n_kv_heads=2, model_vocab=40032, prompt_len=96, gen_len=64, block_len=32, k=16)
        tau, keep_logits = 1.0, False
    else:
        cfg = C.scaled(C.LLADA_STACK, name="stack_graph", model_n_layers=2, model_d=256,
                       model_n_q_heads=4, model_n_kv_heads=2, model_head_dim=64, model_vocab=2048,
                       model_d_ffn=512, prompt_len=96, gen_len=64, block_len=32, k=16)
        tau = 1.0
    w = G.model_weights(cfg)
    toks, masked = G.initial_sequence(cfg)
    dm = DeviceModel(cfg.model, cfg.dtype, cfg.L, w)
    ds = DeviceSequence(dm, toks, masked, history_cap=cfg.gen_len, max_block=cfg.block_len,
                        keep_logits=keep_logits)
    sched = C.unmask_schedule(cfg)
    state = lambda: [ds.tokens, ds.is_masked, ds.history, ds.history_len, ds.full_flag,
                     *ds.k_cache, *ds.v_cache]
    for bs, bl, n in sched[:2]:                  # a full step first, then the cache exists
        ds.step(tau, cfg.k, bs, bl, n)
    torch.cuda.synchronize()
    start = [t.clone() for t in state()]
    steps = sched[2:8]

    def outputs():
        out = [ds.row_entropy.clone(), ds.row_top1.clone(), ds.row_argmax.clone(), ds.e_max.clone()]
        return [t.clone() for t in state()] + out + ([ds.logits.clone()] if keep_logits else [])

    for bs, bl, n in steps:                      # the eager reference
        ds.step(tau, cfg.k, bs, bl, n)
    torch.cuda.synchronize()
    ref = outputs()

    def restore():
        for d, s in zip(state(), start):
            d.copy_(s)

    restore()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for bs, bl, n in steps:
            ds.step(tau, cfg.k, bs, bl, n)
    torch.cuda.synchronize()
    for rep in range(3):
        restore()
        junk = torch.randn(1 << 16, device="cuda").sum()    # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = outputs()
        for i, (a, b) in enumerate(zip(ref, got)):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), (rep, i)
        del junk
