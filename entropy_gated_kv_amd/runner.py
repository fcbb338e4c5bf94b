"""Device buffers for one model and one sequence, and a step loop over ec_step.

Argument marshalling only: this module allocates torch tensors, fills the
ec_model / ec_state structs with their addresses and calls the C entry point.
Every step of the computation runs inside libec.so.
"""
from __future__ import annotations

import ctypes as C
from typing import Dict, List, Optional, Sequence

import numpy as np

from . import lib as L


def _torch_dtype(dtype: str):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]


def to_device(a: np.ndarray, dtype: str):
    """Upload a float32 array (holding values exact in `dtype`) as a device tensor."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(_torch_dtype(dtype)).cuda()


class DeviceModel:
    """Weights in HBM plus the ec_model struct that points at them.

    pack_lm_head: for a bf16 LM head with V % 16 == 0, also keep the copy that
    ec_pack_lm_head lays out for streaming (the LM head then reads it)."""

    def __init__(self, shape, dtype: str, L_cap: int, weights: Dict[str, object],
                 pack_lm_head: bool = True):
        import torch
        self.shape, self.dtype, self.L_cap = shape, dtype, L_cap
        self.code = L.EC_BF16 if dtype == "bf16" else L.EC_F32
        up = lambda a: None if a is None else to_device(a, dtype)  # noqa: E731
        self.tok_emb = up(weights["tok_emb"])
        pos = np.zeros((L_cap, shape.d), dtype=np.float32)
        pos[: weights["pos_emb"].shape[0]] = weights["pos_emb"]
        self.pos_emb = up(pos)
        self.w_lm = up(weights.get("w_lm"))          # None: no LM head (the caller decodes)
        self.norm_final = up(weights.get("norm_final"))
        ls = weights.get("logit_scale")
        self.logit_scale = None
        if ls is not None:
            buf = np.ones(L_cap, dtype=np.float32)
            buf[: len(ls)] = ls
            self.logit_scale = torch.from_numpy(buf).cuda()
        self.layers = []
        for lw in weights["layers"]:
            self.layers.append({k: up(v) for k, v in lw.items()})
        self._layer_arr = (L.ec_layer * len(self.layers))()
        for i, lw in enumerate(self.layers):
            ptr = lambda k: None if lw.get(k) is None else lw[k].data_ptr()  # noqa: E731
            self._layer_arr[i] = L.ec_layer(ptr("w_qkv"), ptr("w_o"), ptr("norm_attn"),
                                            ptr("norm_ffn"), ptr("w_gate"), ptr("w_up"),
                                            ptr("w_down"))
        m = L.ec_model()
        m.n_layers, m.d, m.Hq, m.Hkv = len(self.layers), shape.d, shape.n_q_heads, shape.n_kv_heads
        m.dh, m.d_ffn, m.V, m.L_cap, m.dtype = shape.head_dim, shape.d_ffn, shape.vocab, L_cap, self.code
        m.rms_eps = shape.rms_eps
        m.tok_emb, m.pos_emb = self.tok_emb.data_ptr(), self.pos_emb.data_ptr()
        m.layers = C.cast(self._layer_arr, C.POINTER(L.ec_layer))
        m.norm_final = None if self.norm_final is None else self.norm_final.data_ptr()
        m.w_lm = None if self.w_lm is None else self.w_lm.data_ptr()
        m.logit_scale = None if self.logit_scale is None else self.logit_scale.data_ptr()
        self.w_lm_packed = None
        if (pack_lm_head and self.w_lm is not None and dtype == "bf16" and shape.vocab % 16 == 0
                and shape.d % 32 == 0):
            self.w_lm_packed = torch.empty_like(self.w_lm)
            L.ec_pack_lm_head(self.w_lm, self.w_lm_packed)
            torch.cuda.synchronize()
        m.w_lm_packed = None if self.w_lm_packed is None else self.w_lm_packed.data_ptr()
        self.struct = m


class DeviceSequence:
    """Per-sequence device state (tokens, mask, history, flag, KV caches, step outputs)."""

    def __init__(self, model: DeviceModel, tokens: np.ndarray, masked: np.ndarray,
                 history_cap: int, max_block: int, ws=None, keep_logits: bool = True):
        import torch
        sh = model.shape
        self.model, self.L, self.max_block = model, len(tokens), max_block
        dev = "cuda"
        i32 = torch.int32
        self.tokens = torch.tensor(np.asarray(tokens, dtype=np.int32), device=dev)
        self.is_masked = torch.tensor(np.asarray(masked, dtype=np.uint8), device=dev)
        self.history = torch.full((history_cap,), -1, dtype=i32, device=dev)
        self.history_len = torch.zeros(1, dtype=i32, device=dev)
        self.full_flag = torch.ones(1, dtype=i32, device=dev)
        td = _torch_dtype(model.dtype)
        self.k_cache = [torch.zeros((sh.n_kv_heads, model.L_cap, sh.head_dim), dtype=td, device=dev)
                        for _ in range(sh.n_layers)]
        self.v_cache = [torch.zeros((sh.n_kv_heads, sh.head_dim, model.L_cap), dtype=td, device=dev)
                        for _ in range(sh.n_layers)]
        self.rows = torch.zeros(model.L_cap, dtype=i32, device=dev)
        self.n_rows = torch.zeros(1, dtype=i32, device=dev)
        # keep_logits=False: no logits buffer (a packed LM head then writes
        # softmax statistics instead, see ec.h); self.logits is None
        self.logits = torch.zeros((max_block, sh.vocab), dtype=td, device=dev) if keep_logits else None
        self.row_entropy = torch.zeros(max_block, dtype=torch.float32, device=dev)
        self.row_argmax = torch.zeros(max_block, dtype=i32, device=dev)
        self.row_top1 = torch.zeros(max_block, dtype=torch.float32, device=dev)
        self.chosen = torch.zeros(max_block, dtype=i32, device=dev)
        self.n_chosen = torch.zeros(1, dtype=i32, device=dev)
        self.e_max = torch.zeros(1, dtype=torch.float32, device=dev)
        self.kv_drift = None                      # enable_drift(): [n_layers, 2] on full steps
        nbytes = L.ec_step_workspace_bytes(model.struct, max_block)
        if nbytes == 0:
            raise RuntimeError("ec_step_workspace_bytes rejected the model shape")
        # the workspace is scratch: sequences whose steps run one after another
        # on one stream may share it
        if ws is not None and ws.numel() * ws.element_size() < nbytes:
            raise ValueError("shared workspace too small")
        self.ws = torch.zeros(nbytes, dtype=torch.uint8, device=dev) if ws is None else ws
        self._k_arr = (C.c_void_p * sh.n_layers)(*[t.data_ptr() for t in self.k_cache])
        self._v_arr = (C.c_void_p * sh.n_layers)(*[t.data_ptr() for t in self.v_cache])
        s = L.ec_state()
        s.L, s.tokens, s.is_masked = self.L, self.tokens.data_ptr(), self.is_masked.data_ptr()
        s.history, s.history_len, s.history_cap = (self.history.data_ptr(),
                                                   self.history_len.data_ptr(), history_cap)
        s.full_flag = self.full_flag.data_ptr()
        s.k_cache = C.cast(self._k_arr, C.POINTER(C.c_void_p))
        s.v_cache = C.cast(self._v_arr, C.POINTER(C.c_void_p))
        s.rows, s.n_rows = self.rows.data_ptr(), self.n_rows.data_ptr()
        s.logits = self.logits.data_ptr() if keep_logits else None
        s.row_entropy, s.row_argmax = self.row_entropy.data_ptr(), self.row_argmax.data_ptr()
        s.row_top1, s.chosen = self.row_top1.data_ptr(), self.chosen.data_ptr()
        s.n_chosen, s.e_max = self.n_chosen.data_ptr(), self.e_max.data_ptr()
        s.kv_drift = None
        s.attn_out = None
        self.attn_out = None                      # enable_attn_out(): last layer's attention output
        self.struct = s

    def enable_attn_out(self):
        """Have every step copy the last layer's attention output of its
        selected rows into self.attn_out ([L_cap, Hq, dh], rows [0, n_rows))."""
        import torch
        sh = self.model.shape
        self.attn_out = torch.zeros((self.model.L_cap, sh.n_q_heads, sh.head_dim),
                                    dtype=_torch_dtype(self.model.dtype), device="cuda")
        self.struct.attn_out = self.attn_out.data_ptr()

    def enable_drift(self):
        """Have full steps report each layer's Value drift (mean, max of 1 - cos)."""
        import torch
        self.kv_drift = torch.full((len(self.k_cache), 2), float("nan"), dtype=torch.float32,
                                   device="cuda")
        self.struct.kv_drift = self.kv_drift.data_ptr()

    def step(self, tau: float, k: int, block_start: int, block_len: int, n_unmask: int,
             phase_events=None, mode: int = L.EC_MODE_DEVICE, block_causal: bool = False) -> None:
        """One ec_step.  mode: EC_MODE_DEVICE (the flag stays on the device), or
        EC_MODE_FULL / EC_MODE_PARTIAL when the caller has read full_flag.
        block_causal: block diffusion (rows of the current block only, keys
        before its end)."""
        cfg = L.ec_step_cfg(float(tau), int(k), int(n_unmask), int(block_start), int(block_len),
                            int(mode), int(bool(block_causal)))
        L.ec_step(self.model.struct, self.struct, cfg, self.ws, phase_events)

    def commit(self, k: int, block_start: int, block_len: int, phase_events=None) -> None:
        """Block diffusion: make a finished block's K/V final (the flag set on
        the device, then a full pass over the block that decodes nothing)."""
        self.full_flag.fill_(1)
        self.step(0.0, k, block_start, block_len, 0, phase_events, block_causal=True)

    def step_host_mode(self, tau: float, k: int, block_start: int, block_len: int, n_unmask: int,
                       phase_events=None) -> int:
        """One step whose mode the host reads first (a 4-byte copy that waits
        for the previous step), so only that mode's kernels are launched.
        Returns the mode used (1 full, 0 partial)."""
        full = int(self.full_flag.item())
        self.step(tau, k, block_start, block_len, n_unmask, phase_events,
                  L.EC_MODE_FULL if full else L.EC_MODE_PARTIAL)
        return full

    def step_external(self, tau: float, k: int, block_start: int, block_len: int, decoded_logits,
                      phase_events=None) -> None:
        """A step of a model without LM head: `decoded_logits` ([n, V] device
        tensor, contiguous, the model's dtype) are the rows the caller decoded."""
        if self.model.w_lm is not None:
            raise ValueError("step_external needs a model without LM head")
        if not decoded_logits.is_contiguous() or decoded_logits.shape[1] != self.model.shape.vocab:
            raise ValueError("decoded_logits must be a contiguous [n, V] tensor")
        saved = self.struct.logits
        self.struct.logits = decoded_logits.data_ptr()
        try:
            self.step(tau, k, block_start, block_len, decoded_logits.shape[0], phase_events)
        finally:
            self.struct.logits = saved

    def copy_state_from(self, other: "DeviceSequence") -> None:
        """Device-side copy of another sequence's state (same model and sizes):
        tokens, mask, history, flag and every layer's caches."""
        for a, b in ((self.tokens, other.tokens), (self.is_masked, other.is_masked),
                     (self.history, other.history), (self.history_len, other.history_len),
                     (self.full_flag, other.full_flag)):
            a.copy_(b)
        for a, b in zip(self.k_cache + self.v_cache, other.k_cache + other.v_cache):
            a.copy_(b)

    # -- state transfer (tests: teacher forcing and read-back) -------------------
    def load_state(self, tokens, masked, history: Sequence[int], flag: int,
                   K: Optional[List[np.ndarray]] = None, V: Optional[List[np.ndarray]] = None):
        """Overwrite the device state; K/V given as [Hkv, L, dh] float arrays."""
        import torch
        cap = self.history.numel()
        ring = np.full(cap, -1, dtype=np.int32)
        for i, p in enumerate(history):
            ring[i % cap] = p
        self.tokens.copy_(torch.from_numpy(np.asarray(tokens, dtype=np.int32)))
        self.is_masked.copy_(torch.from_numpy(np.asarray(masked, dtype=np.uint8)))
        self.history.copy_(torch.from_numpy(ring))
        self.history_len.fill_(len(history))
        self.full_flag.fill_(int(flag))
        if K is not None:
            for l in range(len(self.k_cache)):
                Lq = K[l].shape[1]
                self.k_cache[l][:, :Lq].copy_(to_device(K[l].astype(np.float32), self.model.dtype))
                vt = np.ascontiguousarray(V[l].transpose(0, 2, 1)).astype(np.float32)
                self.v_cache[l][:, :, :Lq].copy_(to_device(vt, self.model.dtype))

    def caches(self, layer: int):
        """(K [Hkv, L, dh], V [Hkv, L, dh]) of one layer as float64 numpy arrays."""
        Lq = self.L
        k = self.k_cache[layer][:, :Lq].float().cpu().numpy().astype(np.float64)
        v = self.v_cache[layer][:, :, :Lq].float().cpu().numpy().astype(np.float64).transpose(0, 2, 1)
        return k, v

