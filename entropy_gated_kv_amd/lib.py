"""ctypes binding of libec.so: argument marshalling only.

Each Python function has the name of the C entry point it calls and takes
torch tensors where the C call takes device pointers (None for NULL).  Work
is enqueued on torch's current HIP stream.  A non-zero status raises
EcError.  There is no fallback: if libec.so is missing or fails to load,
every call raises.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Sequence

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libec.so")

EC_F32, EC_BF16 = 0, 1
EC_MODE_DEVICE, EC_MODE_FULL, EC_MODE_PARTIAL = 0, 1, 2
EC_NOALLOC_SCRATCH_BYTES = 8 << 20     # of include/ec.h
PHASES = ("select", "embed", "qkv", "attn", "oproj", "ffn", "lmhead", "entropy", "decide")

_lib: Optional[C.CDLL] = None
ABI_VERSION = 6                  # EC_ABI_VERSION of include/ec.h


class EcError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = _lib.ec_status_string(status).decode() if _lib is not None else str(status)
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


class ec_layer(C.Structure):
    _fields_ = [("w_qkv", C.c_void_p), ("w_o", C.c_void_p), ("norm_attn", C.c_void_p),
                ("norm_ffn", C.c_void_p), ("w_gate", C.c_void_p), ("w_up", C.c_void_p),
                ("w_down", C.c_void_p)]


class ec_model(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("d", C.c_int32), ("Hq", C.c_int32), ("Hkv", C.c_int32),
                ("dh", C.c_int32), ("d_ffn", C.c_int32), ("V", C.c_int32), ("L_cap", C.c_int32),
                ("dtype", C.c_int32), ("rms_eps", C.c_float), ("tok_emb", C.c_void_p),
                ("pos_emb", C.c_void_p), ("layers", C.POINTER(ec_layer)),
                ("norm_final", C.c_void_p), ("w_lm", C.c_void_p), ("logit_scale", C.c_void_p),
                ("w_lm_packed", C.c_void_p)]


class ec_state(C.Structure):
    _fields_ = [("L", C.c_int32), ("tokens", C.c_void_p), ("is_masked", C.c_void_p),
                ("history", C.c_void_p), ("history_len", C.c_void_p), ("history_cap", C.c_int32),
                ("full_flag", C.c_void_p), ("k_cache", C.POINTER(C.c_void_p)),
                ("v_cache", C.POINTER(C.c_void_p)), ("rows", C.c_void_p), ("n_rows", C.c_void_p),
                ("logits", C.c_void_p), ("row_entropy", C.c_void_p), ("row_argmax", C.c_void_p),
                ("row_top1", C.c_void_p), ("chosen", C.c_void_p), ("n_chosen", C.c_void_p),
                ("e_max", C.c_void_p), ("kv_drift", C.c_void_p), ("attn_out", C.c_void_p)]


class ec_step_cfg(C.Structure):
    _fields_ = [("tau", C.c_float), ("k", C.c_int32), ("n_unmask", C.c_int32),
                ("block_start", C.c_int32), ("block_len", C.c_int32), ("mode", C.c_int32),
                ("block_causal", C.c_int32)]


_P, _I32, _I64, _F32, _SZ = C.c_void_p, C.c_int32, C.c_int64, C.c_float, C.c_size_t

_SIGS = {
    "ec_status_string": (C.c_char_p, [_I32]),
    "ec_abi_version": (_I32, []),
    "ec_entropy_workspace_bytes": (_SZ, [_I64, _I64]),
    "ec_entropy_max": (_I32, [_P, _I32, _I64, _I64, _I64, _P, _P, _I32, _F32, _P, _P, _P, _P, _P,
                              _P, _SZ, _P]),
    "ec_entropy_max_noalloc": (_I32, [_P, _I32, _I64, _I64, _I64, _P, _P, _I32, _F32, _P, _P, _P,
                                      _P, _P, _P]),
    "ec_select_rows": (_I32, [_P, _P, _I32, _I32, _I32, _I32, _P, _P, _I32, _I32, _P, _P, _P]),
    "ec_kv_refresh_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32, _I32, _I32]),
    "ec_kv_refresh": (_I32, [_P, _I64, _P, _P, _I32, _P, _I32, _I32, _I32, _I32, _I32, _P, _P, _P,
                             _I32, _P, _SZ, _P]),
    "ec_attention_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32, _I32]),
    "ec_bidir_attention": (_I32, [_P, _P, _I32, _P, _P, _I32, _I32, _I32, _I32, _I32, _F32, _I32,
                                  _P, _P, _SZ, _P]),
    "ec_step_workspace_bytes": (_SZ, [C.POINTER(ec_model), _I32]),
    "ec_pack_lm_head": (_I32, [_P, _I32, _I32, _I32, _P, _P]),
    "ec_step": (_I32, [C.POINTER(ec_model), C.POINTER(ec_state), C.POINTER(ec_step_cfg), _P, _SZ,
                       _P, _P]),
}

EXPORTED = tuple(_SIGS)


def load(path: Optional[str] = None) -> C.CDLL:
    """Load libec.so (once).  Raises if it is missing: there is no fallback."""
    global _lib
    if _lib is None:
        p = path or LIB_PATH
        if not os.path.exists(p):
            raise RuntimeError(f"{p} is not built; run __graft_entry__.build() first")
        lib = C.CDLL(p)
        for name, (res, args) in _SIGS.items():
            f = getattr(lib, name)
            f.restype = res
            f.argtypes = args
        if lib.ec_abi_version() != ABI_VERSION:   # the struct layouts below must match ec.h
            raise RuntimeError(f"{p}: ABI version {lib.ec_abi_version()}, this binding expects {ABI_VERSION}")
        _lib = lib
    return _lib


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream=None) -> Optional[int]:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _check(fn: str, st: int) -> None:
    if st != 0:
        raise EcError(fn, st)


def dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return EC_F32
    if t.dtype == torch.bfloat16:
        return EC_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


# ---------------------------------------------------------------------------
def ec_entropy_workspace_bytes(n_rows: int, V: int) -> int:
    return load().ec_entropy_workspace_bytes(n_rows, V)


def ec_entropy_max(logits, tau: float, row_entropy, e_max, full_flag, ws, *, V: Optional[int] = None,
                   decoded_rows=None, n_decoded=None, max_decoded: int = 0, row_argmax=None,
                   row_top1=None, stream=None) -> None:
    n_rows = logits.shape[0]
    V = logits.shape[1] if V is None else V
    _check("ec_entropy_max", load().ec_entropy_max(
        _ptr(logits), dtype_code(logits), n_rows, V, logits.stride(0), _ptr(decoded_rows),
        _ptr(n_decoded), max_decoded, float(tau), _ptr(row_entropy), _ptr(row_argmax),
        _ptr(row_top1), _ptr(e_max), _ptr(full_flag), _ptr(ws), ws.numel() * ws.element_size(),
        _stream(stream)))


def ec_entropy_max_noalloc(logits, tau: float, row_entropy, e_max, full_flag, *,
                           V: Optional[int] = None, decoded_rows=None, n_decoded=None,
                           max_decoded: int = 0, row_argmax=None, row_top1=None,
                           stream=None) -> None:
    n_rows = logits.shape[0]
    V = logits.shape[1] if V is None else V
    _check("ec_entropy_max_noalloc", load().ec_entropy_max_noalloc(
        _ptr(logits), dtype_code(logits), n_rows, V, logits.stride(0), _ptr(decoded_rows),
        _ptr(n_decoded), max_decoded, float(tau), _ptr(row_entropy), _ptr(row_argmax),
        _ptr(row_top1), _ptr(e_max), _ptr(full_flag), _stream(stream)))


def ec_select_rows(full_flag, is_masked, block_start: int, block_len: int, history, history_len,
                   k: int, rows, n_rows, *, L: Optional[int] = None, block_causal: int = 0,
                   stream=None) -> None:
    L = is_masked.numel() if L is None else L
    _check("ec_select_rows", load().ec_select_rows(
        _ptr(full_flag), _ptr(is_masked), L, block_start, block_len, block_causal, _ptr(history),
        _ptr(history_len), history.numel(), k, _ptr(rows), _ptr(n_rows), _stream(stream)))


def ec_kv_refresh_workspace_bytes(max_rows: int, d: int, Hq: int, Hkv: int, dh: int,
                                  dtype: int) -> int:
    return load().ec_kv_refresh_workspace_bytes(max_rows, d, Hq, Hkv, dh, dtype)


def ec_kv_refresh(x, rows, n_rows, w_qkv, Hq: int, Hkv: int, dh: int, q_out, k_cache, v_cache,
                  ws=None, *, stream=None) -> None:
    max_rows, d = x.shape[0], w_qkv.shape[1]
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check("ec_kv_refresh", load().ec_kv_refresh(
        _ptr(x), x.stride(0), _ptr(rows), _ptr(n_rows), max_rows, _ptr(w_qkv), d, Hq, Hkv, dh,
        dtype_code(x), _ptr(q_out), _ptr(k_cache), _ptr(v_cache), k_cache.shape[1], _ptr(ws),
        nbytes, _stream(stream)))


def ec_attention_workspace_bytes(max_rows: int, L: int, Hq: int, Hkv: int, dh: int) -> int:
    return load().ec_attention_workspace_bytes(max_rows, L, Hq, Hkv, dh)


def ec_bidir_attention(q, n_rows, k_cache, v_cache, L: int, out, ws, *, scale: Optional[float] = None,
                       stream=None) -> None:
    max_rows, Hq, dh = q.shape
    Hkv, L_cap = k_cache.shape[0], k_cache.shape[1]
    scale = dh ** -0.5 if scale is None else scale
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check("ec_bidir_attention", load().ec_bidir_attention(
        _ptr(q), _ptr(n_rows), max_rows, _ptr(k_cache), _ptr(v_cache), L, L_cap, Hq, Hkv, dh,
        float(scale), dtype_code(q), _ptr(out), _ptr(ws), nbytes, _stream(stream)))


def ec_pack_lm_head(w_lm, w_packed, *, stream=None) -> None:
    V, d = w_lm.shape
    _check("ec_pack_lm_head", load().ec_pack_lm_head(_ptr(w_lm), V, d, dtype_code(w_lm),
                                                     _ptr(w_packed), _stream(stream)))


def ec_step_workspace_bytes(model: ec_model, max_block: int) -> int:
    return load().ec_step_workspace_bytes(C.byref(model), max_block)


def ec_step(model: ec_model, state: ec_state, cfg: ec_step_cfg, ws, phase_events=None,
            stream=None) -> None:
    ev = None
    if phase_events is not None:
        handles = []
        for e in phase_events:            # None: that record is skipped
            if e is not None and not e.cuda_event:   # torch creates events on first record
                e.record()
            handles.append(None if e is None else e.cuda_event)
        arr = (C.c_void_p * len(handles))(*handles)
        ev = C.cast(arr, C.c_void_p)
    _check("ec_step", load().ec_step(C.byref(model), C.byref(state), C.byref(cfg), _ptr(ws),
                                     ws.numel() * ws.element_size(), ev, _stream(stream)))
