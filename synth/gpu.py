"""Device-side draw of the bulk keys/values (GPU twin of ``synth.bulk_keys`` / ``synth.bulk_values``).

Input generation only.  Loads ``synth/libsynth_gen.so`` (built by
``python -m decode_attention_write_amd.build``); raises if it is missing.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import TAG_K, TAG_V, bulk_key, key_params

_LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsynth_gen.so")
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            raise RuntimeError(f"{_LIB} missing: run `python -m decode_attention_write_amd.build`")
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        lib.synth_bulk_kv.argtypes = [P, P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, P, P,
                                      ctypes.c_uint32, P, P, P]
        lib.synth_bulk_kv.restype = ctypes.c_int
        _lib = lib
    return _lib


class HeadParams:
    """Per-KV-head generator parameters of one (workload, layer), resident on the device."""

    def __init__(self, cfg: int, layer: int, hkv: int, device="cuda"):
        import torch
        mus, mults = zip(*[key_params(cfg, layer, h) for h in range(hkv)])
        self.hkv = hkv
        self.mu = torch.from_numpy(np.stack(mus).astype(np.float32)).to(device)
        self.mult = torch.from_numpy(np.stack(mults).astype(np.float32)).to(device)
        kk = np.array([bulk_key(cfg, layer, h, TAG_K) for h in range(hkv)], dtype=np.uint32)
        kvv = np.array([bulk_key(cfg, layer, h, TAG_V) for h in range(hkv)], dtype=np.uint32)
        self.key_k = torch.from_numpy(kk.view(np.int32)).to(device)
        self.key_v = torch.from_numpy(kvv.view(np.int32)).to(device)


def draw_kv(params: HeadParams, seq: int, token0: int, n_tokens: int, k_out, v_out, stream=None):
    """Fill bf16 device tensors k_out, v_out [n_tokens, hkv, 128] (either may be None)."""
    import torch
    st = torch.cuda.current_stream().cuda_stream if stream is None else int(stream)
    ptr = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None  # noqa: E731
    rc = _load().synth_bulk_kv(ptr(k_out), ptr(v_out), int(n_tokens), int(token0), params.hkv,
                               ptr(params.key_k), ptr(params.key_v), ctypes.c_uint32(int(seq) & 0xFFFFFFFF),
                               ptr(params.mu), ptr(params.mult), ctypes.c_void_p(st))
    if rc != 0:
        raise RuntimeError(f"synth_bulk_kv failed ({rc})")
