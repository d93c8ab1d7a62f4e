"""Python binding of liboscar (INT2 paged KV cache: write path and fused decode attention, gfx950).

Argument marshalling only: every step of the write and read paths runs in the
HIP kernels of ``liboscar.so``.  PyTorch provides device memory and the current
stream.  The functions named like the C ABI (``oscar_calibrate_host``,
``oscar_kv_write``, ``oscar_kv_evict_window``, ``oscar_decode_attn``) take the
same arguments as their C counterparts, with tensors in place of pointers;
``KVStore`` bundles one layer's device buffers and handle.

Loading fails loudly when the library has not been built; there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboscar.so")

HEAD_DIM = 128
PAGE_TOKENS = 64
SINK_TOKENS = 64
WINDOW_TOKENS = 256
RING_SLOTS = 320
HEAD_BLOCK = 5120
FLAG_PLAN_ONLY = 1

OK, E_ARG, E_NOPAGE, E_WINDOW_FULL, E_WINDOW_SHORT, E_NUMERIC, E_HIP, E_WORKSPACE, E_STATE = 0, -1, -2, -3, -4, -5, -6, -7, -8
TIMED_DECODE, TIMED_WRITE = 0, 1  # kernels recorded by KVStore.set_timing
TIMING_PAIRS = 4096               # event pairs per timed kernel
_NAMES = {E_ARG: "E_ARG", E_NOPAGE: "E_NOPAGE", E_WINDOW_FULL: "E_WINDOW_FULL", E_WINDOW_SHORT: "E_WINDOW_SHORT",
          E_NUMERIC: "E_NUMERIC", E_HIP: "E_HIP", E_WORKSPACE: "E_WORKSPACE", E_STATE: "E_STATE"}

EXPORTS = [
    "oscar_calibrate_host", "oscar_calibrate_value_host", "oscar_fold_value_rotation", "oscar_kv_buffer_bytes", "oscar_kv_create", "oscar_kv_set_rotation",
    "oscar_kv_write", "oscar_kv_evict_window", "oscar_decode_workspace_bytes", "oscar_decode_attn",
    "oscar_kv_seq_info", "oscar_kv_get_page_table", "oscar_kv_free_pages", "oscar_kv_reset_seq",
    "oscar_kv_decode_write", "oscar_kv_set_decode_split", "oscar_kv_set_decode_kernel",
    "oscar_kv_set_decode_deterministic",
    "oscar_kv_set_timing",
    "oscar_kv_read_timing", "oscar_last_error", "oscar_kv_destroy",
    "oscar_decode_step_workspace_bytes", "oscar_decode_step", "oscar_kv_set_write_evicts",
    "oscar_kv_set_output_bf16", "oscar_decode_step_noalloc", "oscar_kv_set_key_mean",
]
NOALLOC_SCRATCH_BYTES = 32 << 20   # OSCAR_NOALLOC_SCRATCH_BYTES


class OscarError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{_NAMES.get(status, status)}: {msg}")
        self.status = status


class _Desc(ctypes.Structure):
    _fields_ = [
        ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32), ("max_seqs", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32), ("num_pages", ctypes.c_int32), ("flags", ctypes.c_int32),
        ("pool", ctypes.c_void_p), ("ring", ctypes.c_void_p), ("page_table", ctypes.c_void_p), ("rot", ctypes.c_void_p),
    ]


_lib = None


def load():
    """Load liboscar.so (built in-tree); raises when it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: run `python -m decode_attention_write_amd.build` first")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    sig = {
        "oscar_calibrate_host": [P, I64, I32, P, P],
        "oscar_calibrate_value_host": [P, P, I64, I64, I32, P, P],
        "oscar_fold_value_rotation": [I32, I32, I32, P, P, P],
        "oscar_kv_buffer_bytes": [P, P, P, P, P],
        "oscar_kv_create": [P, P, I32, P, P],
        "oscar_kv_set_rotation": [P, P, P],
        "oscar_kv_set_key_mean": [P, P, P],
        "oscar_kv_write": [P, P, I32, I32, P, P, P],
        "oscar_kv_evict_window": [P, P, I32, I32, P],
        "oscar_decode_workspace_bytes": [P, P, I32, P],
        "oscar_decode_attn": [P, P, I32, P, ctypes.c_float, P, P, SZ, P],
        "oscar_kv_seq_info": [P, I32, P, P],
        "oscar_kv_get_page_table": [P, P],
        "oscar_kv_free_pages": [P, P, P],
        "oscar_kv_reset_seq": [P, I32, P],
        "oscar_kv_set_decode_split": [P, I32],
        "oscar_kv_decode_write": [P, P, I32, P, P, P],
        "oscar_kv_set_decode_kernel": [P, I32],
        "oscar_kv_set_decode_deterministic": [P, I32],
        "oscar_kv_set_timing": [P, I32],
        "oscar_kv_read_timing": [P, I32, P, P, P],
        "oscar_decode_step_workspace_bytes": [P, P, I32, P],
        "oscar_decode_step": [P, P, I32, P, P, P, ctypes.c_float, P, P, SZ, P],
        "oscar_kv_set_write_evicts": [P, I32],
        "oscar_kv_set_output_bf16": [P, I32],
        "oscar_decode_step_noalloc": [P, P, I32, P, P, P, ctypes.c_float, P, P],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.oscar_last_error.argtypes = []
    lib.oscar_last_error.restype = ctypes.c_char_p
    lib.oscar_kv_destroy.argtypes = [P]
    lib.oscar_kv_destroy.restype = None
    _lib = lib
    return lib


def _check(rc):
    if rc != OK:
        raise OscarError(rc, load().oscar_last_error().decode())


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def check_tensor(t, name, shape, dtypes, device=None):
    """Raise ValueError unless t is a contiguous tensor of exactly `shape` whose dtype is one of
    `dtypes` (on `device`, when given).  The library reads and writes raw device memory through
    these pointers, so a wrong size, stride or element width would go out of bounds silently."""
    if t is None:
        raise ValueError(f"{name}: missing tensor")
    if t.shape != shape and tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name}: dtype {t.dtype}, expected one of {[str(d) for d in dtypes]}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: not contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")


_BF16_TYPES = None


def _bf16_types():
    global _BF16_TYPES
    if _BF16_TYPES is None:
        import torch
        _BF16_TYPES = (torch.bfloat16, torch.int16, torch.uint16)   # bf16 values or their raw bits
    return _BF16_TYPES


def _out_types(store):
    import torch
    return (torch.bfloat16,) if store.out_bf16 else (torch.float32,)


def _check_ws(ws, device):
    if ws is None or not ws.is_contiguous():
        raise ValueError("ws: missing or not contiguous")
    if device is not None and ws.device != device:
        raise ValueError(f"ws: on {ws.device}, expected {device}")


def _current_raw_stream():
    """torch's current stream on the current device as an integer handle.  The raw query costs a
    tenth of a microsecond against about three for torch.cuda.current_stream(), which builds a
    Python stream object: it dominated the host time of a one-token decode-step write."""
    import torch
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None:
        return raw(torch._C._cuda_getDevice())
    return torch.cuda.current_stream().cuda_stream


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(_current_raw_stream())
    return ctypes.c_void_p(int(stream))


_I32_CACHE = {}


def _i32(seq_ids):
    """int32 array of sequence ids and its address.  Short id lists are cached by value (the
    library only reads them), which saves building the array on every decode-step call."""
    if isinstance(seq_ids, (list, tuple)) and len(seq_ids) <= 64:
        key = tuple(seq_ids)
        hit = _I32_CACHE.get(key)
        if hit is not None:
            return hit
        a = np.ascontiguousarray(np.asarray(seq_ids, dtype=np.int32))
        a.setflags(write=False)
        r = (a, a.ctypes.data_as(ctypes.c_void_p))
        if len(_I32_CACHE) < 4096:
            _I32_CACHE[key] = r
        return r
    a = np.ascontiguousarray(np.asarray(seq_ids, dtype=np.int32))
    return a, a.ctypes.data_as(ctypes.c_void_p)


# ---------------------------------------------------------------------------- C-ABI-named functions

def oscar_calibrate_host(q_rows):
    """R_K (float32 [128,128]) and descending eigenvalues (float64 [128]) from query rows (host)."""
    q = np.ascontiguousarray(np.asarray(q_rows, dtype=np.float32))
    rot = np.empty((HEAD_DIM, HEAD_DIM), dtype=np.float32)
    eig = np.empty(HEAD_DIM, dtype=np.float64)
    _check(load().oscar_calibrate_host(q.ctypes.data_as(ctypes.c_void_p), q.shape[0], q.shape[1],
                                       rot.ctypes.data_as(ctypes.c_void_p), eig.ctypes.data_as(ctypes.c_void_p)))
    return rot, eig


def oscar_calibrate_value_host(s_probs, v_rows):
    """R_V (float32 [128,128]) and descending eigenvalues of C_S from calibration attention
    probabilities s [n_q, n_tok] and values v [n_tok, 128] (host)."""
    s = np.ascontiguousarray(np.asarray(s_probs, dtype=np.float32))
    v = np.ascontiguousarray(np.asarray(v_rows, dtype=np.float32))
    if s.ndim != 2 or v.ndim != 2 or s.shape[1] != v.shape[0]:
        raise ValueError("s must be [n_q, n_tok] and v [n_tok, 128]")
    rot = np.empty((HEAD_DIM, HEAD_DIM), dtype=np.float32)
    eig = np.empty(HEAD_DIM, dtype=np.float64)
    _check(load().oscar_calibrate_value_host(s.ctypes.data_as(ctypes.c_void_p), v.ctypes.data_as(ctypes.c_void_p),
                                             s.shape[0], s.shape[1], v.shape[1],
                                             rot.ctypes.data_as(ctypes.c_void_p), eig.ctypes.data_as(ctypes.c_void_p)))
    return rot, eig


def oscar_fold_value_rotation(w_v, w_o, r_v, num_q_heads, num_kv_heads):
    """Fold R_V into copies of w_v [d_model, Hkv*128] and w_o [Hq*128, d_model] (host, float32)."""
    wv = np.array(w_v, dtype=np.float32, order="C", copy=True)
    wo = np.array(w_o, dtype=np.float32, order="C", copy=True)
    r = np.ascontiguousarray(np.asarray(r_v, dtype=np.float32))
    if wv.shape[1] != num_kv_heads * HEAD_DIM or wo.shape != (num_q_heads * HEAD_DIM, wv.shape[0]) \
            or r.shape != (num_kv_heads, HEAD_DIM, HEAD_DIM):
        raise ValueError("shape mismatch between w_v, w_o, r_v and the head counts")
    _check(load().oscar_fold_value_rotation(wv.shape[0], num_q_heads, num_kv_heads, r.ctypes.data_as(ctypes.c_void_p),
                                            wv.ctypes.data_as(ctypes.c_void_p), wo.ctypes.data_as(ctypes.c_void_p)))
    return wv, wo


def oscar_kv_write(store, seq_ids, k, v, stream=None):
    """k, v: bf16 device tensors [n_seqs, n_new, Hkv, 128] (contiguous)."""
    ids, p = _i32(seq_ids)
    if k is None or k.dim() != 4:
        raise ValueError("k must be [n_seqs, n_new, Hkv, 128]")
    n_new = int(k.shape[1])
    for t, name in ((k, "k"), (v, "v")):
        check_tensor(t, name, (len(ids), n_new, store.hkv, HEAD_DIM), _bf16_types(), store.device)
    _check(load().oscar_kv_write(store.handle, p, len(ids), n_new, _ptr(k), _ptr(v),
                                 None if store.plan_only else _stream(stream)))


def oscar_kv_evict_window(store, seq_ids, n_evict, stream=None):
    ids, p = _i32(seq_ids)
    _check(load().oscar_kv_evict_window(store.handle, p, len(ids), int(n_evict),
                                        None if store.plan_only else _stream(stream)))


def oscar_kv_decode_write(store, seq_ids, k, v, stream=None):
    """The decode step's write: evict when the window is full, then append one token.
    k, v: bf16 device tensors [n_seqs, Hkv, 128] (contiguous)."""
    ids, p = _i32(seq_ids)
    if not store.plan_only:
        shape = (len(ids), store.hkv, HEAD_DIM)
        check_tensor(k, "k", shape, _bf16_types(), store.device)
        check_tensor(v, "v", shape, _bf16_types(), store.device)
    _check(load().oscar_kv_decode_write(store.handle, p, len(ids), _ptr(k), _ptr(v),
                                        None if store.plan_only else _stream(stream)))


def oscar_decode_workspace_bytes(store, seq_ids):
    ids, p = _i32(seq_ids)
    n = ctypes.c_size_t(0)
    _check(load().oscar_decode_workspace_bytes(store.handle, p, len(ids), ctypes.byref(n)))
    return n.value


def oscar_decode_attn(store, seq_ids, q, sm_scale, out, ws, stream=None):
    """q: bf16 [n_seqs, Hq, 128]; out: fp32 [n_seqs, Hq, 128] (bf16 when the store's output is
    bf16); ws: device workspace tensor."""
    ids, p = _i32(seq_ids)
    if store.plan_only:
        _check(load().oscar_decode_attn(store.handle, p, len(ids), None, ctypes.c_float(sm_scale), None, None, 0, None))
        return
    check_tensor(q, "q", (len(ids), store.hq, HEAD_DIM), _bf16_types(), store.device)
    check_tensor(out, "out", (len(ids), store.hq, HEAD_DIM), _out_types(store), store.device)
    _check_ws(ws, store.device)
    nbytes = ws.numel() * ws.element_size()
    _check(load().oscar_decode_attn(store.handle, p, len(ids), _ptr(q), ctypes.c_float(sm_scale), _ptr(out),
                                    _ptr(ws), nbytes, _stream(stream)))


def oscar_decode_step_workspace_bytes(store, seq_ids):
    ids, p = _i32(seq_ids)
    n = ctypes.c_size_t(0)
    _check(load().oscar_decode_step_workspace_bytes(store.handle, p, len(ids), ctypes.byref(n)))
    return n.value


def oscar_decode_step(store, seq_ids, k, v, q, sm_scale, out, ws, stream=None):
    """One whole decode step (the decode-step write of k, v, then attention of q over everything
    stored).  k, v: bf16 [n_seqs, Hkv, 128]; q: bf16 [n_seqs, Hq, 128]; out: fp32 [n_seqs, Hq, 128]."""
    ids, p = _i32(seq_ids)
    if store.plan_only:
        _check(load().oscar_decode_step(store.handle, p, len(ids), None, None, None, ctypes.c_float(sm_scale),
                                        None, None, 0, None))
        return
    for t, name in ((k, "k"), (v, "v")):
        check_tensor(t, name, (len(ids), store.hkv, HEAD_DIM), _bf16_types(), store.device)
    check_tensor(q, "q", (len(ids), store.hq, HEAD_DIM), _bf16_types(), store.device)
    check_tensor(out, "out", (len(ids), store.hq, HEAD_DIM), _out_types(store), store.device)
    _check_ws(ws, store.device)
    nbytes = ws.numel() * ws.element_size()
    _check(load().oscar_decode_step(store.handle, p, len(ids), _ptr(k), _ptr(v), _ptr(q), ctypes.c_float(sm_scale),
                                    _ptr(out), _ptr(ws), nbytes, _stream(stream)))


def oscar_decode_step_noalloc(store, seq_ids, k, v, q, sm_scale, out, stream=None):
    """oscar_decode_step with the workspace taken from the library's per-GPU scratch array
    (NOALLOC_SCRATCH_BYTES): allocates nothing.  Calls that overlap on one GPU race."""
    ids, p = _i32(seq_ids)
    if store.plan_only:
        _check(load().oscar_decode_step_noalloc(store.handle, p, len(ids), None, None, None, ctypes.c_float(sm_scale),
                                                None, None))
        return
    for t, name in ((k, "k"), (v, "v")):
        check_tensor(t, name, (len(ids), store.hkv, HEAD_DIM), _bf16_types(), store.device)
    check_tensor(q, "q", (len(ids), store.hq, HEAD_DIM), _bf16_types(), store.device)
    check_tensor(out, "out", (len(ids), store.hq, HEAD_DIM), _out_types(store), store.device)
    _check(load().oscar_decode_step_noalloc(store.handle, p, len(ids), _ptr(k), _ptr(v), _ptr(q),
                                            ctypes.c_float(sm_scale), _ptr(out), _stream(stream)))


# ---------------------------------------------------------------------------- store object

class KVStore:
    """One attention layer's store: caller-owned torch device buffers + the liboscar handle."""

    def __init__(self, num_q_heads, num_kv_heads, max_seqs, max_pages_per_seq, num_pages,
                 free_pages=None, device="cuda", plan_only=False, stream=None):
        lib = load()
        self.hq, self.hkv = num_q_heads, num_kv_heads
        self.max_seqs, self.max_pages, self.num_pages = max_seqs, max_pages_per_seq, num_pages
        self.plan_only = plan_only
        self.out_bf16 = False
        self.device = None
        d = _Desc(num_q_heads, num_kv_heads, max_seqs, max_pages_per_seq, num_pages,
                  FLAG_PLAN_ONLY if plan_only else 0, None, None, None, None)
        sizes = [ctypes.c_size_t(0) for _ in range(4)]
        _check(lib.oscar_kv_buffer_bytes(ctypes.byref(d), *[ctypes.byref(s) for s in sizes]))
        self.bytes = {k: s.value for k, s in zip(("pool", "ring", "page_table", "rot"), sizes)}
        self.pool = self.ring = self.page_table_dev = self.rot = None
        if not plan_only:
            import torch
            self.pool = torch.empty(self.bytes["pool"], dtype=torch.uint8, device=device)
            self.ring = torch.empty(self.bytes["ring"] // 2, dtype=torch.int16, device=device)
            self.page_table_dev = torch.empty(self.bytes["page_table"] // 4, dtype=torch.int32, device=device)
            self.rot = torch.empty(self.bytes["rot"], dtype=torch.uint8, device=device)
            self.device = self.pool.device
            d.pool, d.ring = self.pool.data_ptr(), self.ring.data_ptr()
            d.page_table, d.rot = self.page_table_dev.data_ptr(), self.rot.data_ptr()
        fp = np.arange(num_pages, dtype=np.int32) if free_pages is None else np.asarray(free_pages, dtype=np.int32)
        fp = np.ascontiguousarray(fp)
        h = ctypes.c_void_p(0)
        _check(lib.oscar_kv_create(ctypes.byref(d), fp.ctypes.data_as(ctypes.c_void_p), len(fp),
                                   None if plan_only else _stream(stream), ctypes.byref(h)))
        self.handle = h

    def close(self):
        if getattr(self, "handle", None):
            load().oscar_kv_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ---- API
    def set_rotation(self, rot, stream=None):
        r = np.ascontiguousarray(np.asarray(rot, dtype=np.float32).reshape(self.hkv, HEAD_DIM, HEAD_DIM))
        _check(load().oscar_kv_set_rotation(self.handle, r.ctypes.data_as(ctypes.c_void_p),
                                            None if self.plan_only else _stream(stream)))

    def set_key_mean(self, mean, stream=None):
        """Per-KV-head key mean subtracted from every key written afterwards (fp32 [hkv, 128]),
        or None to write keys as they are."""
        if mean is None:
            _check(load().oscar_kv_set_key_mean(self.handle, None, None if self.plan_only else _stream(stream)))
            return
        m = np.ascontiguousarray(np.asarray(mean, dtype=np.float32).reshape(self.hkv, HEAD_DIM))
        _check(load().oscar_kv_set_key_mean(self.handle, m.ctypes.data_as(ctypes.c_void_p),
                                            None if self.plan_only else _stream(stream)))

    def write(self, seq_ids, k, v, stream=None, n_new=None):
        if self.plan_only:
            ids, p = _i32(seq_ids)
            _check(load().oscar_kv_write(self.handle, p, len(ids), int(n_new), None, None, None))
            return
        oscar_kv_write(self, seq_ids, k, v, stream)

    def set_output_bf16(self, on):
        """Decode outputs as bf16 (torch.bfloat16 tensors from decode / decode_step) instead of fp32."""
        _check(load().oscar_kv_set_output_bf16(self.handle, 1 if on else 0))
        self.out_bf16 = bool(on)

    def _out(self, n, device):
        import torch
        return torch.empty((n, self.hq, HEAD_DIM), dtype=torch.bfloat16 if self.out_bf16 else torch.float32,
                           device=device)

    def set_write_evicts(self, on):
        """Let writes overflow a non-empty window, evicting as they go (chunked prefill)."""
        _check(load().oscar_kv_set_write_evicts(self.handle, 1 if on else 0))

    def evict(self, seq_ids, n_evict=1, stream=None):
        oscar_kv_evict_window(self, seq_ids, n_evict, stream)

    def decode_write(self, seq_ids, k, v, stream=None):
        oscar_kv_decode_write(self, seq_ids, k, v, stream)

    def workspace_bytes(self, seq_ids):
        return oscar_decode_workspace_bytes(self, seq_ids)

    def decode(self, seq_ids, q, sm_scale, out=None, ws=None, stream=None):
        import torch
        n = len(seq_ids)
        if out is None:
            out = self._out(n, q.device)
        if ws is None:
            ws = torch.empty(max(4, self.workspace_bytes(seq_ids)) // 4, dtype=torch.float32, device=q.device)
        oscar_decode_attn(self, seq_ids, q, sm_scale, out, ws, stream)
        return out

    def step_workspace_bytes(self, seq_ids):
        return oscar_decode_step_workspace_bytes(self, seq_ids)

    def decode_step(self, seq_ids, k, v, q, sm_scale, out=None, ws=None, stream=None):
        """The decode-step write and the decode attention in one call; returns out."""
        if out is None and not self.plan_only:
            out = self._out(len(seq_ids), q.device)
        if ws is None and not self.plan_only:
            import torch
            ws = torch.empty(max(4, self.step_workspace_bytes(seq_ids)) // 4, dtype=torch.float32, device=q.device)
        oscar_decode_step(self, seq_ids, k, v, q, sm_scale, out, ws, stream)
        return out

    def decode_step_noalloc(self, seq_ids, k, v, q, sm_scale, out, stream=None):
        """decode_step with the library's scratch array instead of a workspace; `out` is required
        (this form allocates nothing)."""
        oscar_decode_step_noalloc(self, seq_ids, k, v, q, sm_scale, out, stream)
        return out

    def seq_info(self, seq):
        ln, n2 = ctypes.c_int64(0), ctypes.c_int64(0)
        _check(load().oscar_kv_seq_info(self.handle, int(seq), ctypes.byref(ln), ctypes.byref(n2)))
        return ln.value, n2.value

    def page_table(self):
        out = np.empty((self.max_seqs, self.max_pages), dtype=np.int32)
        _check(load().oscar_kv_get_page_table(self.handle, out.ctypes.data_as(ctypes.c_void_p)))
        return out

    def free_pages(self):
        n = ctypes.c_int32(0)
        _check(load().oscar_kv_free_pages(self.handle, ctypes.byref(n), None))
        out = np.empty(n.value, dtype=np.int32)
        _check(load().oscar_kv_free_pages(self.handle, None, out.ctypes.data_as(ctypes.c_void_p)))
        return out

    def reset_seq(self, seq, stream=None):
        _check(load().oscar_kv_reset_seq(self.handle, int(seq), None if self.plan_only else _stream(stream)))

    def set_decode_split(self, pages_per_split):
        _check(load().oscar_kv_set_decode_split(self.handle, int(pages_per_split)))

    def set_decode_kernel(self, kernel):
        """0 = matrix-core kernel (default), 1 = reference-grade fp32 kernel."""
        _check(load().oscar_kv_set_decode_kernel(self.handle, int(kernel)))

    def set_decode_deterministic(self, on=True):
        """Fixed page range per split (bitwise repeatable decode) instead of the default page
        sharing between the splits of a (sequence, KV head)."""
        _check(load().oscar_kv_set_decode_deterministic(self.handle, 1 if on else 0))

    def set_timing(self, enable=True):
        """Record HIP events around every launch of the decode split kernel and the write kernel
        (measurement aid)."""
        _check(load().oscar_kv_set_timing(self.handle, int(bool(enable))))

    def read_timing(self, kernel, each=False):
        """(timed launches, summed milliseconds[, per-launch milliseconds]) of TIMED_DECODE or
        TIMED_WRITE since the last read of that kernel; waits for them."""
        n = ctypes.c_int32(0)
        ms = ctypes.c_double(0.0)
        per = np.zeros(TIMING_PAIRS, dtype=np.float32) if each else None
        _check(load().oscar_kv_read_timing(self.handle, int(kernel), ctypes.byref(n), ctypes.byref(ms),
                                           per.ctypes.data_as(ctypes.c_void_p) if each else None))
        return (n.value, ms.value, per[:n.value].copy()) if each else (n.value, ms.value)

    # ---- views of the device buffers (for tests and export)
    def pool_view(self):
        return self.pool.view(self.num_pages, self.hkv, HEAD_BLOCK)

    def ring_view(self):
        return self.ring.view(self.max_seqs, self.hkv, 2, RING_SLOTS, HEAD_DIM)

    def table_view(self):
        return self.page_table_dev.view(self.max_seqs, self.max_pages)
