"""Mixed-precision paged KV store: routing, window eviction, FIFO page allocator.

Test infrastructure only (see package header).

Follows axbrief, section "Together AI, INT2 KV 캐시 시스템 'OSCAR' 공개" and
techllm, OSCAR section: recent tokens stay BF16, old history is INT2, an
attention-sink region is BF16 too, the BF16 share is about 0.24 % at 128K
context, and the cache stays a paged cache.  The write path rotates every key
by R_K, clips and quantizes (axbrief rotation section); values arrive already
rotated by R_V (folded into the projection weights offline, axbrief rotation
section) and are never rotated here.

Readings taken where the pages are silent:
* 64 sink tokens + a 256-token recent window (320 / 131072 = 0.244 %).
* Position p < 64 is a sink token.  On the first write into an empty sequence
  of length L, positions 64 .. L-257 go straight to INT2 (INT2 index p - 64);
  the last min(L-64, 256) positions go to the window.  A later write appends to
  the window only; a full window is an error (the caller evicts first).
* Sink and window keys are stored as bf16(k . R_K) (fp64 product, one
  rounding).  INT2 keys written by that first write are quantized from
  fp32(k . R_K).  Values are stored / quantized as given.
* Optional key mean (gist.science summary of OptR, section "해결책: OptR (출력
  인지 회전)", step 1: keys centred before the rotation): with a per-KV-head
  mean mu set, every key written afterwards enters as (k - mu) . R_K in fp64
  (subtraction, then the product) and is stored / quantized from that.
  Queries are rotated by R_K alone: each query's scores all move by
  -q . mu, which the softmax removes (attention-exact; pinned to 1e-12).
* Eviction moves the oldest window token (position 64 + n_int2) to INT2 index
  n_int2, quantizing from its stored bf16 key and value.
* Window token at position p sits in ring slot 64 + ((p - 64) mod 256);
  sink token p in slot p.  Ring: bf16 [seq][kv_head][K,V][320][128].
* Pages come from a FIFO free list.  A page is popped when INT2 index i with
  i % 64 == 0 is first written: sequences in call order, pages ascending
  within a sequence.  ``reset_seq`` returns a sequence's pages to the tail of
  the FIFO in ascending logical order.  A call that cannot get every page it
  needs, or would overfill a window, changes nothing.

Parity: pinned (store invariants, BF16 share, allocator order, bf16-only store
against unquantized attention, eviction of a known token, attention-exactness of
the key mean).
"""
from __future__ import annotations

from collections import deque

import numpy as np

from . import layout, quantizer
from .calibration import second_moment  # noqa: F401  (re-export for convenience)

SINK = 64
WINDOW = 256
RING_SLOTS = SINK + WINDOW
PAGE = layout.PAGE_TOKENS
D = layout.HEAD_DIM


class StoreError(Exception):
    pass


def to_bf16_bits_f64(x) -> np.ndarray:
    """Round fp64 values to bf16 (nearest, ties to even) directly from fp64; uint16 bits."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    flat = x.ravel()
    m, e = np.frexp(flat)                  # flat = m * 2^e, 0.5 <= |m| < 1
    # bf16 keeps 8 significant bits: scale mantissa to [128, 256) and round half to even.
    q = np.rint(m * 256.0)                 # np.rint rounds half to even
    y = np.ldexp(q, e - 8)
    b = (y.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    out.ravel()[:] = b
    return out


def rotate_keys(k64, rot, key_mean=None) -> np.ndarray:
    """The write path's key transform in fp64: (k - mu) . R_K per KV head, or k . R_K without a
    mean.  k64: [n, Hkv, 128]; rot: [Hkv, 128, 128]; key_mean: [Hkv, 128] or None."""
    k = np.asarray(k64, dtype=np.float64)
    if key_mean is not None:
        k = k - np.asarray(key_mean, dtype=np.float32).astype(np.float64)[None]
    return np.matmul(k.transpose(1, 0, 2), np.asarray(rot, dtype=np.float64)).transpose(1, 0, 2)


def bf16_to_f64(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


class OracleStore:
    """One attention layer's store, mirroring the library's semantics in plain NumPy."""

    def __init__(self, n_kv_heads, max_seqs, max_pages_per_seq, num_pages, free_pages, rot):
        self.hkv = n_kv_heads
        self.max_seqs = max_seqs
        self.max_pages = max_pages_per_seq
        self.num_pages = num_pages
        self.free = deque(int(p) for p in free_pages)
        self.rot = np.asarray(rot, dtype=np.float32).astype(np.float64)   # [Hkv, d, d]
        self.pool = np.zeros((num_pages, n_kv_heads, layout.HEAD_BLOCK), dtype=np.uint8)
        self.ring = np.zeros((max_seqs, n_kv_heads, 2, RING_SLOTS, D), dtype=np.uint16)
        self.page_table = np.full((max_seqs, max_pages_per_seq), -1, dtype=np.int32)
        self.length = np.zeros(max_seqs, dtype=np.int64)
        self.n_int2 = np.zeros(max_seqs, dtype=np.int64)
        # a write that overflows a non-empty window evicts token by token (else "window full")
        self.write_evicts = False
        self.key_mean = None          # [Hkv, 128] fp32 or None

    def set_key_mean(self, mean):
        """Per-KV-head key mean subtracted from every key written afterwards (None: none)."""
        self.key_mean = None if mean is None else np.asarray(mean, dtype=np.float32).reshape(self.hkv, D).copy()

    # ------------------------------------------------------------------ helpers
    def window_count(self, seq):
        return max(0, int(self.length[seq]) - SINK - int(self.n_int2[seq]))

    @staticmethod
    def ring_slot(pos):
        return pos if pos < SINK else SINK + (pos - SINK) % WINDOW

    def _put_int2(self, seq, idx0, k32, v32):
        """Quantize and store INT2 tokens idx0 .. idx0+n-1 (all heads); k32, v32 float32 [n, Hkv, d]."""
        n = k32.shape[0]
        kc, ks, kl = quantizer.quantize(k32, quantizer.C_K)    # [n, Hkv, 128], [n, Hkv, 2]
        vc, vs, vl = quantizer.quantize(v32, quantizer.C_V)
        t = 0
        while t < n:
            idx = idx0 + t
            page_i, slot = divmod(idx, PAGE)
            run = min(PAGE - slot, n - t)
            page = int(self.page_table[seq, page_i])
            assert page >= 0
            for h in range(self.hkv):
                if slot == 0:
                    cur = [np.zeros((PAGE, D), np.uint8), np.zeros((PAGE, D), np.uint8)] + \
                          [np.zeros((PAGE, 2), np.float16) for _ in range(4)]
                else:
                    cur = [np.array(a) for a in layout.unpack_head_block(self.pool[page, h], PAGE)]
                sl = slice(slot, slot + run)
                src = slice(t, t + run)
                cur[0][sl], cur[1][sl] = kc[src, h], vc[src, h]
                cur[2][sl], cur[3][sl], cur[4][sl], cur[5][sl] = ks[src, h], kl[src, h], vs[src, h], vl[src, h]
                self.pool[page, h] = layout.pack_head_block(*cur)
            t += run

    # ------------------------------------------------------------------ API
    def write(self, seq_ids, k_bits, v_bits):
        """k_bits, v_bits: bf16 uint16 [n_seqs, n_new, Hkv, 128]."""
        k_bits = np.asarray(k_bits, dtype=np.uint16)
        v_bits = np.asarray(v_bits, dtype=np.uint16)
        n_new = k_bits.shape[1]
        need = 0
        for b, s in enumerate(seq_ids):
            L0 = int(self.length[s])
            if L0 == 0:
                n_int2 = max(0, n_new - RING_SLOTS)
                need += -(-n_int2 // PAGE)
                if -(-n_int2 // PAGE) > self.max_pages:
                    raise StoreError("too many pages for one sequence")
            else:
                # tokens beyond the free sink + window slots each evict the oldest window token
                evictions = max(0, n_new - (RING_SLOTS - (L0 - int(self.n_int2[s]))))
                if evictions and not self.write_evicts:
                    raise StoreError("window full")
                n2 = int(self.n_int2[s])
                if -(-(n2 + evictions) // PAGE) > self.max_pages:
                    raise StoreError("too many pages for one sequence")
                need += -(-(n2 + evictions) // PAGE) - -(-n2 // PAGE)
        if need > len(self.free):
            raise StoreError("out of pages")
        for b, s in enumerate(seq_ids):
            L0 = int(self.length[s])
            k64 = bf16_to_f64(k_bits[b])                          # [n_new, Hkv, d]
            x = rotate_keys(k64, self.rot, self.key_mean)         # (k - mu) . R_K per head, fp64
            kx_bf = to_bf16_bits_f64(x)
            if L0 == 0:
                L = n_new
                n_int2 = max(0, L - RING_SLOTS)
                for i in range(-(-n_int2 // PAGE)):
                    self.page_table[s, i] = self.free.popleft()
                if n_int2:
                    self._put_int2(s, 0, x[SINK:SINK + n_int2].astype(np.float32),
                                   bf16_to_f64(v_bits[b, SINK:SINK + n_int2]).astype(np.float32))
                for p in list(range(min(L, SINK))) + list(range(SINK + n_int2, L)):
                    slot = self.ring_slot(p)
                    self.ring[s, :, 0, slot] = kx_bf[p]
                    self.ring[s, :, 1, slot] = v_bits[b, p]
                self.n_int2[s] = n_int2
                self.length[s] = L
            else:
                for t in range(n_new):
                    p = L0 + t
                    if p >= SINK and self.window_count(s) == WINDOW:
                        self.evict([s], 1)                    # the oldest window token moves to INT2
                    slot = self.ring_slot(p)
                    self.ring[s, :, 0, slot] = kx_bf[t]
                    self.ring[s, :, 1, slot] = v_bits[b, t]
                    self.length[s] = p + 1

    def evict(self, seq_ids, n_evict):
        need = 0
        for s in seq_ids:
            if self.window_count(s) < n_evict:
                raise StoreError("window holds fewer tokens")
            n0 = int(self.n_int2[s])
            for i in range(n0, n0 + n_evict):
                if i % PAGE == 0:
                    need += 1
                    if i // PAGE >= self.max_pages:
                        raise StoreError("too many pages for one sequence")
        if need > len(self.free):
            raise StoreError("out of pages")
        for s in seq_ids:
            for _ in range(n_evict):
                i = int(self.n_int2[s])
                if i % PAGE == 0:
                    self.page_table[s, i // PAGE] = self.free.popleft()
                slot = self.ring_slot(SINK + i)
                k32 = bf16_to_f64(self.ring[s, :, 0, slot]).astype(np.float32)
                v32 = bf16_to_f64(self.ring[s, :, 1, slot]).astype(np.float32)
                self._put_int2(s, i, k32[None], v32[None])
                self.n_int2[s] = i + 1

    def reset_seq(self, seq):
        n_pages = -(-int(self.n_int2[seq]) // PAGE)
        for i in range(n_pages):
            self.free.append(int(self.page_table[seq, i]))
            self.page_table[seq, i] = -1
        self.length[seq] = 0
        self.n_int2[seq] = 0

    def seq_state(self):
        return self.length.copy(), self.n_int2.copy()


def gather_tokens(pool, ring, page_table, length, n_int2, seq, kv_head):
    """Dequantized keys and values (fp64 [L, 128]) of one (seq, kv_head), position order.

    Works on any store arrays (the oracle's own, or ones exported from the GPU).
    """
    L = int(length)
    n2 = int(n_int2)
    ks, vs = [], []
    for p in range(min(L, SINK)):
        ks.append(bf16_to_f64(ring[seq, kv_head, 0, p]))
        vs.append(bf16_to_f64(ring[seq, kv_head, 1, p]))
    for pg in range(-(-n2 // PAGE)):
        page = int(page_table[seq, pg])
        n_tok = min(PAGE, n2 - pg * PAGE)
        kc, vc, kS, kL, vS, vL = layout.unpack_head_block(pool[page, kv_head], n_tok)
        ks.extend(quantizer.dequantize(kc, kS, kL))
        vs.extend(quantizer.dequantize(vc, vS, vL))
    for p in range(SINK + n2, L):
        slot = OracleStore.ring_slot(p)
        ks.append(bf16_to_f64(ring[seq, kv_head, 0, slot]))
        vs.append(bf16_to_f64(ring[seq, kv_head, 1, slot]))
    return np.array(ks).reshape(-1, D), np.array(vs).reshape(-1, D)


def evict_from_ring(ring, seq, n_int2):
    """Quantize the oldest window token (position 64 + n_int2) from a ring array.

    Returns per KV head (k_codes, k_s16, k_lo16, v_codes, v_s16, v_lo16).
    """
    slot = OracleStore.ring_slot(SINK + int(n_int2))
    k32 = bf16_to_f64(ring[seq, :, 0, slot]).astype(np.float32)
    v32 = bf16_to_f64(ring[seq, :, 1, slot]).astype(np.float32)
    kc, ks, kl = quantizer.quantize(k32, quantizer.C_K)
    vc, vs, vl = quantizer.quantize(v32, quantizer.C_V)
    return kc, ks, kl, vc, vs, vl
