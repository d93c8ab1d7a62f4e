"""Byte layout of the INT2 paged store.  Test infrastructure only.

The pages say the INT2 cache keeps the paged-attention page structure (axbrief,
section "Together AI, INT2 KV 캐시 시스템 'OSCAR' 공개") and that the read path
unpacks bytes holding four 2-bit codes (axbrief, rotation section).  They give
no byte layout; this module writes out the one the library documents, from
that documentation, independently of the library's code.

One page holds 64 consecutive INT2 tokens of one sequence for every KV head of
one layer.  For KV head h the page holds a 5120-byte block at h * 5120:

  bytes    0 .. 2047  key codes    (64 tokens x 128 channels x 2 bits)
  bytes 2048 .. 4095  value codes  (64 tokens x 128 channels x 2 bits)
  bytes 4096 .. 5119  metadata     16 bytes per token j at 4096 + 16 j:
                      fp16 [sK0, loK0, sK1, loK1, sV0, loV0, sV1, loV1]
                      (scale and minimum of channel groups 0..63 and 64..127)

Both code areas are 512 little-endian 32-bit words.

Key word index for token j, channel c:
  t = j // 16, n = j % 16, g = c // 64, kq = (c % 64) // 16, u = c % 16
  word = 256 * (t // 2) + 4 * (16 * kq + n) + 2 * (t % 2) + g
  bit  = 8 * (u % 4) + 2 * (u // 4)

Value word index for token j, channel c:
  ct = c // 16, n = c % 16, s = j // 32, kq = (j % 32) // 8, kk = j % 8
  word = 256 * (ct // 4) + 4 * (16 * kq + n) + ct % 4
  bit  = 2 * (4 * s + kk // 2) + 16 * (kk % 2)

Code slots of tokens not yet written in a partially filled page are zero.

Parity: pinned (bijection of code positions, hand-derived bit positions,
round trip).
"""
from __future__ import annotations

import numpy as np

PAGE_TOKENS = 64
HEAD_DIM = 128
HEAD_BLOCK = 5120
K_CODES_OFF = 0
V_CODES_OFF = 2048
META_OFF = 4096
META_BYTES = 16
INT2_TOKEN_HEAD_BYTES = 80   # 32 B K codes + 32 B V codes + 16 B metadata
BF16_TOKEN_HEAD_BYTES = 512  # 256 B K + 256 B V


def k_code_position(j, c):
    """(word index, bit offset) of key code (token j, channel c) in the key-code area."""
    j = np.asarray(j)
    c = np.asarray(c)
    t, n = j // 16, j % 16
    g, kq, u = c // 64, (c % 64) // 16, c % 16
    word = 256 * (t // 2) + 4 * (16 * kq + n) + 2 * (t % 2) + g
    bit = 8 * (u % 4) + 2 * (u // 4)
    return word, bit


def v_code_position(j, c):
    """(word index, bit offset) of value code (token j, channel c) in the value-code area."""
    j = np.asarray(j)
    c = np.asarray(c)
    ct, n = c // 16, c % 16
    s, kq, kk = j // 32, (j % 32) // 8, j % 8
    word = 256 * (ct // 4) + 4 * (16 * kq + n) + ct % 4
    bit = 2 * (4 * s + kk // 2) + 16 * (kk % 2)
    return word, bit


def _positions_sorted(position):
    """(order, bits) so that codes.ravel()[order].reshape(512, 16) groups the 16 codes of each word."""
    jj, cc = np.meshgrid(np.arange(PAGE_TOKENS), np.arange(HEAD_DIM), indexing="ij")
    word, bit = position(jj, cc)
    key = (word * 32 + bit).ravel()
    order = np.argsort(key, kind="stable")
    return order, bit.ravel()[order].reshape(512, 16).astype(np.uint32)


_SORTED = {}


def _pack_area(codes, position) -> np.ndarray:
    if position not in _SORTED:
        _SORTED[position] = _positions_sorted(position)
    order, bits = _SORTED[position]
    c = np.asarray(codes, dtype=np.uint32).ravel()[order].reshape(512, 16)
    words = np.bitwise_or.reduce(c << bits, axis=1).astype(np.uint32)
    return words.view(np.uint8)


def _unpack_area(area, n_tokens, position) -> np.ndarray:
    words = np.asarray(area, dtype=np.uint8).view(np.uint32).astype(np.uint64)
    jj, cc = np.meshgrid(np.arange(n_tokens), np.arange(HEAD_DIM), indexing="ij")
    word, bit = position(jj, cc)
    return ((words[word] >> bit.astype(np.uint64)) & np.uint64(3)).astype(np.uint8)


def pack_head_block(k_codes, v_codes, k_s16, k_lo16, v_s16, v_lo16) -> np.ndarray:
    """One KV head's 5120-byte page block from up to 64 tokens (missing tokens are zero)."""
    n = np.asarray(k_codes).shape[0]
    assert n <= PAGE_TOKENS
    blk = np.zeros(HEAD_BLOCK, dtype=np.uint8)
    kc = np.zeros((PAGE_TOKENS, HEAD_DIM), dtype=np.uint8)
    vc = np.zeros((PAGE_TOKENS, HEAD_DIM), dtype=np.uint8)
    kc[:n] = k_codes
    vc[:n] = v_codes
    blk[K_CODES_OFF:K_CODES_OFF + 2048] = _pack_area(kc, k_code_position)
    blk[V_CODES_OFF:V_CODES_OFF + 2048] = _pack_area(vc, v_code_position)
    meta = np.zeros((PAGE_TOKENS, 8), dtype=np.float16)
    meta[:n, 0] = np.asarray(k_s16)[:, 0]
    meta[:n, 1] = np.asarray(k_lo16)[:, 0]
    meta[:n, 2] = np.asarray(k_s16)[:, 1]
    meta[:n, 3] = np.asarray(k_lo16)[:, 1]
    meta[:n, 4] = np.asarray(v_s16)[:, 0]
    meta[:n, 5] = np.asarray(v_lo16)[:, 0]
    meta[:n, 6] = np.asarray(v_s16)[:, 1]
    meta[:n, 7] = np.asarray(v_lo16)[:, 1]
    blk[META_OFF:] = meta.view(np.uint8).ravel()
    return blk


def unpack_head_block(blk, n_tokens: int = PAGE_TOKENS):
    """Inverse of ``pack_head_block`` for the first ``n_tokens`` tokens.

    Returns k_codes, v_codes (uint8 [n,128]) and k_s16, k_lo16, v_s16, v_lo16 (float16 [n,2]).
    """
    blk = np.asarray(blk, dtype=np.uint8)
    kc = _unpack_area(blk[K_CODES_OFF:K_CODES_OFF + 2048], n_tokens, k_code_position)
    vc = _unpack_area(blk[V_CODES_OFF:V_CODES_OFF + 2048], n_tokens, v_code_position)
    meta = blk[META_OFF:].view(np.float16).reshape(PAGE_TOKENS, 8)[:n_tokens]
    return kc, vc, meta[:, [0, 2]], meta[:, [1, 3]], meta[:, [4, 6]], meta[:, [5, 7]]


_GRID = {}


def _grid(position):
    """(word, bit) of every (token, channel) of a full page for one code area, computed once."""
    if position not in _GRID:
        jj, cc = np.meshgrid(np.arange(PAGE_TOKENS), np.arange(HEAD_DIM), indexing="ij")
        word, bit = position(jj, cc)
        _GRID[position] = (np.asarray(word), np.asarray(bit).astype(np.uint32))
    return _GRID[position]


def unpack_pages(blocks):
    """``unpack_head_block`` of many full page blocks at once (blocks uint8 [P, 5120]).

    Returns k_codes, v_codes (uint8 [P, 64, 128]) and k_s16, k_lo16, v_s16, v_lo16
    (float16 [P, 64, 2]); tokens past a partially filled page's count come out as stored (zero).
    """
    blocks = np.ascontiguousarray(np.asarray(blocks, dtype=np.uint8)).reshape(-1, HEAD_BLOCK)
    out = []
    for off, position in ((K_CODES_OFF, k_code_position), (V_CODES_OFF, v_code_position)):
        words = blocks[:, off:off + 2048].view(np.uint32)          # [P, 512]
        word, bit = _grid(position)
        out.append(((words[:, word] >> bit) & np.uint32(3)).astype(np.uint8))
    meta = blocks[:, META_OFF:].view(np.float16).reshape(-1, PAGE_TOKENS, 8)
    return (out[0], out[1], meta[..., [0, 2]], meta[..., [1, 3]], meta[..., [4, 6]], meta[..., [5, 7]])
