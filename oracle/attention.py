"""GQA decode attention over the mixed-precision cache, by its plain definition.

Test infrastructure only (see package header).

Follows axbrief, section "어텐션 통계 기반 회전과 Triton 커널의 결합": the read
path unpacks the INT2 bytes, dequantizes, undoes the key rotation and runs
attention, all in one pass.  Because R_K is orthogonal, scoring the stored
rotated key k' = k R_K against the rotated query q' = q R_K gives exactly
q . k; this oracle rotates the query (the same scores as rotating every key
back).  Values stay in the R_V basis (R_V is folded into the output
projection), so the output is in that basis too.

Readings taken where the pages are silent:
* query head h reads KV head h // (Hq / Hkv) (consecutive GQA grouping).
* the softmax scale is passed in explicitly (1/sqrt(128) in the workloads).
* one query token per sequence attends to every stored token, the newest
  included.

``combine_partials`` is the exact merge of softmax partials computed over
disjoint token subsets (the split-K combine); the pages are silent on how the
decode kernel splits work, so this is the textbook rescaling identity.

Parity: pinned (pure-Python loops on small slices, closed forms for uniform
scores and a single token, GQA head mapping, split/merge identity, rotation
equivalence with and without the store).
"""
from __future__ import annotations

import numpy as np

from . import store as _store


def attend(q, k, v, sm_scale):
    """softmax(sm_scale * q k^T) v for one query row; fp64.  Returns (o, m, l).

    m is the maximum scaled score and l = sum exp(score - m), so o = (sum e^(s-m) v) / l.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    s = sm_scale * (k @ q)
    m = s.max()
    e = np.exp(s - m)
    l = e.sum()
    return (e @ v) / l, m, l


def combine_partials(ms, ls, os_):
    """Merge partials (m_i, l_i, o_i) of disjoint token subsets into the full output."""
    ms = np.asarray(ms, dtype=np.float64)
    ls = np.asarray(ls, dtype=np.float64)
    os_ = np.asarray(os_, dtype=np.float64)
    m = ms.max()
    w = ls * np.exp(ms - m)
    return (w[:, None] * os_).sum(axis=0) / w.sum()


def decode(pool, ring, page_table, length, n_int2, rot, q_bits, seq_ids, sm_scale, n_q_heads):
    """Decode attention for the listed sequences on store arrays (the oracle's or exported).

    rot: float32 R_K [Hkv, 128, 128]; q_bits: bf16 uint16 [n_seqs, Hq, 128].
    Returns float32 [n_seqs, Hq, 128].
    """
    rot = np.asarray(rot, dtype=np.float32).astype(np.float64)
    hkv = rot.shape[0]
    g = n_q_heads // hkv
    q = _store.bf16_to_f64(q_bits)
    out = np.zeros((len(seq_ids), n_q_heads, rot.shape[1]), dtype=np.float32)
    for b, s in enumerate(seq_ids):
        if int(length[s]) == 0:
            raise ValueError("decode over an empty sequence")
        for kv in range(hkv):
            k, v = _store.gather_tokens(pool, ring, page_table, length[s], n_int2[s], s, kv)
            for h in range(kv * g, (kv + 1) * g):
                qr = q[b, h] @ rot[kv]
                o, _, _ = attend(qr, k, v, sm_scale)
                out[b, h] = o.astype(np.float32)
    return out


def decode_store(st, q_bits, seq_ids, sm_scale, n_q_heads):
    """Decode attention on an ``OracleStore``."""
    return decode(st.pool, st.ring, st.page_table, st.length, st.n_int2, st.rot.astype(np.float32),
                  q_bits, seq_ids, sm_scale, n_q_heads)
