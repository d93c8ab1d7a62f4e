"""Pins for the CPU oracle: facts fixed by the pages or by mathematics, not by the oracle itself.

Each test is chosen so that a plausible slip in the oracle (a dropped term, a wrong sign,
index or factor order, a transposed operand) fails at least one of them.
"""
import os

import numpy as np
import pytest

import synth
from oracle import attention, calibration, layout, quantizer, store

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
D = 128


# ----------------------------------------------------------------------------- synth generator

def test_philox_known_answers():
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.txt")) as f:
        rows = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    assert rows
    for r in rows:
        v = [int(x, 16) for x in r]
        ctr, key, want = v[0:4], v[4:6], v[6:10]
        got = synth.philox4x32_10(*[np.array([c], dtype=np.uint64) for c in ctr], *key)
        assert [int(g[0]) for g in got] == want


def test_bulk_normal_moments():
    z = synth.bulk_normal(7, 3, 0, 4096).astype(np.float64)
    assert abs(z.mean()) < 0.01 and abs(z.std() - 1.0) < 0.01
    assert np.abs(z).max() < 3.47  # Irwin-Hall(4) support, scaled
    # counter-based: any slice redraws identically
    assert np.array_equal(synth.bulk_normal(7, 3, 100, 5), z[100:105].astype(np.float32))


# ----------------------------------------------------------------------------- calibration

def test_hadamard_closed_form():
    h2 = calibration.sylvester_hadamard(2)
    assert np.allclose(h2, np.array([[1, 1], [1, -1]]) / np.sqrt(2), atol=0)
    h = calibration.sylvester_hadamard(D)
    assert np.array_equal(h, h.T)
    assert np.allclose(np.abs(h), 1 / np.sqrt(D), atol=0)
    assert np.abs(h @ h.T - np.eye(D)).max() < 1e-15
    assert (h[0] > 0).all() and (h[:, 0] > 0).all()
    # Sylvester recursion H_2n = [[H, H], [H, -H]] / sqrt(2)
    h64 = calibration.sylvester_hadamard(64)
    rec = np.block([[h64, h64], [h64, -h64]]) / np.sqrt(2)
    assert np.abs(rec - h).max() < 1e-15


def test_bit_reversal():
    assert list(calibration.bit_reverse_indices(8)) == [0, 4, 2, 6, 1, 5, 3, 7]
    br = calibration.bit_reverse_indices(D)
    assert np.array_equal(br[br], np.arange(D))          # involution
    p = calibration.bit_reversal_matrix(D)
    x = np.arange(D, dtype=np.float64)
    assert np.array_equal(x @ p, x[br])                   # (x P)_j = x_br(j)
    h = calibration.sylvester_hadamard(D)
    assert np.abs(p @ h @ p - h).max() == 0               # P H P = H for the Sylvester matrix


def test_eigen_exact_covariance_input():
    basis = synth.haar(D, synth.stream(99, 0, 0, 0))
    lam = 0.9 ** np.arange(D)
    q = np.sqrt(D * lam)[:, None] * basis.T             # row i = sqrt(128 lam_i) b_i^T
    c = calibration.second_moment(q)
    assert np.abs(c - basis @ np.diag(lam) @ basis.T).max() < 1e-13
    w, u = calibration.eig_descending(c)
    assert np.abs(w - lam).max() < 1e-12
    # U = B up to column signs; after the sign rule, each column's largest entry is positive
    sgn = np.sign(basis[np.argmax(np.abs(basis), axis=0), np.arange(D)])
    assert np.abs(u - basis * sgn[None, :]).max() < 1e-8
    for j in range(D):
        assert u[np.argmax(np.abs(u[:, j])), j] > 0


def test_eigen_statistical_spectrum():
    qb = synth.calibration_queries(synth.CFG_TINY, 0, 0)       # 4096 bf16 queries
    q = synth.bf16_bits_to_f32(qb).astype(np.float64)
    c = calibration.second_moment(q)
    w, u = calibration.eig_descending(c)
    lam = 0.9 ** np.arange(D)
    rel = np.abs(w - lam) / lam
    assert rel.max() < 5 * np.sqrt(2.0 / 4096)                 # 5-sigma sampling band
    assert np.abs(c @ u - u * w[None, :]).max() < 1e-10 * np.abs(c).max()
    assert np.all(np.diff(w) <= 0)


def test_key_rotation_structure():
    q = synth.bf16_bits_to_f32(synth.calibration_queries(synth.CFG_TINY, 0, 0)).astype(np.float64)
    r, w = calibration.key_rotation(q)
    assert np.abs(r.T @ r - np.eye(D)).max() < 1e-12
    r32 = r.astype(np.float32).astype(np.float64)
    assert np.abs(r32.T @ r32 - np.eye(D)).max() < 2e-6
    c = calibration.second_moment(q)
    # factor order U.H.P: the rotated query energy is spread evenly over channels
    diag = np.diag(r.T @ c @ r)
    assert np.abs(diag - np.trace(c) / D).max() < 1e-12
    # U is recovered as R P^T H and is the (sign-canonical) eigenbasis
    h = calibration.sylvester_hadamard(D)
    p = calibration.bit_reversal_matrix(D)
    u = r @ p.T @ h
    assert np.abs(c @ u - u * w[None, :]).max() < 1e-10
    _, u_ref = calibration.eig_descending(c)
    assert np.abs(u - u_ref).max() < 1e-12


# ----------------------------------------------------------------------------- quantizer

def test_quantizer_hand_worked_ramp():
    """Group x_i = i (i = 0..63).  Exact arithmetic: lo = 63(1-c)/2, s = 63c/3.

    Keys (c = 0.96): lo = 1.26, s = 20.16, boundaries lo + (k + 1/2)s = 11.34, 31.5, 51.66
      -> codes 0 for x <= 11, 1 for 12..31, 2 for 32..51, 3 for 52..63.
    Values (c = 0.92): lo = 2.52, s = 19.32, boundaries 12.18, 31.5, 50.82
      -> codes 0 for x <= 12, 1 for 13..31, 2 for 32..50, 3 for 51..63.
    fp16 rounding of (s, lo) moves the boundaries by < 0.05, far from any integer.
    """
    x = np.concatenate([np.arange(64), np.arange(64)]).astype(np.float32)[None, :]
    ck, sk, lk = quantizer.quantize(x, quantizer.C_K)
    want_k = np.repeat([0, 1, 2, 3], [12, 20, 20, 12])
    assert np.array_equal(ck[0, :64], want_k) and np.array_equal(ck[0, 64:], want_k)
    assert abs(float(sk[0, 0]) - 20.16) < 20.16 * 2 ** -10
    assert abs(float(lk[0, 0]) - 1.26) < 1.26 * 2 ** -10
    cv, sv, lv = quantizer.quantize(x, quantizer.C_V)
    want_v = np.repeat([0, 1, 2, 3], [13, 19, 19, 13])
    assert np.array_equal(cv[0, :64], want_v)
    assert abs(float(sv[0, 0]) - 19.32) < 19.32 * 2 ** -10
    assert abs(float(lv[0, 0]) - 2.52) < 2.52 * 2 ** -10


def test_quantizer_degenerate_group():
    x = np.full((1, D), 3.25, dtype=np.float32)
    c, s, lo = quantizer.quantize(x, quantizer.C_K)
    assert (c == 0).all() and (s == 0).all() and (lo == np.float16(3.25)).all()
    assert np.array_equal(quantizer.dequantize(c, s, lo), np.full((1, D), 3.25))


def _c0_like_keys(n=2048):
    kb, vb = synth.unit_kv(synth.CFG_TINY, 0, 0, 0, n)
    return synth.bf16_bits_to_f32(kb), synth.bf16_bits_to_f32(vb)


@pytest.mark.parametrize("which", ["k", "v"])
def test_quantizer_levels_range_and_nearest(which):
    k, v = _c0_like_keys()
    x = k if which == "k" else v
    c = quantizer.C_K if which == "k" else quantizer.C_V
    codes, s16, lo16 = quantizer.quantize(x, c)
    assert codes.max() <= 3
    g = codes.reshape(-1, 2, 64)
    # clipping keeps the midpoint: both extreme levels occur in every group
    assert (g.min(axis=-1) == 0).all() and (g.max(axis=-1) == 3).all()
    # clipped width and midpoint (fp16 metadata: relative 2^-11 each)
    xg = x.reshape(-1, 2, 64).astype(np.float64)
    mn, mx = xg.min(-1), xg.max(-1)
    s, lo = s16.astype(np.float64), lo16.astype(np.float64)
    assert np.all(np.abs(3 * s - float(c) * (mx - mn)) <= 3 * s * 2 ** -10 + 1e-6)
    mid_err = np.abs(lo + 1.5 * s - 0.5 * (mn + mx))
    assert np.all(mid_err <= (np.abs(lo) + 1.5 * s) * 2 ** -10 + 1e-6)
    # brute force: the code is the nearest of the four levels, except within the band
    levels = lo[..., None] + s[..., None] * np.arange(4)
    dist = np.abs(xg[..., None] - levels[..., None, :])
    nearest = np.argmin(dist, axis=-1)
    band = quantizer.boundary_distance(x, s16, lo16).reshape(-1, 2, 64) < 1e-3
    assert np.array_equal(nearest[~band], g[~band])
    # error bound: |xhat - clamp(x, lo, lo + 3s)| <= s/2
    xhat = quantizer.dequantize(codes, s16, lo16).reshape(-1, 2, 64)
    clamped = np.clip(xg, lo[..., None], (lo + 3 * s)[..., None])
    assert np.all(np.abs(xhat - clamped) <= s[..., None] / 2 * (1 + 1e-6) + 1e-7)


# ----------------------------------------------------------------------------- layout

def test_layout_positions_golden():
    with open(os.path.join(GOLDEN, "layout_positions.txt")) as f:
        rows = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    assert len(rows) >= 8
    for area, j, c, word, bit in rows:
        fn = layout.k_code_position if area == "K" else layout.v_code_position
        w, b = fn(int(j), int(c))
        assert (int(w), int(b)) == (int(word), int(bit)), (area, j, c)


@pytest.mark.parametrize("fn", [layout.k_code_position, layout.v_code_position])
def test_layout_bijection(fn):
    jj, cc = np.meshgrid(np.arange(64), np.arange(D), indexing="ij")
    w, b = fn(jj, cc)
    assert w.min() == 0 and w.max() == 511 and (b % 2 == 0).all() and b.max() <= 30
    flat = (w * 32 + b).ravel()
    assert np.unique(flat).size == 64 * D


def test_layout_round_trip_and_saturation():
    rng = np.random.default_rng(0)
    kc = rng.integers(0, 4, (64, D), dtype=np.uint8)
    vc = rng.integers(0, 4, (64, D), dtype=np.uint8)
    meta = rng.standard_normal((4, 64, 2)).astype(np.float16)
    blk = layout.pack_head_block(kc, vc, *meta)
    assert blk.size == 5120
    out = layout.unpack_head_block(blk)
    assert np.array_equal(out[0], kc) and np.array_equal(out[1], vc)
    for a, b in zip(out[2:], meta):
        assert np.array_equal(a, b)
    full = layout.pack_head_block(np.full((64, D), 3, np.uint8), np.full((64, D), 3, np.uint8),
                                  *np.zeros((4, 64, 2), np.float16))
    assert (full[:4096] == 0xFF).all()
    # bytes per INT2 token-head: 2048/64 + 2048/64 + 16
    assert 2048 // 64 * 2 + layout.META_BYTES == layout.INT2_TOKEN_HEAD_BYTES == 80


def test_layout_partial_page_zero_tail():
    kc = np.full((5, D), 3, np.uint8)
    blk = layout.pack_head_block(kc, kc, *np.ones((4, 5, 2), np.float16))
    out = layout.unpack_head_block(blk)
    assert (out[0][5:] == 0).all() and (out[1][5:] == 0).all() and (out[2][5:] == 0).all()


# ----------------------------------------------------------------------------- store

def _rot(n_kv=1, cfg=synth.CFG_TINY):
    rs = []
    for kv in range(n_kv):
        q = synth.bf16_bits_to_f32(synth.calibration_queries(cfg, 0, kv)).astype(np.float64)
        rs.append(calibration.key_rotation(q)[0])
    return np.array(rs).astype(np.float32)


def test_bf16_share_at_128k():
    # The pages: sink + recent window are about 0.24 % of tokens at 128K context.
    st = store.OracleStore(1, 1, 4096, 4096, range(4096), np.eye(D, dtype=np.float32)[None])
    L = 131072
    n_int2 = max(0, L - store.RING_SLOTS)
    assert store.RING_SLOTS == 320 and round(100 * store.RING_SLOTS / L, 2) == 0.24
    assert L - n_int2 == 320 and -(-n_int2 // 64) == 2043
    del st


def test_bf16_to_bits_direct_rounding():
    # ties to even at the bf16 mantissa boundary, directly from fp64
    one = 1.0
    assert store.to_bf16_bits_f64(np.array([one + 2 ** -8]))[0] == 0x3F80        # tie -> even (down)
    assert store.to_bf16_bits_f64(np.array([one + 3 * 2 ** -8]))[0] == 0x3F82    # tie -> even (up)
    assert store.to_bf16_bits_f64(np.array([one + 2 ** -8 + 2 ** -40]))[0] == 0x3F81
    assert store.to_bf16_bits_f64(np.array([-2.0]))[0] == 0xC000


def test_store_routing_and_invariants():
    rot = _rot()
    kb, vb = synth.unit_kv(synth.CFG_TINY, 0, 0, 0, 1024)
    st = store.OracleStore(1, 2, 64, 64, range(64), rot)
    st.write([0], kb[None, :, None, :], vb[None, :, None, :])
    assert st.length[0] == 1024 and st.n_int2[0] == 704 and st.window_count(0) == 256
    assert list(st.page_table[0, :11]) == list(range(11)) and st.page_table[0, 11] == -1
    # sink / window hold bf16(k R), values as given
    x = synth.bf16_bits_to_f32(kb).astype(np.float64) @ rot[0].astype(np.float64)
    for p in (0, 63, 768, 1023):
        slot = st.ring_slot(p)
        assert np.array_equal(st.ring[0, 0, 1, slot], vb[p])
        assert np.array_equal(st.ring[0, 0, 0, slot], store.to_bf16_bits_f64(x[p]))
    # an INT2 token decodes to its clipped rotated key within half a step
    kc, vc, ks, kl, vs, vl = layout.unpack_head_block(st.pool[5, 0])
    tok = 64 + 5 * 64 + 7
    xh = quantizer.dequantize(kc[7:8], ks[7:8], kl[7:8])[0]
    s = np.repeat(ks[7].astype(np.float64), 64)
    lo = np.repeat(kl[7].astype(np.float64), 64)
    assert np.all(np.abs(xh - np.clip(x[tok], lo, lo + 3 * s)) <= s / 2 * (1 + 1e-6))
    # a full window refuses a further append and leaves the store unchanged
    before = (st.ring.copy(), st.length.copy())
    with pytest.raises(store.StoreError):
        st.write([0], kb[None, :1, None, :], vb[None, :1, None, :])
    assert np.array_equal(before[0], st.ring) and np.array_equal(before[1], st.length)
    # evict one, append one: invariants hold
    st.evict([0], 1)
    st.write([0], kb[None, :1, None, :], vb[None, :1, None, :])
    assert st.n_int2[0] == 705 and st.length[0] == 1025 and st.window_count(0) == 256
    assert st.page_table[0, 11] == 11


def test_store_allocator_fifo_order_and_errors():
    rot = np.eye(D, dtype=np.float32)[None]
    free = [9, 3, 7, 1, 0, 2, 4, 5, 6, 8]
    st = store.OracleStore(1, 3, 8, 10, free, rot)
    kb, vb = synth.unit_kv(synth.CFG_TINY, 0, 0, 0, 320 + 130)
    kb2 = np.stack([kb, kb])[:, :, None, :]
    vb2 = np.stack([vb, vb])[:, :, None, :]
    st.write([2, 0], kb2, vb2)                      # 130 INT2 tokens -> 3 pages each
    assert list(st.page_table[2, :3]) == [9, 3, 7] and list(st.page_table[0, :3]) == [1, 0, 2]
    st.evict([0, 2], 62)                            # 130 + 62 = 192: no new page
    assert st.page_table[0, 3] == -1
    st.evict([0, 2], 1)                             # index 192 -> one page each
    assert st.page_table[0, 3] == 4 and st.page_table[2, 3] == 5
    # not enough pages for 2 more sequences' pages: nothing changes
    snap = st.page_table.copy()
    with pytest.raises(store.StoreError):
        st.evict([0, 2], 64 * 2)
    assert np.array_equal(snap, st.page_table)
    st.reset_seq(2)
    assert (st.page_table[2] == -1).all() and list(st.free) == [6, 8, 9, 3, 7, 5]
    # invariants: L = sink + n_int2 + window
    L, n2 = st.seq_state()
    assert L[0] == 64 + n2[0] + st.window_count(0)


def test_evicting_write_is_token_by_token_evict_and_append():
    """An overflowing write with evicting writes on reaches the state of appending its tokens one at
    a time with an explicit one-token eviction whenever the window holds 256 (the decode step's
    order), with 320 tokens left BF16; a token that fits never evicts."""
    rot = _rot()
    kb, vb = synth.unit_kv(synth.CFG_TINY, 0, 0, 0, 1500)
    K, V = kb[None, :, None, :], vb[None, :, None, :]
    a = store.OracleStore(1, 1, 32, 32, range(32), rot)
    b = store.OracleStore(1, 1, 32, 32, range(32), rot)
    a.write_evicts = True
    for st in (a, b):
        st.write([0], K[:, :40], V[:, :40])
    a.write([0], K[:, 40:900], V[:, 40:900])           # sink fill, window fill, 540 evictions
    a.write([0], K[:, 900:1500], V[:, 900:1500])
    for t in range(40, 1500):
        if b.window_count(0) == 256:
            b.evict([0], 1)
        b.write([0], K[:, t:t + 1], V[:, t:t + 1])
    assert np.array_equal(a.pool, b.pool) and np.array_equal(a.ring, b.ring)
    assert np.array_equal(a.page_table, b.page_table) and list(a.free) == list(b.free)
    assert (a.length[0], a.n_int2[0], a.window_count(0)) == (1500, 1500 - 320, 256)
    # a write that fits the free slots evicts nothing
    c = store.OracleStore(1, 1, 32, 32, range(32), rot)
    c.write_evicts = True
    c.write([0], K[:, :10], V[:, :10])
    c.write([0], K[:, 10:320], V[:, 10:320])
    assert c.n_int2[0] == 0 and c.window_count(0) == 256


def test_evict_quantizes_ring_value():
    rot = _rot()
    kb, vb = synth.unit_kv(synth.CFG_TINY, 0, 0, 0, 320)
    st = store.OracleStore(1, 1, 4, 4, [3, 2, 1, 0], rot)
    st.write([0], kb[None, :, None, :], vb[None, :, None, :])
    assert st.n_int2[0] == 0 and st.window_count(0) == 256
    ring_k = store.bf16_to_f64(st.ring[0, 0, 0, 64]).astype(np.float32)
    st.evict([0], 1)
    assert st.page_table[0, 0] == 3 and st.n_int2[0] == 1
    kc, vc, ks, kl, vs, vl = layout.unpack_head_block(st.pool[3, 0], 1)
    c2, s2, l2 = quantizer.quantize(ring_k[None], quantizer.C_K)
    assert np.array_equal(kc, c2) and np.array_equal(ks, s2) and np.array_equal(kl, l2)
    # rest of the fresh page is zero
    full = layout.unpack_head_block(st.pool[3, 0])
    assert (full[0][1:] == 0).all()


# ----------------------------------------------------------------------------- attention

def _attend_loops(q, ks, vs, scale):
    """Pure-Python loops, no NumPy: softmax(scale q.k) v."""
    scores = [scale * sum(qi * ki for qi, ki in zip(q, k)) for k in ks]
    m = max(scores)
    e = [pow(2.718281828459045, s - m) for s in scores]
    tot = sum(e)
    return [sum(e[j] * vs[j][c] for j in range(len(vs))) / tot for c in range(len(vs[0]))]


def test_attend_matches_pure_python_loops():
    rng = np.random.default_rng(1)
    for n in (1, 3, 8):
        q = rng.standard_normal(D)
        k = rng.standard_normal((n, D)) * 3
        v = rng.standard_normal((n, D))
        o, _, _ = attention.attend(q, k, v, 1 / np.sqrt(D))
        ref = _attend_loops(list(q), [list(r) for r in k], [list(r) for r in v], 1 / np.sqrt(D))
        assert np.abs(o - np.array(ref)).max() < 1e-12


def test_attend_closed_forms():
    rng = np.random.default_rng(2)
    v = rng.standard_normal((37, D))
    k = rng.standard_normal((37, D))
    o, m, l = attention.attend(np.zeros(D), k, v, 0.1)       # equal scores -> mean of values
    assert np.abs(o - v.mean(axis=0)).max() < 1e-14 and m == 0 and abs(l - 37) < 1e-12
    o1, _, _ = attention.attend(rng.standard_normal(D), k[:1], v[:1], 0.1)
    assert np.abs(o1 - v[0]).max() < 1e-15


def test_split_combine_identity():
    rng = np.random.default_rng(3)
    q = rng.standard_normal(D)
    k = rng.standard_normal((500, D)) * 2
    v = rng.standard_normal((500, D))
    full, _, _ = attention.attend(q, k, v, 1 / np.sqrt(D))
    cuts = np.sort(rng.choice(np.arange(1, 500), 6, replace=False))
    parts = np.split(np.arange(500), cuts)
    os_, ms, ls = zip(*[attention.attend(q, k[p], v[p], 1 / np.sqrt(D)) for p in parts])
    assert np.abs(attention.combine_partials(ms, ls, os_) - full).max() < 1e-12


def test_rotation_is_attention_exact():
    rng = np.random.default_rng(4)
    r = _rot()[0].astype(np.float64)
    r = np.linalg.qr(r)[0]   # exactly orthogonal in fp64
    rv = synth.haar(D, rng)
    q = rng.standard_normal(D)
    k = rng.standard_normal((300, D)) * 2
    v = rng.standard_normal((300, D))
    o, _, _ = attention.attend(q, k, v, 1 / np.sqrt(D))
    o_r, _, _ = attention.attend(q @ r, k @ r, v @ rv, 1 / np.sqrt(D))
    assert np.abs(o_r - o @ rv).max() < 1e-12


def test_decode_bf16_store_matches_unquantized_attention():
    """L <= 320 keeps every token BF16: decode == plain attention up to bf16 key rounding."""
    rot = _rot(2)
    n_q = 4
    kb = np.stack([synth.unit_kv(synth.CFG_TINY, 0, 0, kv, 300)[0] for kv in range(2)], axis=1)
    vb = np.stack([synth.unit_kv(synth.CFG_TINY, 0, 0, kv, 300)[1] for kv in range(2)], axis=1)
    st = store.OracleStore(2, 1, 4, 4, range(4), rot)
    st.write([0], kb[None], vb[None])
    qb = synth.decode_queries(synth.CFG_TINY, 0, 1, n_q, 2)
    out = attention.decode_store(st, qb, [0], 1 / np.sqrt(D), n_q)
    q = synth.bf16_bits_to_f32(qb).astype(np.float64)
    k = synth.bf16_bits_to_f32(kb).astype(np.float64)
    v = synth.bf16_bits_to_f32(vb).astype(np.float64)
    for h in range(n_q):
        kv = h // 2                                  # consecutive GQA grouping
        o, _, _ = attention.attend(q[0, h], k[:, kv], v[:, kv], 1 / np.sqrt(D))
        err = np.linalg.norm(out[0, h] - o) / np.linalg.norm(o)
        assert err < 2e-2, (h, err)
        other, _, _ = attention.attend(q[0, h], k[:, 1 - kv], v[:, 1 - kv], 1 / np.sqrt(D))
        assert np.linalg.norm(out[0, h] - other) / np.linalg.norm(other) > 0.3


def test_key_mean_transform_is_attention_exact():
    """The write path's key transform with a key mean, (k - mu) . R_K (oracle store.rotate_keys),
    with queries rotated by R_K alone: every score of a query moves by the same -q . mu, so the
    attention output equals plain attention over the raw keys to 1e-12 (gist.science summary of
    OptR, solution section, step 1).  A per-token centring (each key minus its own channel mean)
    is not exact: it is rejected."""
    rng = np.random.default_rng(21)
    r = np.linalg.qr(_rot()[0].astype(np.float64))[0]   # exactly orthogonal in fp64
    k = rng.standard_normal((400, D)) * 1.5 + rng.standard_normal(D) * 4
    v = rng.standard_normal((400, D))
    mu = k.mean(axis=0).astype(np.float32)
    x = store.rotate_keys(k[:, None, :], r[None], mu[None])[:, 0, :]
    assert np.abs(x - (k - mu.astype(np.float64)) @ r).max() < 1e-12 * np.abs(x).max()
    for _ in range(5):
        q = rng.standard_normal(D)
        o, _, _ = attention.attend(q, k, v, 1 / np.sqrt(D))
        o_m, _, _ = attention.attend(q @ r, x, v, 1 / np.sqrt(D))
        assert np.abs(o_m - o).max() <= 1e-12 * max(1.0, np.abs(o).max())
        bad = (k - k.mean(axis=1, keepdims=True)) @ r
        o_b, _, _ = attention.attend(q @ r, bad, v, 1 / np.sqrt(D))
        assert np.abs(o_b - o).max() > 1e-3


def test_decode_bf16_store_with_key_mean_matches_unquantized_attention():
    """With a key mean set, an all-BF16 store (L <= 320) holds bf16((k - mu) . R_K) and decodes to
    plain attention over the raw keys up to the bf16 rounding of the stored keys."""
    rot = _rot(2)
    n_q = 4
    kb = np.stack([synth.unit_kv(synth.CFG_TINY, 0, 0, kv, 300)[0] for kv in range(2)], axis=1)
    vb = np.stack([synth.unit_kv(synth.CFG_TINY, 0, 0, kv, 300)[1] for kv in range(2)], axis=1)
    k = synth.bf16_bits_to_f32(kb).astype(np.float64)
    v = synth.bf16_bits_to_f32(vb).astype(np.float64)
    mu = (k.mean(axis=0) + 3.0).astype(np.float32)            # [2, 128], off the keys' centre
    st = store.OracleStore(2, 1, 4, 4, range(4), rot)
    st.set_key_mean(mu)
    st.write([0], kb[None], vb[None])
    want = store.to_bf16_bits_f64(store.rotate_keys(k, rot.astype(np.float64), mu))
    assert np.array_equal(st.ring[0, :, 0, :300], want.transpose(1, 0, 2))
    qb = synth.decode_queries(synth.CFG_TINY, 0, 1, n_q, 2)
    out = attention.decode_store(st, qb, [0], 1 / np.sqrt(D), n_q)
    q = synth.bf16_bits_to_f32(qb).astype(np.float64)
    for h in range(n_q):
        kv = h // 2
        o, _, _ = attention.attend(q[0, h], k[:, kv], v[:, kv], 1 / np.sqrt(D))
        assert np.linalg.norm(out[0, h] - o) / np.linalg.norm(o) < 2e-2, h


def test_decode_gqa_mapping_uniform_scores():
    """Zero queries give uniform attention: head h returns the mean value of KV head h // g."""
    rot = np.stack([np.eye(D, dtype=np.float32)] * 2)
    st = store.OracleStore(2, 1, 8, 8, range(8), rot)
    rng = np.random.default_rng(5)
    vb = synth.f32_to_bf16_bits(rng.standard_normal((1, 40, 2, D)).astype(np.float32))
    kb = synth.f32_to_bf16_bits(rng.standard_normal((1, 40, 2, D)).astype(np.float32))
    st.write([0], kb, vb)
    out = attention.decode_store(st, np.zeros((1, 8, D), np.uint16), [0], 0.1, 8)
    vm = synth.bf16_bits_to_f32(vb[0]).astype(np.float64).mean(axis=0)    # [2, D]
    for h in range(8):
        assert np.abs(out[0, h] - vm[h // 4]).max() < 1e-6


# ----------------------------------------------------------------------------- value rotation
def _softmax_rows(z):
    z = z - z.max(axis=1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=1, keepdims=True)


def test_value_moment_is_second_moment_of_attention_outputs():
    """The printed C_S = (1/N) V^T S^T S V equals the second moment of the calibration attention
    outputs computed one query at a time by the attention routine."""
    rng = np.random.default_rng(11)
    q = rng.standard_normal((40, D))
    k = rng.standard_normal((300, D))
    v = rng.standard_normal((300, D)) + rng.standard_normal(D)
    scale = 1 / np.sqrt(D)
    s = _softmax_rows(scale * q @ k.T)
    outs = np.stack([attention.attend(qi, k, v, scale)[0] for qi in q])
    c_ref = sum(np.outer(o, o) for o in outs) / len(outs)
    assert np.abs(calibration.value_moment(s, v) - c_ref).max() < 1e-12 * np.abs(c_ref).max()


def test_value_rotation_closed_form_eigenbasis():
    """S = identity and values whose rows are sqrt(128 lam_i) b_i^T: C_S = B diag(lam) B^T, so
    U_S is B (up to the sign rule) and R_V = B . H . P_br."""
    basis = synth.haar(D, synth.stream(98, 0, 0, 0))
    lam = (D - np.arange(D)) / D          # distinct, well separated: eigenvectors well conditioned
    v = np.sqrt(D * lam)[:, None] * basis.T
    r, w = calibration.value_rotation(np.eye(D), v)
    assert np.abs(w - lam).max() < 1e-12
    sgn = np.sign(basis[np.argmax(np.abs(basis), axis=0), np.arange(D)])
    expect = (basis * sgn[None, :]) @ calibration.sylvester_hadamard(D) @ calibration.bit_reversal_matrix(D)
    assert np.abs(r - expect).max() < 1e-8
    assert np.abs(r.T @ r - np.eye(D)).max() < 1e-12


def test_value_rotation_and_fold_are_output_exact():
    """Values stored as v . R_V give attention outputs o . R_V; the folded output projection
    R_V^T . W_O turns them back into the original layer output (fp64)."""
    rng = np.random.default_rng(12)
    hq, hkv, d_model = 4, 2, 96
    g = hq // hkv
    r_v = []
    for h in range(hkv):
        s = _softmax_rows(rng.standard_normal((50, 200)) * 3)
        r, _ = calibration.value_rotation(s, rng.standard_normal((200, D)) * (1 + np.arange(D) / 16))
        r_v.append(r)
    r_v = np.stack(r_v)
    w_v = rng.standard_normal((d_model, hkv * D))
    w_o = rng.standard_normal((hq * D, d_model))
    w_v2, w_o2 = calibration.fold_value_rotation(w_v, w_o, r_v, hq, hkv)
    x = rng.standard_normal((300, d_model))          # token activations
    k = rng.standard_normal((hkv, 300, D))
    q = rng.standard_normal((hq, D))
    ref = np.zeros(d_model)
    got = np.zeros(d_model)
    for j in range(hq):
        h = j // g
        v = x @ w_v[:, h * D:(h + 1) * D]
        v2 = x @ w_v2[:, h * D:(h + 1) * D]
        assert np.abs(v2 - v @ r_v[h]).max() < 1e-11 * np.abs(v).max()
        o, _, _ = attention.attend(q[j], k[h], v, 1 / np.sqrt(D))
        o2, _, _ = attention.attend(q[j], k[h], v2, 1 / np.sqrt(D))
        ref += o @ w_o[j * D:(j + 1) * D]
        got += o2 @ w_o2[j * D:(j + 1) * D]
    assert np.abs(got - ref).max() < 1e-10 * np.abs(ref).max()


# ----------------------------------------------------------------------------- code decision and the
# parity band

def _group_with(s_target, lo_target, ts):
    """A 64-value group whose clipped range gives fp32 parameters near (s_target, lo_target) under
    c_K, with the listed values placed at t = (x - lo16) / s16 (filled up with t = 1)."""
    # mn, mx such that c r = 3 s and mn + (r - c r) / 2 = lo: r = 3 s / c, mn = lo - (1 - c) r / 2
    c = float(quantizer.C_K)
    r = 3.0 * s_target / c
    mn = lo_target - 0.5 * (1.0 - c) * r
    x = np.full(64, mn, np.float32)
    x[1] = np.float32(mn + r)
    _, _, s16, lo16 = quantizer.params(np.concatenate([x, x])[None], quantizer.C_K)
    s, lo = float(s16[0, 0]), float(lo16[0, 0])
    vals = np.array([lo + t * s for t in ts], np.float64)
    assert np.all(vals.astype(np.float32).astype(np.float64) == vals), "placed values must be exact in fp32"
    x[2:2 + len(ts)] = vals.astype(np.float32)
    x[2 + len(ts):] = np.float32(lo + s)
    row = np.concatenate([x, x])[None]
    return row, s, lo


def test_code_decision_ties_and_boundary_distance():
    """Hand-placed values around each rounding boundary b in {0.5, 1.5, 2.5}: the code is the
    exact fp64 decision with ties to even, and boundary_distance returns the placement offset.
    Scale and minimum: s16 = 1, lo16 = -1 exactly (r = 3.125, c_K: w = 3, half = 1/16), and a
    second group whose fp32 scale 0.9921875... is not an fp16 number, so that a distance or a code
    taken with the fp32 parameters instead of the stored fp16 ones fails."""
    want = [0, 2, 2, 1, 1, 3, 2, 0, 3, 1]
    # offsets small enough to be exact in fp32 with each group's fp16 scale
    for s_t, lo_t, d in ((1.0, -1.0, 2.0 ** -16), (0.99, 0.37, 2.0 ** -9)):
        ts = [0.5, 1.5, 2.5, 0.5 + d, 1.5 - d, 2.5 + d, 2.5 - d, 0.0, 3.0, 1.25]
        want_dist = [0, 0, 0, d, d, d, d, 0.5, 0.5, 0.25]
        row, s, lo = _group_with(s_t, lo_t, ts)
        s32, lo32, s16, lo16 = quantizer.params(row, quantizer.C_K)
        if s_t == 1.0:
            assert (s, lo) == (1.0, -1.0) and float(s32[0, 0]) == 1.0 and float(lo32[0, 0]) == -1.0
        else:
            assert float(s32[0, 0]) != s       # the stored scale differs from the fp32 one
        codes, _, _ = quantizer.quantize(row, quantizer.C_K)
        assert list(codes[0, 2:2 + len(ts)]) == want, (s_t, codes[0, 2:2 + len(ts)])
        dist = quantizer.boundary_distance(row, s16, lo16)[0, 2:2 + len(ts)]
        assert np.abs(dist - np.array(want_dist)).max() < 1e-12, dist
    # a group whose scale rounds to fp16 zero: distance +inf, every code 0
    tiny = np.full((1, D), 1.0, np.float32)
    tiny[0, :64:2] += np.float32(1e-8)
    c0, s0, l0 = quantizer.quantize(tiny, quantizer.C_K)
    assert float(s0[0, 0]) == 0 and (c0 == 0).all()
    assert np.isinf(quantizer.boundary_distance(tiny, s0, l0)[0, :64]).all()


def test_store_partial_last_page_decode_by_hand():
    """A store holding 64 sink + 145 INT2 (two full pages and a 17-token page, shuffled physical
    pages) + 256 window tokens, decoded by the oracle, against a hand-built cache: each position
    routed by its index, INT2 tokens dequantized element by element as lo16 + s16 * code from the
    quantizer's output on fp32(k R) (values on v), BF16 tokens from bf16(k R) / v, and attention
    by pure-Python loops."""
    import math
    hkv, hq, L = 2, 4, 320 + 2 * 64 + 17
    rot = _rot(hkv)
    kb = np.stack([synth.unit_kv(synth.CFG_TINY, 0, 3, kv, L)[0] for kv in range(hkv)], axis=1)
    vb = np.stack([synth.unit_kv(synth.CFG_TINY, 0, 3, kv, L)[1] for kv in range(hkv)], axis=1)
    free = [5, 2, 7, 0, 3, 6, 1, 4]
    st = store.OracleStore(hkv, 2, 4, 8, free, rot)
    st.write([1], kb[None], vb[None])
    assert st.n_int2[1] == 145 and list(st.page_table[1, :3]) == [5, 2, 7]
    qb = synth.decode_queries(synth.CFG_TINY, 0, 1, hq, hkv)
    out = attention.decode_store(st, qb, [1], 1 / math.sqrt(D), hq)
    q = synth.bf16_bits_to_f32(qb).astype(np.float64)[0]
    g = hq // hkv
    for kv in range(hkv):
        k = synth.bf16_bits_to_f32(kb[:, kv]).astype(np.float64)
        v = synth.bf16_bits_to_f32(vb[:, kv]).astype(np.float64)
        x = k @ rot[kv].astype(np.float64)
        kc, ks, kl = quantizer.quantize(x[64:209].astype(np.float32), quantizer.C_K)
        vc, vs, vl = quantizer.quantize(v[64:209].astype(np.float32), quantizer.C_V)
        keys, vals = [], []
        for p in range(L):
            if 64 <= p < 209:
                i = p - 64
                keys.append([float(kl[i, c // 64]) + float(ks[i, c // 64]) * int(kc[i, c]) for c in range(D)])
                vals.append([float(vl[i, c // 64]) + float(vs[i, c // 64]) * int(vc[i, c]) for c in range(D)])
            else:
                keys.append(list(store.bf16_to_f64(store.to_bf16_bits_f64(x[p]))))
                vals.append(list(v[p]))
        for h in range(kv * g, (kv + 1) * g):
            qr = list(q[h] @ rot[kv].astype(np.float64))
            scores = [sum(a * b for a, b in zip(qr, kk)) / math.sqrt(D) for kk in keys]
            m = max(scores)
            e = [math.exp(s_ - m) for s_ in scores]
            tot = sum(e)
            ref = [sum(e[j] * vals[j][c] for j in range(L)) / tot for c in range(D)]
            assert np.abs(out[0, h] - np.array(ref)).max() < 1e-6 * np.abs(ref).max() + 1e-7, (kv, h)


def test_layout_batched_unpack_equals_per_block():
    """The batched page unpack used by the full-size comparisons returns what the per-block
    unpack (pinned above by hand-derived positions and the round trip) returns, page by page."""
    rng = np.random.default_rng(21)
    blocks = []
    for n in (64, 64, 17, 1):
        kc = rng.integers(0, 4, (n, D), dtype=np.uint8)
        vc = rng.integers(0, 4, (n, D), dtype=np.uint8)
        meta = [rng.standard_normal((n, 2)).astype(np.float16) for _ in range(4)]
        blocks.append(layout.pack_head_block(kc, vc, *meta))
    batched = layout.unpack_pages(np.stack(blocks))
    for i, blk in enumerate(blocks):
        for a, b in zip(batched, layout.unpack_head_block(blk)):
            assert np.array_equal(np.ascontiguousarray(a[i]).view(np.uint8), np.ascontiguousarray(b).view(np.uint8))
