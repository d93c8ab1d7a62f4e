"""GPU parity at the workloads' full sizes, on sampled (sequence, KV head) units.

Inputs are drawn on the GPU by the counter-based generator; the oracle side redraws the
sampled units' inputs with the CPU twin (bit-identical).  The decode check runs the oracle on
the GPU's exported store (identical state); the write check compares the sampled units' INT2
pages, ring slots and the page table under the tolerance rules.
"""
import math

import numpy as np
import pytest

import parity
import synth
from test_gpu_parity import poison
from oracle import attention, store as ostore

pytestmark = pytest.mark.gpu
D = 128
SCALE = 1.0 / math.sqrt(D)


def _case(name):
    print(f"[case] {name}", flush=True)


def _unit_view(gpu, kv):
    pool, ring, table = gpu
    return pool[:, kv:kv + 1], ring[:, kv:kv + 1], table


def _iso_decode_unit(gpu, lens, n2s, rot, q, s, kv, g):
    pool, ring, table = _unit_view(gpu, kv)
    return attention.decode(pool, ring, table, lens, n2s, rot[kv:kv + 1], q[s:s + 1, kv * g:(kv + 1) * g],
                            [s], SCALE, g)[0]


def _host_bits(t):
    """bf16 bits of a device tensor drawn by the generator's GPU twin (bit-identical to the CPU twin)."""
    return t.cpu().numpy().view(np.uint16)


def _check_write_unit(gpu, rot, s, kv, kb, vb, n2):
    """One (seq, KV head) written by a first write of len(kb) tokens, against the oracle on the same
    inputs: prefill INT2 pages under the tolerance rules (key-metadata flips explained by the
    rotation error), sink ring slots and the window slots still holding prefill tokens (values
    bit-exact, keys within the rotation bound).  kb, vb: bf16 bits [L, 128]."""
    L_pre = len(kb)
    n_pre = max(0, L_pre - 320)
    gpool, gring, gtable = gpu
    pages = [int(p) for p in gtable[s, : -(-n_pre // 64)]]
    ora = ostore.OracleStore(1, 1, max(1, len(pages)), max(pages + [0]) + 1, pages, rot[kv:kv + 1])
    ora.write([0], kb[None, :, None, :], vb[None, :, None, :])
    xk = parity.quant_input_k(kb[64:64 + n_pre], rot[kv])
    xv = synth.bf16_bits_to_f32(vb[64:64 + n_pre]).astype(np.float64)
    rep = parity.compare_int2_unit(gpool, gtable[s:s + 1], ora.pool, ora.page_table, 0, kv, 0, n_pre, xk, xv,
                                   check_tail=(n_pre == n2),
                                   k_bound=parity.rotation_error_bound(kb[64:64 + n_pre], rot[kv]))
    assert rep["unexplained"] == 0, rep
    assert rep["code_mismatch"] <= max(1, 1e-4 * rep["elements"]), rep
    assert rep["v_meta_flips"] == 0 and rep["meta_far"] == 0, rep
    assert rep["k_meta_flips"] <= 1e-2 * rep["groups"], rep
    assert rep["k_meta_unexplained"] == 0, rep
    positions = np.array(list(range(min(64, L_pre))) + list(range(64 + n2, L_pre)), dtype=np.int64)
    slots = np.array([ostore.OracleStore.ring_slot(int(p)) for p in positions])
    assert np.array_equal(gring[s, kv, 1, slots], vb[positions])
    parity.check_ring_keys(gring[s, kv, 0, slots], kb[positions], rot[kv])
    print(f"[parity] unit seq={s} kv={kv}: {rep}; ring slots checked {len(slots)}", flush=True)
    return rep


def _oracle_table(n_seqs_lengths, max_pages, num_pages, free):
    """Page table the oracle allocator produces for prefill writes of the given lengths (one call each)."""
    st = ostore.OracleStore(1, len(n_seqs_lengths), max_pages, num_pages, free, np.eye(D, dtype=np.float32)[None])
    for s, L in enumerate(n_seqs_lengths):
        n_int2 = max(0, L - 320)
        for i in range(-(-n_int2 // 64)):
            st.page_table[s, i] = st.free.popleft()
    return st.page_table


def _decode_units(out, gpu, lens, n2s, rot, q, units, g):
    """Decode outputs of the listed (seq, kv) units against the oracle on the GPU's exported state."""
    worst = 0.0
    for s, kv in units:
        iso = _iso_decode_unit(gpu, lens, n2s, rot, q, s, kv, g)
        err = parity.rel_l2(out[s, kv * g:(kv + 1) * g], iso)
        print(f"[parity] decode unit seq={s} kv={kv} rel-l2 {err:.2e}", flush=True)
        assert err <= 1e-3, (s, kv, err)
        worst = max(worst, err)
    return worst


def test_qwen3_4b_full_context(gpu_lib):
    """32 q / 8 kv heads, batch 8, 32768-token context, one decode step with eviction + append."""
    import torch
    from synth import gpu as sg
    cfg, hkv, hq, B, L = synth.CFG_QWEN3_4B, 8, 32, 8, 32768
    _case("qwen3-4b full: 8 x 32768")
    rot = parity.calibrate(cfg, 0, hkv)
    max_pages = 520
    num_pages = B * max_pages
    st = gpu_lib.KVStore(hq, hkv, B, max_pages, num_pages)
    poison(st)
    st.set_rotation(rot)
    prm = sg.HeadParams(cfg, 0, hkv)
    kbuf = torch.empty((B, L + 1, hkv, D), dtype=torch.int16, device="cuda")
    vbuf = torch.empty_like(kbuf)
    for s in range(B):
        sg.draw_kv(prm, s, 0, L + 1, kbuf[s], vbuf[s])
    seqs = list(range(B))
    st.write(seqs, kbuf[:, :L].contiguous(), vbuf[:, :L].contiguous())
    before = parity.export(st)
    st.decode_write(seqs, kbuf[:, L].contiguous(), vbuf[:, L].contiguous())   # evicts, then appends
    gpu = parity.export(st)
    # allocator: one call, sequences in order, FIFO identity
    ora_t = ostore.OracleStore(1, B, max_pages, num_pages, range(num_pages), np.eye(D, dtype=np.float32)[None])
    for s in seqs:
        for i in range(-(-(L - 320) // 64)):
            ora_t.page_table[s, i] = ora_t.free.popleft()
    for s in seqs:   # eviction of INT2 index L-320 starts page 507 of each sequence, in call order
        ora_t.page_table[s, (L - 320) // 64] = ora_t.free.popleft()
    assert np.array_equal(gpu[2], ora_t.page_table)
    for s, kv in [(0, 0), (5, 6), (2, 3), (7, 7)]:
        _check_write_unit(gpu, rot, s, kv, _host_bits(kbuf[s, :L, kv]), _host_bits(vbuf[s, :L, kv]), L - 320 + 1)
    explained = 0
    for s in seqs:   # the evicted token (INT2 index L-320) of every (seq, head), on the GPU's ring
        explained += parity.check_evicted(gpu[0], gpu[2], before[1], s, L - 320)
    print(f"[parity] evictions: {B * hkv} token-heads, explained code mismatches {explained}", flush=True)
    q = synth.decode_queries(cfg, 0, B, hq, hkv)
    out = st.decode(seqs, parity.to_dev_bf16(q), SCALE).cpu().numpy()
    units = [(0, 0), (5, 6), (7, 3), (1, 1), (2, 7), (3, 2), (4, 5), (6, 4)]
    _decode_units(out, gpu, np.full(B, L + 1), np.full(B, L - 320 + 1), rot, q, units, hq // hkv)


def test_qwen3_8b_layer_100k_b32(gpu_lib):
    """One layer of the 36-layer Qwen3-8B-shaped step at full size (32 q / 8 kv heads, batch 32,
    100000-token context, shuffled physical pages), in the launch configuration the benchmark
    times: one-call decode steps (write + attention).  Page table exact; sampled units' INT2
    pages and ring, every (seq, head)'s evicted tokens, and 8 units' decode outputs against the
    oracle."""
    import torch
    from synth import gpu as sg
    cfg, hkv, hq, B, L = synth.CFG_QWEN3_8B, 8, 32, 32, 100000
    _case("qwen3-8b layer full: 32 x 100000, one-call decode step")
    rot = parity.calibrate(cfg, 0, hkv)
    max_pages = -(-(L + 2) // 64) + 1
    num_pages = B * max_pages
    free = synth.page_permutation(cfg, 0, num_pages)
    st = gpu_lib.KVStore(hq, hkv, B, max_pages, num_pages, free_pages=free)
    poison(st)
    st.set_rotation(rot)
    prm = sg.HeadParams(cfg, 0, hkv)
    kbuf = torch.empty((1, L + 2, hkv, D), dtype=torch.int16, device="cuda")
    vbuf = torch.empty_like(kbuf)
    newk = torch.empty((2, B, hkv, D), dtype=torch.int16, device="cuda")
    newv = torch.empty_like(newk)
    write_units = [(0, 0), (19, 5), (31, 2), (8, 7)]
    inputs = {}
    for s in range(B):
        sg.draw_kv(prm, s, 0, L + 2, kbuf[0], vbuf[0])
        st.write([s], kbuf[:, :L], vbuf[:, :L])
        newk[:, s] = kbuf[0, L:L + 2]
        newv[:, s] = vbuf[0, L:L + 2]
        for s2, kv in write_units:
            if s2 == s:
                inputs[(s, kv)] = (_host_bits(kbuf[0, :L, kv]), _host_bits(vbuf[0, :L, kv]))
    del kbuf, vbuf
    seqs = list(range(B))
    q = synth.decode_queries(cfg, 0, B, hq, hkv)
    qd = parity.to_dev_bf16(q)
    before = parity.export(st)
    st.decode_step(seqs, newk[0], newv[0], qd, SCALE)            # evicts INT2 index L-320, appends
    gpu = parity.export(st)
    out = st.decode_step(seqs, newk[1], newv[1], qd, SCALE).cpu().numpy()
    after = parity.export(st)
    # allocator: one write per sequence in order, then the steps' evictions (index L-320 starts
    # no page: (L-320) % 64 = 32)
    ora_t = _oracle_table([L] * B, max_pages, num_pages, free)
    assert np.array_equal(after[2], ora_t)
    for (s, kv), (kb, vb) in inputs.items():
        _check_write_unit(gpu, rot, s, kv, kb, vb, L - 320 + 1)
    explained = 0
    for s in seqs:
        explained += parity.check_evicted(gpu[0], gpu[2], before[1], s, L - 320)
        explained += parity.check_evicted(after[0], after[2], gpu[1], s, L - 320 + 1)
    print(f"[parity] evictions: {2 * B * hkv} token-heads, explained code mismatches {explained}", flush=True)
    units = [(0, 0), (19, 5), (31, 7), (4, 1), (8, 2), (12, 3), (25, 4), (28, 6)]
    _decode_units(out, after, np.full(B, L + 2), np.full(B, L - 320 + 2), rot, q, units, hq // hkv)


def _prefill_131072(gpu_lib, n_app):
    import torch
    from synth import gpu as sg
    cfg, hkv, hq, L = synth.CFG_PREFILL, 8, 32, 131072
    rot = parity.calibrate(cfg, 0, hkv)
    max_pages = -(-(L + n_app) // 64) + 1
    st = gpu_lib.KVStore(hq, hkv, 1, max_pages, max_pages)
    poison(st)
    st.set_rotation(rot)
    prm = sg.HeadParams(cfg, 0, hkv)
    kbuf = torch.empty((1, L + n_app, hkv, D), dtype=torch.int16, device="cuda")
    vbuf = torch.empty_like(kbuf)
    sg.draw_kv(prm, 0, 0, L + n_app, kbuf[0], vbuf[0])
    st.write([0], kbuf[:, :L].contiguous(), vbuf[:, :L].contiguous())
    return cfg, hkv, hq, L, rot, st, kbuf, vbuf


def test_prefill_131072_all_heads(gpu_lib):
    """One 131072-token sequence x 8 KV heads written in one call: page table, the BF16 share, and
    every head's INT2 pages and ring slots against the oracle."""
    _case("prefill 131072, all 8 heads")
    cfg, hkv, hq, L, rot, st, kbuf, vbuf = _prefill_131072(gpu_lib, 0)
    gpu = parity.export(st)
    ln, n2 = st.seq_info(0)
    assert (ln, n2) == (131072, 131072 - 320)
    assert round(100 * (ln - n2) / ln, 2) == 0.24          # the pages' 0.24 % BF16 share at 128K
    assert np.array_equal(gpu[2][0, :2043], np.arange(2043)) and (gpu[2][0, 2043:] == -1).all()
    tot = dict(elements=0, code_mismatch=0, k_meta_flips=0, groups=0)
    for kv in range(hkv):
        rep = _check_write_unit(gpu, rot, 0, kv, _host_bits(kbuf[0, :, kv]), _host_bits(vbuf[0, :, kv]), n2)
        for k in tot:
            tot[k] += rep[k]
    print(f"[parity] all heads: {tot}", flush=True)


def test_prefill_131072_then_1024_appends(gpu_lib):
    """One 131072-token sequence x 8 KV heads, then 1024 decode-step writes (evict 1 + append 1
    each): every 64th eviction checked for all heads on the GPU's own ring, the appended tokens'
    ring keys and values after the last step, the page table, and decode on the final state."""
    import torch
    n_app = 1024
    _case("prefill 131072 + 1024 appends")
    cfg, hkv, hq, L, rot, st, kbuf, vbuf = _prefill_131072(gpu_lib, n_app)
    explained = checked = 0
    for i in range(n_app):
        ring_before = None
        if i % 64 == 0 or i == n_app - 1:
            torch.cuda.synchronize()
            ring_before = st.ring_view().cpu().numpy().view(np.uint16)
        st.decode_write([0], kbuf[:, L + i].contiguous(), vbuf[:, L + i].contiguous())
        if ring_before is not None:
            after = parity.export(st)
            explained += parity.check_evicted(after[0], after[2], ring_before, 0, L - 320 + i)
            checked += 1
    gpu = parity.export(st)
    assert st.seq_info(0) == (L + n_app, L + n_app - 320)
    print(f"[parity] evictions checked {checked} x {hkv} heads, explained code mismatches {explained}", flush=True)
    n_pages_now = -(-(L + n_app - 320) // 64)
    assert np.array_equal(gpu[2][0, :n_pages_now], np.arange(n_pages_now)) and (gpu[2][0, n_pages_now:] == -1).all()
    # the window now holds appended tokens only (single-token rotation on the VALU)
    positions = np.arange(L + n_app - 256, L + n_app)
    slots = np.array([ostore.OracleStore.ring_slot(int(p)) for p in positions])
    for kv in range(hkv):
        kb = _host_bits(kbuf[0, L + n_app - 256:L + n_app, kv])
        assert np.array_equal(gpu[1][0, kv, 1, slots], _host_bits(vbuf[0, L + n_app - 256:L + n_app, kv]))
        parity.check_ring_keys(gpu[1][0, kv, 0, slots], kb, rot[kv])
    q = synth.decode_queries(cfg, 0, 1, hq, hkv)
    out = st.decode([0], parity.to_dev_bf16(q), SCALE).cpu().numpy()
    _decode_units(out, gpu, np.array([L + n_app]), np.array([L + n_app - 320]), rot, q, [(0, 0), (0, 5)],
                  hq // hkv)


def test_qwen3_32b_ragged_full(gpu_lib):
    """64 q / 8 kv heads (GQA 8), batch 16, lengths U[8192, 131072], pages scattered in the pool."""
    import torch
    from synth import gpu as sg
    cfg, hkv, hq, B = synth.CFG_QWEN3_32B, 8, 64, 16
    _case("qwen3-32b ragged full")
    lengths = [int(x) for x in synth.ragged_lengths(cfg, B, 8192, 131072)]
    rot = parity.calibrate(cfg, 0, hkv)
    max_pages = -(-131072 // 64)
    num_pages = sum(-(-(L - 320) // 64) for L in lengths) + 64
    free = synth.page_permutation(cfg, 0, num_pages)
    st = gpu_lib.KVStore(hq, hkv, B, max_pages, num_pages, free_pages=free)
    poison(st)
    st.set_rotation(rot)
    prm = sg.HeadParams(cfg, 0, hkv)
    kbuf = torch.empty((1, max(lengths), hkv, D), dtype=torch.int16, device="cuda")
    vbuf = torch.empty_like(kbuf)
    s_short, s_long = int(np.argmin(lengths)), int(np.argmax(lengths))
    inputs = {}
    for s, L in enumerate(lengths):
        sg.draw_kv(prm, s, 0, L, kbuf[0, :L], vbuf[0, :L])
        st.write([s], kbuf[:, :L], vbuf[:, :L])
        for s2, kv in ((s_short, 3), (s_long, 6)):
            if s2 == s:
                inputs[(s, kv)] = (_host_bits(kbuf[0, :L, kv]), _host_bits(vbuf[0, :L, kv]))
    del kbuf, vbuf
    gpu = parity.export(st)
    assert np.array_equal(gpu[2], _oracle_table(lengths, max_pages, num_pages, free))
    for (s, kv), (kb, vb) in inputs.items():
        _check_write_unit(gpu, rot, s, kv, kb, vb, lengths[s] - 320)
    seqs = list(range(B))
    q = synth.decode_queries(cfg, 0, B, hq, hkv)
    out = st.decode(seqs, parity.to_dev_bf16(q), SCALE).cpu().numpy()
    lens = np.array(lengths)
    units = [(s_short, 0), (s_long, 7), (3, 4), (0, 1), (5, 2), (9, 3), (12, 5), (15, 6)]
    _decode_units(out, gpu, lens, lens - 320, rot, q, units, hq // hkv)
