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
from oracle import attention, layout, store as ostore

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


def _check_write_unit(gpu, cfg, layer, s, kv, L_pre, rot, table_row, n2):
    """Prefill INT2 pages + ring of one unit vs the oracle on the CPU twin's inputs."""
    kb, vb = synth.unit_kv(cfg, layer, s, kv, L_pre)
    pages = [int(p) for p in table_row[: -(-max(0, L_pre - 320) // 64)]]
    n_pages = max(1, len(pages))
    ora = ostore.OracleStore(1, 1, n_pages, max(pages + [0]) + 1, pages, rot[kv:kv + 1])
    ora.write([0], kb[None, :, None, :], vb[None, :, None, :])
    n_pre = max(0, L_pre - 320)
    xk = parity.quant_input_k(kb[64:64 + n_pre], rot[kv])
    xv = synth.bf16_bits_to_f32(vb[64:64 + n_pre]).astype(np.float64)
    gpool, gring, gtable = gpu
    gt = gtable[s:s + 1]
    rep = parity.compare_int2_unit(gpool, gt, ora.pool, ora.page_table, 0, kv, 0, n_pre, xk, xv,
                                   check_tail=(n_pre == n2))
    assert rep["unexplained"] == 0, rep
    assert rep["code_mismatch"] <= max(1, 1e-4 * rep["elements"]), rep
    assert rep["v_meta_flips"] == 0 and rep["meta_far"] == 0, rep
    assert rep["k_meta_flips"] <= 1e-2 * rep["groups"], rep
    # sink ring slots: values bit-exact
    assert np.array_equal(gring[s, kv, 1, :64], vb[:64])
    print(f"[parity] unit seq={s} kv={kv}: {rep}", flush=True)
    return rep


def _oracle_table(n_seqs_lengths, max_pages, num_pages, free):
    """Page table the oracle allocator produces for prefill writes of the given lengths (one call each)."""
    st = ostore.OracleStore(1, len(n_seqs_lengths), max_pages, num_pages, free, np.eye(D, dtype=np.float32)[None])
    for s, L in enumerate(n_seqs_lengths):
        n_int2 = max(0, L - 320)
        for i in range(-(-n_int2 // 64)):
            st.page_table[s, i] = st.free.popleft()
    return st.page_table


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
    for s, kv in [(0, 0), (5, 6)]:
        _check_write_unit(gpu, cfg, 0, s, kv, L, rot, gpu[2][s], L - 320 + 1)
        # evicted token (INT2 index L-320) vs the oracle on the GPU's ring before eviction
        kc, ksc, klo, vc, vsc, vlo = ostore.evict_from_ring(before[1], s, L - 320)
        blk = layout.unpack_head_block(gpu[0][gpu[2][s, (L - 320) // 64], kv])
        j = (L - 320) % 64
        assert np.array_equal(blk[0][j], kc[kv]) and np.array_equal(blk[1][j], vc[kv])
        assert np.array_equal(blk[2][j], ksc[kv]) and np.array_equal(blk[5][j], vlo[kv])
    q = synth.decode_queries(cfg, 0, B, hq, hkv)
    out = st.decode(seqs, parity.to_dev_bf16(q), SCALE).cpu().numpy()
    lens = np.full(B, L + 1)
    n2s = np.full(B, L - 320 + 1)
    g = hq // hkv
    for s, kv in [(0, 0), (5, 6), (7, 3)]:
        iso = _iso_decode_unit(gpu, lens, n2s, rot, q, s, kv, g)
        err = parity.rel_l2(out[s, kv * g:(kv + 1) * g], iso)
        print(f"[parity] decode unit seq={s} kv={kv} rel-l2 {err:.2e}", flush=True)
        assert err <= 1e-3


def test_qwen3_8b_layer_100k_b32(gpu_lib):
    """One layer of the 36-layer Qwen3-8B-shaped step at full size (32 q / 8 kv heads, batch 32,
    100000-token context, shuffled physical pages), in the launch configuration the benchmark
    times: one-call decode steps (write + attention).  Page table exact; sampled units' INT2
    pages, evicted tokens and decode outputs against the oracle."""
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
    for s in range(B):
        sg.draw_kv(prm, s, 0, L + 2, kbuf[0], vbuf[0])
        st.write([s], kbuf[:, :L], vbuf[:, :L])
        newk[:, s] = kbuf[0, L:L + 2]
        newv[:, s] = vbuf[0, L:L + 2]
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
    for s, kv in [(0, 0), (19, 5)]:
        _check_write_unit(gpu, cfg, 0, s, kv, L, rot, gpu[2][s], L - 320 + 1)
        kc, ksc, klo, vc, vsc, vlo = ostore.evict_from_ring(before[1], s, L - 320)
        blk = layout.unpack_head_block(gpu[0][gpu[2][s, (L - 320) // 64], kv])
        j = (L - 320) % 64
        assert np.array_equal(blk[0][j], kc[kv]) and np.array_equal(blk[1][j], vc[kv])
        assert np.array_equal(blk[2][j], ksc[kv]) and np.array_equal(blk[3][j], klo[kv])
        assert np.array_equal(blk[4][j], vsc[kv]) and np.array_equal(blk[5][j], vlo[kv])
    lens = np.full(B, L + 2)
    n2s = np.full(B, L - 320 + 2)
    g = hq // hkv
    for s, kv in [(0, 0), (19, 5), (31, 7)]:
        iso = _iso_decode_unit(after, lens, n2s, rot, q, s, kv, g)
        err = parity.rel_l2(out[s, kv * g:(kv + 1) * g], iso)
        print(f"[parity] decode unit seq={s} kv={kv} rel-l2 {err:.2e}", flush=True)
        assert err <= 1e-3


def test_prefill_131072_then_1024_appends(gpu_lib):
    """One 131072-token sequence x 8 KV heads, then 1024 decode-step writes (evict 1 + append 1 each)."""
    import torch
    from synth import gpu as sg
    cfg, hkv, hq, L, n_app = synth.CFG_PREFILL, 8, 32, 131072, 1024
    _case("prefill 131072 + 1024 appends")
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
    gpu = parity.export(st)
    ln, n2 = st.seq_info(0)
    assert (ln, n2) == (131072, 131072 - 320)
    assert round(100 * (ln - n2) / ln, 2) == 0.24          # the pages' 0.24 % BF16 share at 128K
    assert np.array_equal(gpu[2][0, :2043], np.arange(2043)) and gpu[2][0, 2043] == -1
    for kv in (0, 7):
        _check_write_unit(gpu, cfg, 0, 0, kv, L, rot, gpu[2][0], n2)
    ring_before = None
    for i in range(n_app):
        if i == n_app - 1:
            ring_before = parity.export(st)[1]
        st.decode_write([0], kbuf[:, L + i].contiguous(), vbuf[:, L + i].contiguous())
    gpu = parity.export(st)
    assert st.seq_info(0) == (L + n_app, L + n_app - 320)
    n_pages_now = -(-(L + n_app - 320) // 64)
    assert np.array_equal(gpu[2][0, :n_pages_now], np.arange(n_pages_now)) and (gpu[2][0, n_pages_now:] == -1).all()
    idx = L + n_app - 320 - 1
    kc, ksc, klo, vc, vsc, vlo = ostore.evict_from_ring(ring_before, 0, idx)
    for kv in range(hkv):
        blk = layout.unpack_head_block(gpu[0][gpu[2][0, idx // 64], kv])
        j = idx % 64
        assert np.array_equal(blk[0][j], kc[kv]) and np.array_equal(blk[1][j], vc[kv])
        assert np.array_equal(blk[2][j], ksc[kv]) and np.array_equal(blk[3][j], klo[kv])
    q = synth.decode_queries(cfg, 0, 1, hq, hkv)
    out = st.decode([0], parity.to_dev_bf16(q), SCALE).cpu().numpy()
    g = hq // hkv
    for kv in (0, 5):
        iso = _iso_decode_unit(gpu, np.array([L + n_app]), np.array([L + n_app - 320]), rot, q, 0, kv, g)
        assert parity.rel_l2(out[0, kv * g:(kv + 1) * g], iso) <= 1e-3


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
    for s, L in enumerate(lengths):
        sg.draw_kv(prm, s, 0, L, kbuf[0, :L], vbuf[0, :L])
        st.write([s], kbuf[:, :L], vbuf[:, :L])
    del kbuf, vbuf
    gpu = parity.export(st)
    assert np.array_equal(gpu[2], _oracle_table(lengths, max_pages, num_pages, free))
    s_short = int(np.argmin(lengths))
    _check_write_unit(gpu, cfg, 0, s_short, 3, lengths[s_short], rot, gpu[2][s_short], lengths[s_short] - 320)
    seqs = list(range(B))
    q = synth.decode_queries(cfg, 0, B, hq, hkv)
    out = st.decode(seqs, parity.to_dev_bf16(q), SCALE).cpu().numpy()
    lens = np.array(lengths)
    n2s = lens - 320
    g = hq // hkv
    s_long = int(np.argmax(lengths))
    for s, kv in [(s_short, 0), (s_long, 7), (3, 4)]:
        iso = _iso_decode_unit(gpu, lens, n2s, rot, q, s, kv, g)
        err = parity.rel_l2(out[s, kv * g:(kv + 1) * g], iso)
        print(f"[parity] decode unit seq={s} (L={lengths[s]}) kv={kv} rel-l2 {err:.2e}", flush=True)
        assert err <= 1e-3
