"""CPU tests of the C-ABI library: exports, host calibration, allocator/bookkeeping (no GPU calls)."""
import ctypes
import os
import re

import numpy as np
import pytest

import decode_attention_write_amd as oscar
import synth
from oracle import calibration, store as ostore

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    src = open(os.path.join(ROOT, "include", "oscar.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(oscar_\w+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = oscar.load()
    names = _header_functions()
    assert len(names) >= 15
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(oscar.EXPORTS)


def test_calibrate_host_matches_oracle():
    for kv in range(2):
        qb = synth.calibration_queries(synth.CFG_QWEN3_4B, 0, kv)
        q = synth.bf16_bits_to_f32(qb)
        rot, eig = oscar.oscar_calibrate_host(q)
        r_ref, w_ref = calibration.key_rotation(q.astype(np.float64))
        assert np.abs(eig - w_ref).max() < 1e-12 * w_ref[0]
        # eigenvectors of close eigenvalues are determined to ~eps*|C|/gap; compare per column
        u = rot.astype(np.float64) @ calibration.bit_reversal_matrix(128).T @ calibration.sylvester_hadamard(128)
        u_ref = r_ref @ calibration.bit_reversal_matrix(128).T @ calibration.sylvester_hadamard(128)
        gaps = np.minimum(np.abs(np.diff(w_ref, prepend=np.inf)), np.abs(np.diff(w_ref, append=-np.inf)))
        col_err = np.abs(u - u_ref).max(axis=0)
        assert np.all(col_err <= 2e-7 + 1e-14 * w_ref[0] / gaps * 100), col_err.max()
        assert np.abs(rot - r_ref.astype(np.float32)).max() < 1e-5
        r64 = rot.astype(np.float64)
        assert np.abs(r64.T @ r64 - np.eye(128)).max() < 2e-6


def test_calibrate_host_errors():
    q = np.ones((4, 128), np.float32)
    q[1, 3] = np.nan
    with pytest.raises(oscar.OscarError) as e:
        oscar.oscar_calibrate_host(q)
    assert e.value.status == oscar.E_NUMERIC
    with pytest.raises(oscar.OscarError) as e:
        oscar.oscar_calibrate_host(np.ones((4, 64), np.float32))
    assert e.value.status == oscar.E_ARG


def _plan_store(hkv=2, hq=8, max_seqs=4, max_pages=8, num_pages=12, free=None):
    s = oscar.KVStore(hq, hkv, max_seqs, max_pages, num_pages, free_pages=free, plan_only=True)
    s.set_rotation(np.stack([np.eye(128, dtype=np.float32)] * hkv))
    return s


def _oracle_store(hkv=2, max_seqs=4, max_pages=8, num_pages=12, free=None):
    free = list(range(num_pages)) if free is None else list(free)
    return ostore.OracleStore(hkv, max_seqs, max_pages, num_pages, free,
                              np.stack([np.eye(128, dtype=np.float32)] * hkv))


def test_plan_only_allocator_matches_oracle():
    free = np.random.default_rng(0).permutation(12).astype(np.int32)
    lib_s = _plan_store(free=free)
    ora = _oracle_store(free=free)
    zeros = lambda n_seqs, n: np.zeros((n_seqs, n, 2, 128), np.uint16)  # noqa: E731
    ops = [("w", [2, 0], 320 + 70), ("e", [0, 2], 58), ("e", [2], 1), ("w", [1], 200),
           ("w", [0, 2], 1), ("e", [0], 64), ("w", [3], 500)]
    for op, ids, n in ops:
        if op == "w":
            lib_s.write(ids, None, None, n_new=n)
            ora.write(ids, zeros(len(ids), n), zeros(len(ids), n))
        else:
            lib_s.evict(ids, n)
            ora.evict(ids, n)
        assert np.array_equal(lib_s.page_table(), ora.page_table), (op, ids, n)
        assert list(lib_s.free_pages()) == list(ora.free)
        for s in range(4):
            assert lib_s.seq_info(s) == (ora.length[s], ora.n_int2[s])
    lib_s.reset_seq(2)
    ora.reset_seq(2)
    assert np.array_equal(lib_s.page_table(), ora.page_table)
    assert list(lib_s.free_pages()) == list(ora.free)


def test_errors_leave_state_unchanged():
    s = _plan_store(num_pages=6, max_pages=4)
    s.write([0], None, None, n_new=320 + 128)      # 2 pages
    snap = (s.page_table().copy(), list(s.free_pages()), s.seq_info(0))

    def unchanged():
        assert np.array_equal(s.page_table(), snap[0]) and list(s.free_pages()) == snap[1]
        assert s.seq_info(0) == snap[2]

    cases = [
        (lambda: s.write([0], None, None, n_new=1), oscar.E_WINDOW_FULL),
        (lambda: s.evict([0], 257), oscar.E_WINDOW_SHORT),
        (lambda: s.evict([1], 1), oscar.E_WINDOW_SHORT),
        (lambda: s.write([1, 2], None, None, n_new=320 + 64 * 3), oscar.E_NOPAGE),
        (lambda: s.write([1], None, None, n_new=320 + 64 * 5), oscar.E_NOPAGE),   # > max_pages_per_seq
        (lambda: s.write([0, 0], None, None, n_new=1), oscar.E_ARG),
        (lambda: s.write([9], None, None, n_new=1), oscar.E_ARG),
        (lambda: s.evict([0], 0), oscar.E_ARG),
    ]
    for fn, status in cases:
        with pytest.raises(oscar.OscarError) as e:
            fn()
        assert e.value.status == status
        unchanged()
    with pytest.raises(oscar.OscarError) as e:
        oscar.oscar_decode_attn(s, [1], None, 0.1, None, None)
    assert e.value.status == oscar.E_STATE


def test_evicting_write_plan_matches_oracle():
    """With evicting writes on, overflowing writes into non-empty sequences take pages exactly as the
    oracle's token-by-token eviction does (FIFO order across the call's sequences, ascending within
    a sequence); with them off the same call is refused; a short FIFO refuses it unchanged."""
    free = list(np.random.default_rng(7).permutation(48))
    s = _plan_store(max_seqs=3, max_pages=32, num_pages=48, free=free)
    o = _oracle_store(max_seqs=3, max_pages=32, num_pages=48, free=free)
    zeros = lambda n, k=1: np.zeros((k, n, 2, 128), dtype=np.uint16)  # noqa: E731
    for ids, n in (([0], 100), ([1], 400), ([0], 200)):
        s.write(ids, None, None, n_new=n)
        o.write(ids, zeros(n, len(ids)), zeros(n, len(ids)))
    with pytest.raises(oscar.OscarError) as e:
        s.write([0, 1], None, None, n_new=300)
    assert e.value.status == oscar.E_WINDOW_FULL
    s.set_write_evicts(True)
    o.write_evicts = True
    for ids, n in (([0, 1], 300), ([1], 1000), ([0], 1), ([2], 5), ([2, 0], 640)):
        s.write(ids, None, None, n_new=n)
        o.write(ids, zeros(n, len(ids)), zeros(n, len(ids)))
        assert np.array_equal(s.page_table(), o.page_table), (ids, n)
        assert list(s.free_pages()) == list(o.free)
        for q in range(3):
            assert s.seq_info(q) == (int(o.length[q]), int(o.n_int2[q]))
            L, n2 = s.seq_info(q)
            # store invariants: the window never holds more than 256 tokens; one page per 64 INT2
            assert 0 <= L - min(L, 64) - n2 <= 256
            assert (s.page_table()[q] >= 0).sum() == -(-n2 // 64)
    snap = (s.page_table().copy(), list(s.free_pages()), [s.seq_info(q) for q in range(3)])
    with pytest.raises(oscar.OscarError) as e:
        s.write([1], None, None, n_new=64 * 30)      # more pages than the FIFO holds
    assert e.value.status in (oscar.E_NOPAGE,)
    assert np.array_equal(s.page_table(), snap[0]) and list(s.free_pages()) == snap[1]
    assert [s.seq_info(q) for q in range(3)] == snap[2]


def test_switch_setters_reject_bad_values():
    s = _plan_store()
    for fn in ("oscar_kv_set_output_bf16", "oscar_kv_set_write_evicts"):
        for bad in (-1, 2):
            with pytest.raises(oscar.OscarError) as e:
                oscar._check(getattr(oscar.load(), fn)(s.handle, bad))
            assert e.value.status == oscar.E_ARG
        with pytest.raises(oscar.OscarError) as e:
            oscar._check(getattr(oscar.load(), fn)(None, 1))
        assert e.value.status == oscar.E_ARG
    s.set_output_bf16(True)
    s.set_output_bf16(False)


def test_decode_step_plan_and_errors():
    """The one-call decode step advances the host state exactly as the decode-step write, sizes its
    workspace for the state after that write, and changes nothing when it fails."""
    a, b = _plan_store(max_pages=8, num_pages=12), _plan_store(max_pages=8, num_pages=12)
    for s in (a, b):
        s.write([0], None, None, n_new=320 + 64 * 2)   # window full, INT2 index 128: next evict takes a page
        s.write([1], None, None, n_new=100)
    ids = [0, 1]
    # the step's workspace is the attention's workspace after the write
    need = a.step_workspace_bytes(ids)
    b.decode_write(ids, None, None)
    assert need == b.workspace_bytes(ids)
    state = (a.seq_info(0), a.seq_info(1), a.page_table().copy(), a.free_pages().copy())
    # plan-only stores pass no workspace: the size check fails first and nothing moves
    with pytest.raises(oscar.OscarError) as e:
        oscar.oscar_decode_step(a, ids, None, None, None, 0.1, None, None)
    assert e.value.status == oscar.E_WORKSPACE
    assert (a.seq_info(0), a.seq_info(1)) == state[:2]
    assert np.array_equal(a.page_table(), state[2]) and np.array_equal(a.free_pages(), state[3])
    # an empty sequence, a bad id and a non-finite scale are refused before anything changes
    for bad_ids, scale, status in (([0, 2], 0.1, oscar.E_STATE), ([0, 9], 0.1, oscar.E_ARG),
                                   (ids, float("nan"), oscar.E_ARG)):
        with pytest.raises(oscar.OscarError) as e:
            oscar.oscar_decode_step(a, bad_ids, None, None, None, scale, None, None)
        assert e.value.status == status
        assert (a.seq_info(0), a.seq_info(1)) == state[:2]
        assert np.array_equal(a.free_pages(), state[3])


def test_workspace_bytes_and_split_choice():
    s = _plan_store(max_pages=64, num_pages=64)
    s.write([0], None, None, n_new=320 + 64 * 20)
    s.write([1], None, None, n_new=100)
    qprep = 2 * 2 * 8448          # prepared-query area: 2 seqs x 2 KV heads

    def expect(records):
        # partials (2 seqs x 8 q heads x records x 130 floats), prepared queries, and one int32
        # page counter per split of each (seq, KV head)
        return 2 * 8 * records * 130 * 4 + qprep + 2 * 2 * records * 4

    nb = s.workspace_bytes([0, 1])
    assert nb > qprep and (nb - qprep) % (130 * 4 * 8 * 2 + 2 * 2 * 4) == 0
    s.set_decode_split(4)
    nb4 = s.workspace_bytes([0, 1])
    # sequence 0: 20 pages / 4 per split = 5 INT2 records; its 320 BF16 tokens weigh 32 pages,
    # cut into min(5, ceil(32 / 4)) = 5 chunk ranges -> 10 records.  Sequence 1 (100 tokens, no
    # INT2): weight 10 -> ceil(10 / 4) = 3 records.
    assert nb4 == expect(10)
    s.set_decode_split(40)
    # 1 INT2 record + 1 BF16 record (weight 32 <= 40 pages per split)
    assert s.workspace_bytes([0, 1]) == expect(2)
    s.set_decode_kernel(1)
    s.set_decode_split(4)
    # the reference kernel keeps one BF16 record per unit: 5 + 1
    assert s.workspace_bytes([0, 1]) == expect(6)
    s.set_decode_deterministic(True)   # with an explicit split size the mode does not change the plan
    assert s.workspace_bytes([0, 1]) == expect(6)
    for bad in (-1, 2):
        with pytest.raises(oscar.OscarError) as e:
            oscar._check(oscar.load().oscar_kv_set_decode_deterministic(s.handle, bad))
        assert e.value.status == oscar.E_ARG


def test_timing_errors():
    s = _plan_store()
    with pytest.raises(oscar.OscarError) as e:
        s.set_timing(True)
    assert e.value.status == oscar.E_STATE
    for kernel in (oscar.TIMED_DECODE, oscar.TIMED_WRITE):
        with pytest.raises(oscar.OscarError) as e:
            s.read_timing(kernel)
        assert e.value.status == oscar.E_STATE
    with pytest.raises(oscar.OscarError) as e:
        s.read_timing(2)
    assert e.value.status == oscar.E_ARG


def test_calibrate_value_host_matches_oracle():
    rng = np.random.default_rng(21)
    q = rng.standard_normal((512, 128))           # more queries than channels: full-rank C_S
    k = rng.standard_normal((400, 128))
    s = np.exp((q @ k.T) / np.sqrt(128) * 4)
    s /= s.sum(axis=1, keepdims=True)
    v = rng.standard_normal((400, 128)) * (1 + np.arange(128) / 16) + rng.standard_normal(128)
    s32, v32 = s.astype(np.float32), v.astype(np.float32)
    rot, eig = oscar.oscar_calibrate_value_host(s32, v32)
    r_ref, w_ref = calibration.value_rotation(s32.astype(np.float64), v32.astype(np.float64))
    assert np.abs(eig - w_ref).max() < 1e-12 * w_ref[0]
    # eigenvectors of close eigenvalues are determined to ~eps*|C|/gap; compare per column
    hp = calibration.bit_reversal_matrix(128).T @ calibration.sylvester_hadamard(128)
    u, u_ref = rot.astype(np.float64) @ hp, r_ref @ hp
    gaps = np.minimum(np.abs(np.diff(w_ref, prepend=np.inf)), np.abs(np.diff(w_ref, append=-np.inf)))
    col_err = np.abs(u - u_ref).max(axis=0)
    assert np.all(col_err <= 2e-7 + 1e-14 * w_ref[0] / gaps * 100), col_err.max()
    r64 = rot.astype(np.float64)
    assert np.abs(r64.T @ r64 - np.eye(128)).max() < 2e-6


def test_fold_value_rotation_matches_oracle():
    rng = np.random.default_rng(22)
    hq, hkv, d_model = 8, 2, 64
    r_v = np.stack([np.linalg.qr(rng.standard_normal((128, 128)))[0] for _ in range(hkv)]).astype(np.float32)
    w_v = rng.standard_normal((d_model, hkv * 128)).astype(np.float32)
    w_o = rng.standard_normal((hq * 128, d_model)).astype(np.float32)
    wv2, wo2 = oscar.oscar_fold_value_rotation(w_v, w_o, r_v, hq, hkv)
    wv_ref, wo_ref = calibration.fold_value_rotation(w_v, w_o, r_v, hq, hkv)
    assert np.abs(wv2 - wv_ref).max() < 1e-5 * np.abs(wv_ref).max()
    assert np.abs(wo2 - wo_ref).max() < 1e-5 * np.abs(wo_ref).max()


def test_value_calibration_errors():
    with pytest.raises(oscar.OscarError) as e:
        oscar.oscar_calibrate_value_host(np.full((2, 3), np.nan, np.float32), np.ones((3, 128), np.float32))
    assert e.value.status == oscar.E_NUMERIC
    with pytest.raises(oscar.OscarError) as e:
        oscar.oscar_calibrate_value_host(np.ones((2, 3), np.float32), np.ones((3, 64), np.float32))
    assert e.value.status == oscar.E_ARG
    bad = np.full((1, 128, 128), np.inf, np.float32)
    with pytest.raises(oscar.OscarError) as e:
        oscar.oscar_fold_value_rotation(np.ones((4, 128), np.float32), np.ones((128, 4), np.float32), bad, 1, 1)
    assert e.value.status == oscar.E_NUMERIC


def test_binding_constants_match_header():
    src = open(os.path.join(ROOT, "include", "oscar.h")).read()
    consts = dict(re.findall(r"#define\s+(OSCAR_\w+)\s+(-?\d+)", src))
    assert int(consts["OSCAR_TIMING_PAIRS"]) == oscar.TIMING_PAIRS
    assert int(consts["OSCAR_TIMED_DECODE"]) == oscar.TIMED_DECODE
    assert int(consts["OSCAR_TIMED_WRITE"]) == oscar.TIMED_WRITE


def test_plan_only_decode_write_matches_evict_then_write():
    """The fused decode-step write keeps the same books as evict-when-full followed by a one-token
    write: page tables, free list and lengths agree step by step, across page boundaries."""
    free = np.random.default_rng(3).permutation(12).astype(np.int32)
    fused, split = _plan_store(free=free), _plan_store(free=free)
    starts = {0: 10, 1: 300, 2: 320 + 63, 3: 320 + 127}
    for s, n in starts.items():
        fused.write([s], None, None, n_new=n)
        split.write([s], None, None, n_new=n)
    ids = [3, 1, 0, 2]
    for step in range(80):
        fused.decode_write(ids, None, None)
        full = [s for s in ids if split.seq_info(s)[0] - 64 - split.seq_info(s)[1] == 256]
        if full:
            split.evict(full, 1)
        split.write(ids, None, None, n_new=1)
        assert np.array_equal(fused.page_table(), split.page_table()), step
        assert list(fused.free_pages()) == list(split.free_pages()), step
        for s in ids:
            assert fused.seq_info(s) == split.seq_info(s), (step, s)
    assert fused.seq_info(3) == (320 + 127 + 80, 127 + 80)
    assert fused.seq_info(1) == (380, 60)


def test_decode_write_errors_leave_state_unchanged():
    s = _plan_store(num_pages=4, max_pages=2)
    s.write([0], None, None, n_new=320 + 128)      # 2 pages = max_pages_per_seq, INT2 full
    s.write([1], None, None, n_new=320 + 64)       # 1 page
    snap = (s.page_table().copy(), list(s.free_pages()), s.seq_info(0), s.seq_info(1))

    def unchanged():
        assert np.array_equal(s.page_table(), snap[0]) and list(s.free_pages()) == snap[1]
        assert (s.seq_info(0), s.seq_info(1)) == snap[2:]

    cases = [
        (lambda: s.decode_write([2], None, None), oscar.E_STATE),        # empty sequence
        (lambda: s.decode_write([1, 2], None, None), oscar.E_STATE),
        (lambda: s.decode_write([0], None, None), oscar.E_NOPAGE),       # > max_pages_per_seq
        (lambda: s.decode_write([1, 1], None, None), oscar.E_ARG),
        (lambda: s.decode_write([7], None, None), oscar.E_ARG),
    ]
    for fn, status in cases:
        with pytest.raises(oscar.OscarError) as e:
            fn()
        assert e.value.status == status
        unchanged()
    s.decode_write([1], None, None)                # takes the last free page
    assert s.seq_info(1) == (320 + 65, 65) and list(s.free_pages()) == []
    for _ in range(63):
        s.decode_write([1], None, None)            # fills that page
    with pytest.raises(oscar.OscarError) as e:
        s.decode_write([1], None, None)            # needs a page, none free
    assert e.value.status == oscar.E_NOPAGE


def test_binding_rejects_mismatched_tensors():
    """The binding checks every device tensor it hands to the library (shape, dtype, contiguity,
    device) before the call, so a wrong one raises instead of reading or writing out of bounds."""
    import torch
    import decode_attention_write_amd as oscar
    ok = torch.zeros((2, 3, 4, 128), dtype=torch.int16)
    oscar.check_tensor(ok, "k", (2, 3, 4, 128), (torch.int16, torch.bfloat16))
    bad = [
        (torch.zeros((2, 3, 5, 128), dtype=torch.int16), "shape"),              # wrong Hkv
        (torch.zeros((2, 3, 4, 128), dtype=torch.float32), "dtype"),            # fp32 where bf16
        (torch.zeros((2, 3, 4, 256), dtype=torch.int16)[..., ::2], "contiguous"),
        (torch.zeros((2, 4, 4, 128), dtype=torch.int16)[:, 1:], "contiguous"),  # a slice of a longer buffer
    ]
    for t, what in bad:
        with pytest.raises(ValueError, match=what):
            oscar.check_tensor(t, "k", (2, 3, 4, 128), (torch.int16, torch.bfloat16))
    with pytest.raises(ValueError, match="on cpu"):
        oscar.check_tensor(ok, "k", (2, 3, 4, 128), (torch.int16,), torch.device("meta"))


def test_noalloc_step_host_limits():
    """The allocation-free decode step plans like the workspace form and refuses a step whose
    workspace would exceed the library's scratch array (plan-only store, host logic)."""
    hkv, hq, B, L = 8, 64, 64, 320 + 64 * 11
    st = oscar.KVStore(hq, hkv, B, 12, B * 12, plan_only=True)
    st.set_rotation(np.stack([np.eye(128, dtype=np.float32)] * hkv))
    ids = list(range(B))
    st.write(ids, None, None, n_new=L)
    st.set_decode_split(1)
    assert st.step_workspace_bytes(ids) > oscar.NOALLOC_SCRATCH_BYTES
    with pytest.raises(oscar.OscarError, match="E_WORKSPACE"):
        oscar.oscar_decode_step_noalloc(st, ids, None, None, None, 0.1, None)
    assert st.seq_info(0) == (L, L - 320)                      # nothing changed
    st.set_decode_split(0)
    assert st.step_workspace_bytes(ids[:4]) <= oscar.NOALLOC_SCRATCH_BYTES
    oscar.oscar_decode_step_noalloc(st, ids[:4], None, None, None, 0.1, None)
    assert st.seq_info(0) == (L + 1, L - 320 + 1)              # the step's write was planned


def test_key_mean_host_checks():
    """oscar_kv_set_key_mean: a null handle and a non-finite entry are refused (E_ARG, nothing
    changes); a finite mean, clearing it (NULL) and setting it before or after the rotation are
    accepted on a plan-only store."""
    lib = oscar.load()
    assert lib.oscar_kv_set_key_mean(None, None, None) == oscar.E_ARG
    s = _plan_store()
    mu = np.zeros((2, 128), np.float32)
    s.set_key_mean(mu)                       # before the rotation: kept for it
    s.set_rotation(np.stack([np.eye(128, dtype=np.float32)] * 2))
    bad = mu.copy()
    bad[1, 5] = np.nan
    with pytest.raises(oscar.OscarError) as e:
        s.set_key_mean(bad)
    assert e.value.status == oscar.E_ARG and "non-finite" in str(e.value)
    bad[1, 5] = np.inf
    with pytest.raises(oscar.OscarError):
        s.set_key_mean(bad)
    s.set_key_mean(mu + 1.5)
    s.set_key_mean(None)
    s.write([0], None, None, n_new=400)      # the store still works
    assert s.seq_info(0) == (400, 80)
