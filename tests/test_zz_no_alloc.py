"""The allocation-free decode step (oscar_decode_step_noalloc, scratch in the library's static
device array) against the workspace form (oscar_decode_step) on identical stores: two calls in a
row, the second over fewer sequences, each compared bit for bit (deterministic mode) in output,
pool, ring and page table, and against the oracle on the GPU's state."""
import math

import numpy as np
import pytest

import parity
import synth
from oracle import attention, store as ostore
from test_gpu_parity import _kv_batch, _store

pytestmark = pytest.mark.gpu
D = 128
SCALE = 1.0 / math.sqrt(D)


@pytest.mark.parametrize("deterministic", [True, False])
def test_noalloc_step_matches_workspace_step(gpu_lib, deterministic):
    import torch
    hkv, hq = 2, 8
    print(f"[case] no-alloc decode step vs workspace decode step, deterministic={deterministic}", flush=True)
    rot = parity.calibrate(synth.CFG_QWEN3_4B, 9, hkv)
    lengths = {0: 320 + 64 * 6 + 3, 1: 100, 2: 320 + 64 * 11, 3: 576}
    free = synth.page_permutation(synth.CFG_QWEN3_4B, 9, 64)
    a = _store(gpu_lib, hq, hkv, 4, 16, 64, free, rot)     # workspace form
    b = _store(gpu_lib, hq, hkv, 4, 16, 64, free, rot)     # allocation-free form
    for st in (a, b):
        st.set_decode_deterministic(deterministic)
    ks, vs = _kv_batch(synth.CFG_QWEN3_4B, [0, 1, 2, 3], hkv, max(lengths.values()) + 2)
    for s, L in lengths.items():
        for st in (a, b):
            st.write([s], parity.to_dev_bf16(ks[s:s + 1, :L]), parity.to_dev_bf16(vs[s:s + 1, :L]))
    pos = dict(lengths)
    # two calls in a row on one device: all four sequences, then a smaller call of two
    for step, ids in enumerate(([2, 0, 3, 1], [1, 2])):
        kt = parity.to_dev_bf16(np.stack([ks[s, pos[s]] for s in ids]))
        vt = parity.to_dev_bf16(np.stack([vs[s, pos[s]] for s in ids]))
        qb = synth.decode_queries(synth.CFG_QWEN3_4B, 9, len(ids), hq, hkv, step=step)
        q = parity.to_dev_bf16(qb)
        assert b.step_workspace_bytes(ids) <= gpu_lib.NOALLOC_SCRATCH_BYTES
        out_a = a.decode_step(ids, kt, vt, q, SCALE).cpu().numpy()
        out_b = torch.empty((len(ids), hq, D), dtype=torch.float32, device="cuda")
        b.decode_step_noalloc(ids, kt, vt, q, SCALE, out_b)
        out_b = out_b.cpu().numpy()
        for s in ids:
            pos[s] += 1
        ea, eb = parity.export(a), parity.export(b)
        for x, y, name in zip(ea, eb, ("pool", "ring", "table")):
            assert np.array_equal(x, y), (step, name)
        if deterministic:
            assert np.array_equal(out_a, out_b), step
        else:
            assert parity.rel_l2(out_b, out_a) <= 1e-4, step
        lens = np.array([b.seq_info(s)[0] for s in range(4)])
        n2s = np.array([b.seq_info(s)[1] for s in range(4)])
        iso = attention.decode(eb[0], eb[1], eb[2], lens, n2s, rot, qb, ids, SCALE, hq)
        err = parity.rel_l2(out_b, iso)
        print(f"[parity] step {step} ({len(ids)} sequences): no-alloc vs oracle rel-l2 {err:.2e}", flush=True)
        assert err <= 1e-3, (step, err)


def test_noalloc_step_rejects_oversized_calls(gpu_lib):
    """A step whose workspace exceeds the scratch array is refused with OSCAR_E_WORKSPACE and
    changes nothing."""
    import torch
    hkv, hq, B = 8, 64, 64
    print("[case] no-alloc decode step: oversized call refused", flush=True)
    L = 320 + 64 * 11                      # 11 INT2 pages: 16 partial records per unit at 1 page a split
    st = gpu_lib.KVStore(hq, hkv, B, 12, B * 12)
    st.set_rotation(np.stack([np.eye(D, dtype=np.float32)] * hkv))
    st.set_decode_split(1)
    kb = torch.zeros((B, L, hkv, D), dtype=torch.int16, device="cuda")
    st.write(list(range(B)), kb, kb)
    ids = list(range(B))
    need = st.step_workspace_bytes(ids)
    if need <= gpu_lib.NOALLOC_SCRATCH_BYTES:
        pytest.skip(f"this shape needs only {need} bytes")
    k1 = torch.zeros((B, hkv, D), dtype=torch.int16, device="cuda")
    q = torch.zeros((B, hq, D), dtype=torch.int16, device="cuda")
    out = torch.empty((B, hq, D), dtype=torch.float32, device="cuda")
    with pytest.raises(gpu_lib.OscarError, match="E_WORKSPACE"):
        st.decode_step_noalloc(ids, k1, k1, q, SCALE, out)
    assert st.seq_info(0) == (L, L - 320)
