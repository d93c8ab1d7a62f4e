"""Helpers for GPU-vs-oracle parity: store export, tolerance rules, workload set-up."""
from __future__ import annotations

import numpy as np

import synth
from oracle import attention, layout, quantizer, store as ostore

D = 128


# ----------------------------------------------------------------------------- GPU side helpers

def to_dev_bf16(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()


def export(st):
    """Copy a KVStore's device buffers to host numpy (pool uint8, ring uint16 bits, table int32)."""
    import torch
    torch.cuda.synchronize()
    pool = st.pool_view().cpu().numpy()
    ring = st.ring_view().cpu().numpy().view(np.uint16)
    table = st.table_view().cpu().numpy()
    return pool, ring, table


def calibrate(cfg, layer, hkv):
    import decode_attention_write_amd as oscar
    rots = []
    for kv in range(hkv):
        q = synth.bf16_bits_to_f32(synth.calibration_queries(cfg, layer, kv))
        rots.append(oscar.oscar_calibrate_host(q)[0])
    return np.stack(rots)


# ----------------------------------------------------------------------------- tolerance rules

class Report(dict):
    pass


def bf16_ulp_diff(a_bits, b_bits):
    """|a - b| in units of bf16 ulps (same-sign finite values; order-preserving integer map)."""
    def key(b):
        b = b.astype(np.int32)
        return np.where(b & 0x8000, 0x8000 - (b & 0x7FFF), 0x8000 + (b & 0x7FFF))
    return np.abs(key(a_bits) - key(b_bits))


def fp16_ulp_diff(a, b):
    def key(x):
        b = np.asarray(x, dtype=np.float16).view(np.uint16).astype(np.int32)
        return np.where(b & 0x8000, 0x8000 - (b & 0x7FFF), 0x8000 + (b & 0x7FFF))
    return np.abs(key(a) - key(b))


def rotation_error_bound(k_bits, rot_h, mean=None):
    """Per-element bound on |x_gpu - (k - mu).R| for keys rotated on the matrix cores (bf16 [n, 128]
    keys, one head's fp32 R, optional key mean mu).  The write kernel carries R^T as three bf16
    terms r0 = bf16(R^T), r1 = bf16(R^T - r0), r2 = bf16(R^T - r0 - r1), so |R - r0 - r1 - r2| <=
    2^-24 |R| (bf16 unit roundoff 2^-8, three times); the bf16 keys enter as they are; the
    accumulator starts from fp32(-(mu . R)) (within 2^-24 |mu . R|; zero without a mean); the
    products are exact in fp32 and the 384 of them go through 12 matrix instructions of 32 into
    the fp32 accumulator: up to 48 roundings of at most (1 + 2^-7) sum_i |k_i R_ij| + |mu . R|_j
    each are allowed.  Products or inputs below the fp32 normal range may be flushed: 2^-116
    absolute covers 384 of them.  Returns [n, 128]."""
    k = synth.bf16_bits_to_f32(k_bits).astype(np.float64)
    r = np.asarray(rot_h, np.float32).astype(np.float64)
    kr = np.abs(k) @ np.abs(r)
    m = _shift_abs(rot_h, mean)[None]
    return kr * 2.0 ** -24 + 48 * 2.0 ** -24 * ((1 + 2.0 ** -7) * kr + m) + 2.0 ** -24 * m + 2.0 ** -116


def _ulp32(x):
    _, e = np.frexp(np.abs(np.asarray(x, dtype=np.float64)))
    return np.ldexp(1.0, e - 24)


def meta_flip_explained(x_ref, c, s16_gpu, lo16_gpu, elem_bound):
    """Which fp16 scale / minimum flips of rotated-key groups are explained by the rotation error.

    x_ref: fp64 [n, 128] the oracle's quantizer input; elem_bound: [n, 128] bound on the GPU's
    input error (rotation_error_bound plus the oracle's own fp32 rounding).  With delta = the
    group's largest element bound, the group minimum and maximum move by at most delta, so the
    fp32 scale c (mx - mn) / 3 moves by at most (2c/3) delta and the fp32 minimum
    mn + (1 - c)(mx - mn)/2 by at most (2 - c) delta, each plus the fp32 roundings of the
    parameter sequence (a few ulps).  A flip is explained when the oracle's fp32 parameter lies
    within that distance of the rounding midpoint between the two fp16 values.  Returns boolean
    arrays (s_ok, lo_ok) [n, 2] (True also where nothing flipped)."""
    s32, lo32, s16o, lo16o = quantizer.params(np.asarray(x_ref, np.float32), c)
    delta = np.asarray(elem_bound, np.float64).reshape(len(x_ref), 2, 64).max(axis=-1)
    xg = np.asarray(x_ref, np.float64).reshape(len(x_ref), 2, 64)
    span = np.abs(xg).max(axis=-1) + (xg.max(axis=-1) - xg.min(axis=-1))
    cf = float(c)
    tol_s = (2 * cf / 3) * delta + 4 * _ulp32(s32)
    tol_lo = (2 - cf) * delta + 4 * _ulp32(span)
    mid_s = 0.5 * (s16o.astype(np.float64) + np.asarray(s16_gpu, np.float16).astype(np.float64))
    mid_lo = 0.5 * (lo16o.astype(np.float64) + np.asarray(lo16_gpu, np.float16).astype(np.float64))
    s_flip = s16o.view(np.uint16) != np.asarray(s16_gpu, np.float16).view(np.uint16)
    lo_flip = lo16o.view(np.uint16) != np.asarray(lo16_gpu, np.float16).view(np.uint16)
    s_ok = ~s_flip | (np.abs(s32.astype(np.float64) - mid_s) <= tol_s)
    lo_ok = ~lo_flip | (np.abs(lo32.astype(np.float64) - mid_lo) <= tol_lo)
    return s_ok, lo_ok


def exact_codes(x, s16, lo16):
    """Codes of fp64 values x [n, 128] under given fp16 metadata [n, 2]: the exact decision
    clamp(round_half_even((x - lo16) / s16), 0, 3), 0 where s16 == 0."""
    xg = np.asarray(x, np.float64).reshape(len(x), 2, 64)
    s = np.asarray(s16, np.float16).astype(np.float64)[..., None]
    lo = np.asarray(lo16, np.float16).astype(np.float64)[..., None]
    t = (xg - lo) / np.where(s != 0, s, 1.0)
    return np.where(s != 0, np.clip(np.rint(t), 0, 3), 0).astype(np.uint8).reshape(len(x), 128)


def compare_int2_unit(gpu_pool, gpu_table, ora_pool, ora_table, seq, gkv, okv, n_int2, x_ref_k, x_ref_v,
                      check_tail=True, k_bound=None):
    """Compare the INT2 tokens of one (seq, kv head) under the parity rules.

    x_ref_k / x_ref_v: fp64 [n_int2, 128] values the oracle quantized (rotated keys, values).
    k_bound: [n_int2, 128] bound on the GPU's key-input error (see rotation_error_bound); when
    given, every key-metadata flip must be explained by it (``k_meta_unexplained``).
    A code mismatch is explained when the value lies within 1e-3 * s16 of a rounding boundary
    under either side's metadata, or, in a group whose metadata flipped, when the GPU's code is
    the exact decision under the GPU's metadata (``explained_by_meta``).
    Returns a dict of counts; asserts nothing (callers assert).
    """
    rep = dict(elements=0, code_mismatch=0, unexplained=0, k_meta_flips=0, v_meta_flips=0,
               meta_far=0, groups=0, tail_nonzero=0, k_meta_unexplained=0, explained_by_meta=0)
    n_pages = -(-n_int2 // 64)
    if n_pages == 0:
        return rep
    n_last = n_int2 - 64 * (n_pages - 1)
    g = layout.unpack_pages(gpu_pool[gpu_table[seq, :n_pages], gkv])
    o = layout.unpack_pages(ora_pool[ora_table[seq, :n_pages], okv])
    # unused slots of the last page are zero
    if check_tail and n_last < 64:
        rep["tail_nonzero"] += int(sum(np.count_nonzero(np.ascontiguousarray(a[-1, n_last:]).view(np.uint8)) for a in g))
    # flatten pages to token rows, keeping the first n_int2
    g = [a.reshape((-1,) + a.shape[2:])[:n_int2] for a in g]
    o = [a.reshape((-1,) + a.shape[2:])[:n_int2] for a in o]
    for which, (gc, gs, gl), (oc, os_, ol), xr in (
            ("k", (g[0], g[2], g[3]), (o[0], o[2], o[3]), x_ref_k[:n_int2]),
            ("v", (g[1], g[4], g[5]), (o[1], o[4], o[5]), x_ref_v[:n_int2])):
        flips = (fp16_ulp_diff(gs, os_) > 0) | (fp16_ulp_diff(gl, ol) > 0)
        far = (fp16_ulp_diff(gs, os_) > 1) | (fp16_ulp_diff(gl, ol) > 1)
        rep[which + "_meta_flips"] += int(flips.sum())
        if which == "k" and k_bound is not None and flips.any():
            rows = np.nonzero(flips.any(axis=1))[0]
            eb = k_bound[rows] + 2.0 ** -24 * np.abs(xr[rows])
            s_ok, lo_ok = meta_flip_explained(xr[rows], quantizer.C_K, gs[rows], gl[rows], eb)
            rep["k_meta_unexplained"] += int((~(s_ok & lo_ok)).sum())
        rep["meta_far"] += int(far.sum())
        rep["groups"] += flips.size
        mism = gc != oc
        rep["elements"] += gc.size
        rep["code_mismatch"] += int(mism.sum())
        if mism.any():
            rows = np.nonzero(mism.any(axis=1))[0]
            d_o = quantizer.boundary_distance(xr[rows], os_[rows], ol[rows])
            d_g = quantizer.boundary_distance(xr[rows], gs[rows], gl[rows])
            explained = (d_o < 1e-3) | (d_g < 1e-3)
            # In a group whose scale or minimum flipped by one fp16 ulp (allowed above), every
            # element near a boundary moves by that ulp / s16, which can exceed the band: there the
            # GPU's code must be the exact decision under the GPU's own metadata.
            own = exact_codes(xr[rows], gs[rows], gl[rows])
            grp_flip = np.repeat(flips[rows], 64, axis=-1)
            by_meta = grp_flip & (gc[rows] == own) & ~explained
            rep["explained_by_meta"] += int((mism[rows] & by_meta).sum())
            rep["unexplained"] += int((mism[rows] & ~explained & ~by_meta).sum())
    return rep


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def oracle_decode_on(pool, ring, table, length, n_int2, rot, q_bits, seq_ids, sm_scale, hq):
    return attention.decode(pool, ring, table, length, n_int2, rot, q_bits, seq_ids, sm_scale, hq)


def rotated_keys_f64(k_bits, rot, mean=None):
    """(k - mu) . R_K in fp64 for bf16 keys [n, 128], one head's fp32 rotation and optional fp32
    key mean [128] (the oracle's rotate_keys for one head)."""
    k = synth.bf16_bits_to_f32(k_bits).astype(np.float64)
    return ostore.rotate_keys(k[:, None, :], np.asarray(rot, np.float32)[None],
                              None if mean is None else np.asarray(mean, np.float32)[None])[:, 0, :]


def quant_input_k(k_bits, rot, mean=None):
    """What the oracle quantizes for prefill INT2 keys: fp32((k - mu) . R_K)."""
    return rotated_keys_f64(k_bits, rot, mean).astype(np.float32).astype(np.float64)


def _shift_abs(rot_h, mean):
    """|mu . R| per output channel [128] (zeros without a mean)."""
    if mean is None:
        return np.zeros(128)
    return np.abs(np.asarray(mean, np.float32).astype(np.float64) @ np.asarray(rot_h, np.float32).astype(np.float64))


def oracle_store_for(hkv, max_seqs, max_pages, num_pages, free, rot):
    return ostore.OracleStore(hkv, max_seqs, max_pages, num_pages, free, rot)


def check_evicted(pool, table, ring_before, seq, n2, heads=None):
    """INT2 index n2 of one sequence against the oracle's quantization of the GPU's ring slot
    (identical inputs): page-table entry present, metadata bit-exact, codes equal except where
    the value lies within 1e-3 * s16 of a rounding boundary (the oracle decides in fp64, the
    kernel in fp32).  Returns the number of explained code mismatches; asserts the rest."""
    kc, ksc, klo, vc, vsc, vlo = ostore.evict_from_ring(ring_before, seq, n2)
    slot = ostore.OracleStore.ring_slot(64 + int(n2))
    page = int(table[seq, n2 // 64])
    assert page >= 0, (seq, n2)
    j = n2 % 64
    explained = 0
    heads = range(kc.shape[0]) if heads is None else heads
    for h in heads:
        g = layout.unpack_head_block(pool[page, h])
        for isv, (codes, s16, lo16, gc, gs, gl) in enumerate(((kc[h], ksc[h], klo[h], g[0][j], g[2][j], g[3][j]),
                                                              (vc[h], vsc[h], vlo[h], g[1][j], g[4][j], g[5][j]))):
            assert np.array_equal(gs.view(np.uint16), s16.view(np.uint16)), (seq, n2, h, isv)
            assert np.array_equal(gl.view(np.uint16), lo16.view(np.uint16)), (seq, n2, h, isv)
            mism = gc != codes
            if mism.any():
                x = ostore.bf16_to_f64(ring_before[seq, h, isv, slot])
                d = quantizer.boundary_distance(x[None], s16[None], lo16[None])[0]
                assert np.all(d[mism] < 1e-3), (seq, n2, h, isv)
                explained += int(mism.sum())
    return explained


def ring_key_bound(k_bits, rot_h, mean=None):
    """Allowed |stored bf16 key - exact (k - mu).R| per channel, besides half a bf16 ulp of the
    stored value.  Multi-token writes rotate on the matrix cores (rotation_error_bound: bf16 terms
    of R^T within 2^-24 of it, exact products, fp32 accumulation from fp32(-(mu . R)));
    single-token appends use a 128-term fp32 dot product from the same start.  Both stay within
    gamma_256 (1 + 2^-8) (sum_i |k_i R_ij| + |mu . R|_j) + 2^-24 (sum_i |k_i R_ij| + |mu . R|_j) +
    2^-116 (dot-product forward-error bound, Higham, Accuracy and Stability of Numerical
    Algorithms, section 3.1).  Returns (bound, exact (k - mu).R) [n, 128]."""
    k = synth.bf16_bits_to_f32(k_bits).astype(np.float64)
    r = np.asarray(rot_h, np.float32).astype(np.float64)
    u = 2.0 ** -24
    gamma = 256 * u / (1 - 256 * u)
    a = np.abs(k) @ np.abs(r) + _shift_abs(rot_h, mean)[None]
    return a * (gamma * (1 + 2.0 ** -8) + 2.0 ** -24) + 2.0 ** -116, rotated_keys_f64(k_bits, rot_h, mean)


def bf16_ulp(x):
    """Spacing of bf16 numbers at |x| (8 significant bits)."""
    _, e = np.frexp(np.abs(np.asarray(x, dtype=np.float64)))
    return np.ldexp(1.0, e - 8)


def check_ring_keys(got_bits, k_bits, rot_h, mean=None):
    """Stored bf16 ring keys [n, 128] of one head within half a bf16 ulp plus ring_key_bound of
    the exact (k - mu).R (asserts)."""
    bound, xk = ring_key_bound(k_bits, rot_h, mean)
    got = ostore.bf16_to_f64(got_bits)
    ulp = np.maximum(bf16_ulp(got), bf16_ulp(xk))
    assert np.all(np.abs(got - xk) <= 0.5 * ulp + bound)
