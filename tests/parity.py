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


def compare_int2_unit(gpu_pool, gpu_table, ora_pool, ora_table, seq, gkv, okv, n_int2, x_ref_k, x_ref_v,
                      check_tail=True):
    """Compare the INT2 tokens of one (seq, kv head) under the parity rules.

    x_ref_k / x_ref_v: fp64 [n_int2, 128] values the oracle quantized (rotated keys, values).
    Returns a dict of counts; asserts nothing (callers assert).
    """
    rep = dict(elements=0, code_mismatch=0, unexplained=0, k_meta_flips=0, v_meta_flips=0,
               meta_far=0, groups=0, tail_nonzero=0)
    n_pages = -(-n_int2 // 64)
    for pg in range(n_pages):
        n_tok = min(64, n_int2 - 64 * pg)
        gblk = gpu_pool[gpu_table[seq, pg], gkv]
        oblk = ora_pool[ora_table[seq, pg], okv]
        g = layout.unpack_head_block(gblk)
        o = layout.unpack_head_block(oblk)
        sl = slice(64 * pg, 64 * pg + n_tok)
        # unused slots of the last page are zero
        if check_tail:
            rep["tail_nonzero"] += int(sum(np.count_nonzero(a[n_tok:]) for a in g))
        for which, (gc, gs, gl), (oc, os_, ol), xr in (
                ("k", (g[0], g[2], g[3]), (o[0], o[2], o[3]), x_ref_k[sl]),
                ("v", (g[1], g[4], g[5]), (o[1], o[4], o[5]), x_ref_v[sl])):
            gc, oc = gc[:n_tok], oc[:n_tok]
            gs, gl, os_, ol = gs[:n_tok], gl[:n_tok], os_[:n_tok], ol[:n_tok]
            flips = (fp16_ulp_diff(gs, os_) > 0) | (fp16_ulp_diff(gl, ol) > 0)
            far = (fp16_ulp_diff(gs, os_) > 1) | (fp16_ulp_diff(gl, ol) > 1)
            rep[which + "_meta_flips"] += int(flips.sum())
            rep["meta_far"] += int(far.sum())
            rep["groups"] += flips.size
            mism = gc != oc
            rep["elements"] += gc.size
            rep["code_mismatch"] += int(mism.sum())
            if mism.any():
                d_o = quantizer.boundary_distance(xr, os_, ol)
                d_g = quantizer.boundary_distance(xr, gs, gl)
                explained = (d_o < 1e-3) | (d_g < 1e-3)
                rep["unexplained"] += int((mism & ~explained).sum())
    return rep


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def oracle_decode_on(pool, ring, table, length, n_int2, rot, q_bits, seq_ids, sm_scale, hq):
    return attention.decode(pool, ring, table, length, n_int2, rot, q_bits, seq_ids, sm_scale, hq)


def rotated_keys_f64(k_bits, rot):
    """k . R_K in fp64 for bf16 keys [n, 128] and one head's fp32 rotation."""
    return synth.bf16_bits_to_f32(k_bits).astype(np.float64) @ np.asarray(rot, np.float32).astype(np.float64)


def quant_input_k(k_bits, rot):
    """What the oracle quantizes for prefill INT2 keys: fp32(k . R_K)."""
    return rotated_keys_f64(k_bits, rot).astype(np.float32).astype(np.float64)


def oracle_store_for(hkv, max_seqs, max_pages, num_pages, free, rot):
    return ostore.OracleStore(hkv, max_seqs, max_pages, num_pages, free, rot)
