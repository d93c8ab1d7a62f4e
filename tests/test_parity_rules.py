"""CPU checks of the GPU-vs-oracle tolerance rules themselves (tests/parity.py).

A tolerance that explains every difference would let a wrong kernel pass, so each rule is run
on a CPU emulation of the kernel's arithmetic (all differences must be explained) and on a
planted systematic error (differences must be reported as unexplained).
"""
import numpy as np

import parity
import synth
from oracle import calibration, quantizer

D = 128


def _bf16_round(x):
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def _emulated_rotation(k, r):
    """k . R as the write kernel forms it: R as two bf16 terms, exact products, each of the 8
    partial sums (4 K-steps of 32 channels x 2 terms) rounded once into an fp32 accumulator."""
    r0 = _bf16_round(r)
    r1 = _bf16_round(r - r0)
    acc = np.zeros((k.shape[0], D), np.float32)
    for ks in range(4):
        sl = slice(32 * ks, 32 * ks + 32)
        for rr in (r1, r0):
            acc = (acc.astype(np.float64) + k[:, sl] @ rr[sl].astype(np.float64)).astype(np.float32)
    return acc


def _setup(n=20000):
    q = synth.bf16_bits_to_f32(synth.calibration_queries(synth.CFG_QWEN3_4B, 0, 1)).astype(np.float64)
    r = calibration.key_rotation(q)[0].astype(np.float32)
    kb, _ = synth.unit_kv(synth.CFG_QWEN3_4B, 0, 2, 1, n)
    k = synth.bf16_bits_to_f32(kb).astype(np.float64)
    x_ref = (k @ r.astype(np.float64)).astype(np.float32).astype(np.float64)
    bound = parity.rotation_error_bound(kb, r) + 2.0 ** -24 * np.abs(x_ref)
    return k, r, x_ref, bound


def test_rotation_error_bound_holds_for_emulated_kernel():
    k, r, x_ref, bound = _setup()
    x_gpu = _emulated_rotation(k, r).astype(np.float64)
    assert np.all(np.abs(x_gpu - x_ref) <= bound)
    # the two-term split's residual is within 2^-16 |R|, and it is not within 2^-18 |R|
    r0 = _bf16_round(r)
    res = np.abs(r.astype(np.float64) - r0 - _bf16_round(r - r0)) / np.abs(r)
    assert res.max() <= 2.0 ** -16 and res.max() > 2.0 ** -18


def test_key_metadata_flips_explained_only_by_rotation_error():
    k, r, x_ref, bound = _setup()
    x_gpu = _emulated_rotation(k, r)
    _, _, s16, lo16 = quantizer.params(x_gpu, quantizer.C_K)
    _, _, s16o, lo16o = quantizer.params(x_ref, quantizer.C_K)
    flips = (s16 != s16o) | (lo16 != lo16o)
    assert flips.sum() > 20                      # the emulation does flip some groups
    s_ok, lo_ok = parity.meta_flip_explained(x_ref, quantizer.C_K, s16, lo16, bound)
    assert np.all(s_ok & lo_ok)
    # a systematic error: the clip constant off by 1e-4 moves the parameters of every group
    _, _, s16b, lo16b = quantizer.params(x_gpu, np.float32(0.9601))
    flips_b = (s16b != s16o) | (lo16b != lo16o)
    s_ok, lo_ok = parity.meta_flip_explained(x_ref, quantizer.C_K, s16b, lo16b, bound)
    bad = ~(s_ok & lo_ok)
    assert flips_b.sum() > 1000 and bad.sum() > 0.5 * flips_b.sum()


def test_code_band_explains_only_boundary_elements():
    """Codes decided in fp32 with a reciprocal scale (as the kernels do) differ from the exact
    decision only within the 1e-3 band; a code decided with a scale one fp16 ulp off does not."""
    _, _, x_ref, _ = _setup(4000)
    x32 = x_ref.astype(np.float32)
    codes, s16, lo16 = quantizer.quantize(x32, quantizer.C_K)
    s = s16.astype(np.float32)
    lo = lo16.astype(np.float32)
    inv = np.where(s != 0, np.float32(1) / np.where(s != 0, s, 1), 0).astype(np.float32)
    xg = x32.reshape(-1, 2, 64)
    t = ((xg - lo[..., None]).astype(np.float32) * inv[..., None]).astype(np.float32)
    c32 = np.clip(np.rint(t), 0, 3).astype(np.uint8).reshape(x32.shape)
    dist = quantizer.boundary_distance(x_ref, s16, lo16)
    mism = c32 != codes
    assert np.all(dist[mism] < 1e-3)
    s_bad = (s16.view(np.uint16) + 1).view(np.float16).astype(np.float32)
    t_bad = ((xg - lo[..., None]) / s_bad[..., None]).astype(np.float32)
    c_bad = np.clip(np.rint(t_bad), 0, 3).astype(np.uint8).reshape(x32.shape)
    mism_b = c_bad != codes
    # the parity rule allows no unexplained mismatch: this one leaves dozens
    assert mism_b.sum() > 100 and np.sum(dist[mism_b] >= 1e-3) > 20
