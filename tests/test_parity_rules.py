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
    """k . R as the write kernel forms it: R as three bf16 terms, the bf16 keys as they are, exact
    products, each of the 12 partial sums (3 terms x 4 K-steps of 32 channels, the smallest term
    first) rounded once into an fp32 accumulator."""
    t0 = _bf16_round(r)
    d1 = (r - t0).astype(np.float32)
    t1 = _bf16_round(d1)
    t2 = _bf16_round((d1 - t1).astype(np.float32))
    acc = np.zeros((k.shape[0], D), np.float32)
    for rr in (t2, t1, t0):
        for kk in range(4):
            sl = slice(32 * kk, 32 * kk + 32)
            acc = (acc.astype(np.float64) + k[:, sl] @ rr[sl].astype(np.float64)).astype(np.float32)
    return acc


def _setup(n=40000):
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
    # the bf16 split of R: residual within 2^-24 |R|; two terms leave a residual above 2^-18 |R|
    rr = r.astype(np.float64)
    t0 = _bf16_round(r)
    d1 = (r - t0).astype(np.float32)
    t1 = _bf16_round(d1)
    t2 = _bf16_round((d1 - t1).astype(np.float32))
    assert np.all(np.abs(rr - t0 - t1 - t2) <= 2.0 ** -24 * np.abs(rr))
    assert (np.abs(rr - t0 - t1) / np.abs(rr)).max() > 2.0 ** -18


def test_key_metadata_flips_explained_only_by_rotation_error():
    k, r, x_ref, bound = _setup()
    x_gpu = _emulated_rotation(k, r)
    _, _, s16, lo16 = quantizer.params(x_gpu, quantizer.C_K)
    _, _, s16o, lo16o = quantizer.params(x_ref, quantizer.C_K)
    flips = (s16 != s16o) | (lo16 != lo16o)
    assert flips.sum() > 5                       # the emulation does flip some groups
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


def _pages_from(codes_k, s_k, lo_k, codes_v, s_v, lo_v):
    from oracle import layout
    n = len(codes_k)
    blocks = []
    for p0 in range(0, n, 64):
        sl = slice(p0, min(n, p0 + 64))
        blocks.append(layout.pack_head_block(codes_k[sl], codes_v[sl], s_k[sl], lo_k[sl], s_v[sl], lo_v[sl]))
    return np.stack(blocks)[:, None, :]          # [pages, 1 head, 5120]


def test_code_rule_in_groups_with_a_flipped_minimum():
    """A key group whose fp16 minimum flipped by one ulp that is large against the scale moves an
    element across a rounding boundary by more than the 1e-3 band: the mismatch is explained
    only when the GPU's code is the exact decision under the GPU's own metadata; any other code
    there stays unexplained."""
    x = np.zeros((1, D), np.float64)
    x[0, :64] = np.linspace(8.0, 8.9, 64)
    x[0, 64:] = np.linspace(-1, 1, 64)
    x32 = x.astype(np.float32)
    co, so, lo_ = quantizer.quantize(x32, quantizer.C_K)
    # the "GPU" minimum one fp16 ulp above the oracle's (ulp 2^-7 at 8: 0.0078, s16 ~ 0.29)
    lg = lo_.copy()
    lg[0, 0] = (lo_[0, 0:1].view(np.uint16) + 1).view(np.float16)[0]
    s = float(so[0, 0])
    assert (float(lg[0, 0]) - float(lo_[0, 0])) / s > 2e-3
    # an element between the two decisions' boundaries: its code differs, both distances > 1e-3
    b = float(lo_[0, 0]) + 1.5 * s + 0.5 * (float(lg[0, 0]) - float(lo_[0, 0]))
    x32[0, 5] = np.float32(b)
    co, so, lo_ = quantizer.quantize(x32, quantizer.C_K)
    cg = parity.exact_codes(x32.astype(np.float64), so, lg)
    assert cg[0, 5] != co[0, 5]
    cv, sv, lv = quantizer.quantize(x32, quantizer.C_V)
    ora = _pages_from(co, so, lo_, cv, sv, lv)
    table = np.zeros((1, 1), np.int32)
    x64 = x32.astype(np.float64)
    bound = np.full((1, D), 2.0 ** -10)
    rep = parity.compare_int2_unit(_pages_from(cg, so, lg, cv, sv, lv), table, ora, table, 0, 0, 0, 1, x64, x64,
                                   k_bound=bound)
    assert rep["code_mismatch"] >= 1 and rep["unexplained"] == 0 and rep["explained_by_meta"] >= 1, rep
    wrong = cg.copy()
    wrong[0, 5] = [c for c in range(4) if c not in (cg[0, 5], co[0, 5])][0]   # no metadata explains it
    rep = parity.compare_int2_unit(_pages_from(wrong, so, lg, cv, sv, lv), table, ora, table, 0, 0, 0, 1, x64,
                                   x64, k_bound=bound)
    assert rep["unexplained"] >= 1, rep
