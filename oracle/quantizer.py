"""Range clipping + per-token asymmetric INT2 quantizer.  Test infrastructure only.

Follows axbrief, section "어텐션 통계 기반 회전과 Triton 커널의 결합": on the write
path each (rotated) token is clipped with the calibrated thresholds c_K = 0.96
(keys) and c_V = 0.92 (values) to limit outliers, then quantized per token,
asymmetrically, to INT2 in groups of G_K = 64 channels.  INT2 has four levels
(axbrief introduction; gist section "문제점").

Readings taken where the pages are silent (each step below is one IEEE fp32
operation, round to nearest even, never fused):
1. mn, mx = min and max of the 64 values of the group (exact).
2. r  = mx - mn
3. w  = c * r                      (clipped width: the range shrinks to c*r)
4. lo = mn + 0.5 * (r - w)         (trim (1-c)/2 of the range from each end)
5. s  = w / 3                      (correctly rounded division; 4 levels)
6. s16 = fp16(s), lo16 = fp16(lo)  (stored metadata, round to nearest even)
7. if s16 == 0 every code is 0; else inv = fp32(1 / s16),
   t = fp32(fp32(x - lo16) * inv), code = clamp(round_half_even(t), 0, 3).
   The pages fix no precision for this decision, so it is taken in the
   kernel's precision (fp32), the same sequence on both sides.
Dequantized value: lo16 + s16 * code.

Parity: pinned (hand-worked golden groups, four-level range, brute-force
nearest level, error bound, clipping width and midpoint).
"""
from __future__ import annotations

import numpy as np

GROUP = 64
C_K = np.float32(0.96)
C_V = np.float32(0.92)


def quantize(x, c):
    """Quantize float32 rows ``x[..., 128]``.

    Returns (codes uint8 [..., 128], s16 float16 [..., n_groups], lo16 float16 [..., n_groups]).
    """
    x = np.asarray(x, dtype=np.float32)
    c = np.float32(c)
    d = x.shape[-1]
    assert d % GROUP == 0
    xg = x.reshape(x.shape[:-1] + (d // GROUP, GROUP))
    mn = xg.min(axis=-1)
    mx = xg.max(axis=-1)
    r = (mx - mn).astype(np.float32)
    w = (c * r).astype(np.float32)
    half = (np.float32(0.5) * (r - w).astype(np.float32)).astype(np.float32)
    lo32 = (mn + half).astype(np.float32)
    s32 = (w / np.float32(3.0)).astype(np.float32)
    s16 = s32.astype(np.float16)
    lo16 = lo32.astype(np.float16)
    s_f = s16.astype(np.float32)
    lo_f = lo16.astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        inv = np.where(s_f != 0, np.float32(1.0) / np.where(s_f != 0, s_f, np.float32(1.0)),
                       np.float32(0.0)).astype(np.float32)
    diff = (xg - lo_f[..., None]).astype(np.float32)
    t = (diff * inv[..., None]).astype(np.float32)
    codes = np.clip(np.rint(t), 0, 3).astype(np.uint8)
    codes = np.where((s_f != 0)[..., None], codes, np.uint8(0))
    return codes.reshape(x.shape), s16, lo16


def dequantize(codes, s16, lo16) -> np.ndarray:
    """lo16 + s16 * code in fp64, shape [..., 128]."""
    codes = np.asarray(codes)
    d = codes.shape[-1]
    cg = codes.reshape(codes.shape[:-1] + (d // GROUP, GROUP)).astype(np.float64)
    out = np.asarray(lo16, dtype=np.float64)[..., None] + np.asarray(s16, dtype=np.float64)[..., None] * cg
    return out.reshape(codes.shape)


def boundary_distance(x, s16, lo16) -> np.ndarray:
    """|t - b| in fp64 for the nearest rounding boundary b in {0.5, 1.5, 2.5}, per element.

    Used by the parity rule: a code mismatch is explained when the value lies within
    1e-3 * s16 of a boundary.  Groups with s16 == 0 give +inf.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    xg = x.reshape(x.shape[:-1] + (d // GROUP, GROUP))
    s = np.asarray(s16, dtype=np.float64)[..., None]
    lo = np.asarray(lo16, dtype=np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        t = (xg - lo) / s
    dist = np.min(np.abs(t[..., None] - np.array([0.5, 1.5, 2.5])), axis=-1)
    dist = np.where(s == 0, np.inf, dist)
    return dist.reshape(x.shape)
