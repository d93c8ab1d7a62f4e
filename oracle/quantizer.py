"""Range clipping + per-token asymmetric INT2 quantizer.  Test infrastructure only.

Follows axbrief, section "어텐션 통계 기반 회전과 Triton 커널의 결합": on the write
path each (rotated) token is clipped with the calibrated thresholds c_K = 0.96
(keys) and c_V = 0.92 (values) to limit outliers, then quantized per token,
asymmetrically, to INT2 in groups of G_K = 64 channels.  INT2 has four levels
(axbrief introduction; gist section "문제점").

Readings taken where the pages are silent (steps 2-6 are each one IEEE fp32
operation, round to nearest even, never fused; the stored metadata must come
out bit for bit the same from any implementation of the same sequence):
1. mn, mx = min and max of the 64 values of the group (exact).
2. r  = mx - mn
3. w  = c * r                      (clipped width: the range shrinks to c*r)
4. lo = mn + 0.5 * (r - w)         (trim (1-c)/2 of the range from each end)
5. s  = w / 3                      (correctly rounded division; 4 levels)
6. s16 = fp16(s), lo16 = fp16(lo)  (stored metadata, round to nearest even)
7. if s16 == 0 every code is 0; else t = (x - lo16) / s16 in fp64 and
   code = clamp(round_half_even(t), 0, 3).
Dequantized value: lo16 + s16 * code.

The code decision in step 7 is exact (fp64 of fp32/fp16 operands); an
implementation that takes it in fp32 can differ only where t lies within a few
fp32 ulps of a rounding boundary b in {0.5, 1.5, 2.5}.  ``boundary_distance``
measures |t - b| for the parity rule that tolerates such elements.

Parity: pinned (hand-worked golden groups, four-level range, brute-force
nearest level, error bound, clipping width and midpoint, boundary distances of
hand-placed values).
"""
from __future__ import annotations

import numpy as np

GROUP = 64
C_K = np.float32(0.96)
C_V = np.float32(0.92)


def params(x, c):
    """Steps 1-6 for float32 rows ``x[..., 128]``, per 64-channel group.

    Returns (s32, lo32, s16, lo16): the fp32 scale and minimum before the fp16
    rounding, and the stored fp16 values; each [..., n_groups].
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
    return s32, lo32, s32.astype(np.float16), lo32.astype(np.float16)


def quantize(x, c):
    """Quantize float32 rows ``x[..., 128]``.

    Returns (codes uint8 [..., 128], s16 float16 [..., n_groups], lo16 float16 [..., n_groups]).
    """
    x = np.asarray(x, dtype=np.float32)
    d = x.shape[-1]
    _, _, s16, lo16 = params(x, c)
    xg = x.reshape(x.shape[:-1] + (d // GROUP, GROUP)).astype(np.float64)
    s = s16.astype(np.float64)[..., None]
    lo = lo16.astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        t = (xg - lo) / np.where(s != 0, s, 1.0)
    codes = np.clip(np.rint(t), 0, 3).astype(np.uint8)     # np.rint: round half to even
    codes = np.where(s != 0, codes, np.uint8(0))
    return codes.reshape(x.shape), s16, lo16


def dequantize(codes, s16, lo16) -> np.ndarray:
    """lo16 + s16 * code in fp64, shape [..., 128]."""
    codes = np.asarray(codes)
    d = codes.shape[-1]
    cg = codes.reshape(codes.shape[:-1] + (d // GROUP, GROUP)).astype(np.float64)
    out = np.asarray(lo16, dtype=np.float64)[..., None] + np.asarray(s16, dtype=np.float64)[..., None] * cg
    return out.reshape(codes.shape)


def boundary_distance(x, s16, lo16) -> np.ndarray:
    """|t - b| in fp64 for the nearest rounding boundary b in {0.5, 1.5, 2.5}, per element,
    with t = (x - lo16) / s16.

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
