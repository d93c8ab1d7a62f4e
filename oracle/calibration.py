"""Key- and value-rotation calibration, fp64.  Test infrastructure only (see package header).

Follows axbrief, section "어텐션 통계 기반 회전과 Triton 커널의 결합" (attention-
statistics rotation): the key rotation is built from the eigenvectors U_Q of the
query covariance C_Q = (1/N) sum_n q_n^T q_n, times a normalized Hadamard
matrix, times a bit-reversal permutation: R_K = U_Q . H_Had . P_br.  The
techllm OSCAR section adds that the Hadamard + bit-reversal stage spreads the
important directions evenly over the channels.

Readings taken where the pages are silent:
* q_n are row vectors, so q_n^T q_n is the d x d outer product; no mean is
  subtracted (the printed formula has none).
* eigenvectors ordered by descending eigenvalue (stable), each column's
  largest-magnitude entry made positive (lowest index on ties).
* H_Had is the Sylvester Hadamard matrix in natural order, scaled by 1/sqrt(d).
* (x . P_br)_j = x_{br(j)} with br the log2(d)-bit index reversal.
* a key row k is rotated as k' = k . R_K; a query row likewise, q' = q . R_K.

Parity: pinned (orthogonality, closed-form H and P_br, exact-covariance
eigen input, statistical spectrum, attention equivalence; value side: the
printed C_S against the second moment of the attention outputs, a closed-form
eigenbasis, exact output equivalence of rotated values and the folded output
projection).
"""
from __future__ import annotations

import numpy as np


def second_moment(q_rows) -> np.ndarray:
    """C = (1/N) sum_n q_n^T q_n with q_n the rows of ``q_rows`` (fp64)."""
    q = np.asarray(q_rows, dtype=np.float64)
    return (q.T @ q) / q.shape[0]


def eig_descending(c: np.ndarray):
    """Eigen-decomposition of a symmetric matrix, descending order, canonical signs."""
    w, u = np.linalg.eigh(np.asarray(c, dtype=np.float64))
    order = np.argsort(-w, kind="stable")
    w = w[order]
    u = u[:, order].copy()
    for j in range(u.shape[1]):
        i = int(np.argmax(np.abs(u[:, j])))  # first index among equal magnitudes
        if u[i, j] < 0:
            u[:, j] = -u[:, j]
    return w, u


def sylvester_hadamard(n: int) -> np.ndarray:
    """H[i, j] = (-1)^popcount(i & j) / sqrt(n), n a power of two."""
    assert n > 0 and n & (n - 1) == 0
    i = np.arange(n)
    bits = i[:, None] & i[None, :]
    parity = np.zeros_like(bits)
    while bits.any():
        parity ^= bits & 1
        bits = bits >> 1
    return np.where(parity == 1, -1.0, 1.0) / np.sqrt(n)


def bit_reverse_indices(n: int) -> np.ndarray:
    nbits = n.bit_length() - 1
    assert 1 << nbits == n
    out = np.zeros(n, dtype=np.int64)
    for j in range(n):
        r = 0
        for b in range(nbits):
            if j >> b & 1:
                r |= 1 << (nbits - 1 - b)
        out[j] = r
    return out


def bit_reversal_matrix(n: int) -> np.ndarray:
    """P with (x . P)_j = x_{br(j)}, i.e. P[br(j), j] = 1."""
    br = bit_reverse_indices(n)
    p = np.zeros((n, n))
    p[br, np.arange(n)] = 1.0
    return p


def key_rotation(q_rows):
    """R_K = U_Q . H . P_br (fp64) and the eigenvalues of C_Q (descending)."""
    c = second_moment(q_rows)
    w, u = eig_descending(c)
    d = c.shape[0]
    return u @ sylvester_hadamard(d) @ bit_reversal_matrix(d), w


# ---------------------------------------------------------------- value side
# Same page and section: the value rotation is R_V = U_S . H_Had . P_br with U_S
# the eigenvectors of C_S = (1/N) V^T S^T S V, where S holds the calibration
# queries' attention probabilities over the calibration tokens and V their
# values; R_V is absorbed offline into the value and output projections, so the
# cache stores values already rotated and attention outputs come out in the
# R_V basis.
#
# Readings: S is [N queries, T tokens] (rows sum to 1), V is [T, d]; (S V) holds
# the N attention outputs as rows, so C_S is their second moment (no mean
# subtracted); GQA: the queries of every head that reads the KV head are pooled
# (as for C_Q); ordering, signs, H and P_br as for R_K.

def value_moment(s, v) -> np.ndarray:
    """C_S = (1/N) V^T S^T S V, evaluated as printed (fp64)."""
    s = np.asarray(s, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    return v.T @ s.T @ s @ v / s.shape[0]


def value_rotation(s, v):
    """R_V = U_S . H . P_br (fp64) and the eigenvalues of C_S (descending)."""
    c = value_moment(s, v)
    w, u = eig_descending(c)
    d = c.shape[0]
    return u @ sylvester_hadamard(d) @ bit_reversal_matrix(d), w


def fold_value_rotation(w_v, w_o, r_v, hq: int, hkv: int):
    """Absorb R_V into the projections (fp64): for KV head h the value-projection
    columns h*d .. h*d+d-1 become W_V[:, block] . R_V[h] (values come out rotated),
    and for every query head j reading KV head h = j // (hq/hkv) the output-
    projection rows j*d .. j*d+d-1 become R_V[h]^T . W_O[block] (undoing the
    rotation of that head's attention output)."""
    w_v = np.array(w_v, dtype=np.float64)
    w_o = np.array(w_o, dtype=np.float64)
    r_v = np.asarray(r_v, dtype=np.float64)
    d = r_v.shape[-1]
    g = hq // hkv
    for h in range(hkv):
        w_v[:, h * d:(h + 1) * d] = w_v[:, h * d:(h + 1) * d] @ r_v[h]
    for j in range(hq):
        h = j // g
        w_o[j * d:(j + 1) * d, :] = r_v[h].T @ w_o[j * d:(j + 1) * d, :]
    return w_v, w_o
