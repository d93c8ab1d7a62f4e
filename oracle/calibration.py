"""Key-rotation calibration, fp64.  Test infrastructure only (see package header).

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
eigen input, statistical spectrum, attention equivalence).
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
