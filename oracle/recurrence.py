"""The online-softmax recurrence as the pages state it, in fp64, tile by tile.

TEST INFRASTRUCTURE. Used only by tests/ to pin the reading of the method:
streaming the keys in tiles with a running maximum and a rescaled running
denominator must reproduce the plain oracle (oracle.attention.forward).

Source: DL0056 FlashAttention (intvml), "Mathematical Formulation".
For key/value tile t, query row i and keys j of that tile, with scaled scores
S_ij = Q_i K_j^T / sqrt(d):

    m_i(t) = max(m_i(t-1), max_j S_ij),               m_i(0) = -inf
    l_i(t) = exp(m_i(t-1) - m_i(t)) * l_i(t-1) + sum_j exp(S_ij - m_i(t)),
                                                       l_i(0) = 0

The output update is not printed; the page (point (2)) and emergent.sh "Flash
Attention" (How it works, step 4) say each K,V tile updates the output block
without keeping earlier scores. The reading taken here rescales the output
accumulator exactly as the denominator is rescaled:

    A_i(t) = exp(m_i(t-1) - m_i(t)) * A_i(t-1) + sum_j exp(S_ij - m_i(t)) Z_ij V_j,
    A_i(0) = 0,    O_i = A_i(T) / (l_i(T) * (1 - p)),    LSE_i = m_i(T) + ln l_i(T).

Z is the dropout keep mask (all ones when p = 0); it scales the output update
only, never the denominator. While every score a row has seen is masked
(m_i = -inf), the rescale factor is taken as 1 and the tile adds nothing.
"""
from __future__ import annotations

import numpy as np

from .philox import keep_mask


def online_forward(q, k, v, scale: float, causal: bool, block: int, dropout_p=0.0,
                   seed: int = 0, b: int = 0, h: int = 0):
    """Tiled forward over key tiles of `block` rows; returns (O, LSE) for all query rows."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    nq, n = q.shape[0], k.shape[0]
    p = float(np.float32(dropout_p))
    m = np.full(nq, -np.inf)
    l = np.zeros(nq)
    acc = np.zeros((nq, v.shape[1]))
    rows = np.arange(nq)
    for j0 in range(0, n, block):
        cols = np.arange(j0, min(j0 + block, n))
        s = float(scale) * (q @ k[cols].T)
        if causal:
            s[cols[None, :] > rows[:, None]] = -np.inf
        m_new = np.maximum(m, s.max(axis=1))
        seen = np.isfinite(m_new)
        alpha = np.ones(nq)
        alpha[seen] = np.exp(m[seen] - m_new[seen])  # exp(-inf) = 0 on a row's first live tile
        pt = np.zeros_like(s)
        with np.errstate(under="ignore"):
            pt[seen] = np.exp(s[seen] - m_new[seen, None])
        l = alpha * l + pt.sum(axis=1)
        if p > 0.0:
            pt = pt * keep_mask(b, h, rows, cols, p, seed)
        acc = alpha[:, None] * acc + pt @ v[cols]
        m = m_new
    return acc / (l[:, None] * (1.0 - p)), m + np.log(l)
