"""Counter-based dropout randomness for the oracle: Philox-4x32-10 and the keep mask.

TEST INFRASTRUCTURE. This module belongs to the CPU oracle. Only tests/, the
smoke check in __graft_entry__.py and the CPU-baseline leg of bench.py may use
it; the GPU library never imports, links or calls it, and it shares no code
with the GPU library.

Sources
-------
* Attention dropout that the backward pass regenerates instead of storing:
  inferensys glossary "FlashAttention" (paragraph on causal masking and
  dropout: a Bernoulli draw per attention score, applied block-wise inside the
  softmax step) and emergent.sh glossary "Flash Attention", section "Key
  Components of Flash Attention" (training kernels regenerate the same random
  pattern during recomputation rather than storing a mask).
* The pages name no generator. The workload this library is measured on keys a
  Philox-4x32 generator by the seed with counter (b, h, i, j). Philox-4x32-10
  is the published counter-based generator of Salmon, Moraes, Dror and Shaw,
  "Parallel random numbers: as easy as 1, 2, 3" (SC'11): ten rounds, each
  multiplying words 0 and 2 by the two round multipliers into 64-bit products
  and mixing the high halves with words 1, 3 and the round key; the key is
  advanced by the two Weyl increments between rounds.

Readings (the pages are silent on all of these)
-----------------------------------------------
* key = (seed mod 2**32, seed >> 32); counter words (c0, c1, c2, c3) =
  (b, h, i, j), with i and j absolute query and key rows inside head (b, h).
* One generator call per attention element; only output word 0 is used.
* Keep iff word0 >= thr with thr = ceil(p * 2**32), p being the float32
  dropout probability widened exactly to double. The drop probability is then
  thr / 2**32, within 2**-32 of p.

Pinned by tests/test_oracle.py against AMD's open-source rocRAND Philox engine
(an independent implementation, compiled as host code) and by the measured
keep fraction.
"""
from __future__ import annotations

import math

import numpy as np

MASK32 = np.uint64(0xFFFFFFFF)
# Round multipliers and Weyl key increments of Philox-4x32 (Salmon et al., SC'11).
PHILOX_M0 = np.uint64(0xD2511F53)
PHILOX_M1 = np.uint64(0xCD9E8D57)
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
PHILOX_ROUNDS = 10


def philox4x32_10(c0, c1, c2, c3, k0: int, k1: int):
    """Philox-4x32-10 block function, vectorised over the counter words.

    c0..c3: integer arrays (broadcastable) holding 32-bit counter words.
    k0, k1: the two 32-bit key words.
    Returns the four 32-bit output words as uint64 arrays.
    """
    x0, x1, x2, x3 = (np.asarray(c, dtype=np.uint64) & MASK32 for c in (c0, c1, c2, c3))
    x0, x1, x2, x3 = np.broadcast_arrays(x0, x1, x2, x3)
    key0, key1 = int(k0) & 0xFFFFFFFF, int(k1) & 0xFFFFFFFF
    for rnd in range(PHILOX_ROUNDS):
        if rnd > 0:
            key0 = (key0 + PHILOX_W0) & 0xFFFFFFFF
            key1 = (key1 + PHILOX_W1) & 0xFFFFFFFF
        p0 = PHILOX_M0 * x0  # < 2**64: exact in uint64
        p1 = PHILOX_M1 * x2
        hi0, lo0 = p0 >> np.uint64(32), p0 & MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & MASK32
        x0, x1, x2, x3 = (hi1 ^ x1 ^ np.uint64(key0), lo1,
                          hi0 ^ x3 ^ np.uint64(key1), lo0)
    return x0, x1, x2, x3


def seed_to_key(seed: int):
    """Split the 64-bit seed into the two Philox key words (low word first)."""
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    return seed & 0xFFFFFFFF, seed >> 32


def dropout_threshold(dropout_p) -> int:
    """thr = ceil(p * 2**32) for the float32 value of p; an element is dropped iff word0 < thr."""
    p = float(np.float32(dropout_p))
    if not (0.0 <= p < 1.0):
        raise ValueError("dropout probability must lie in [0, 1)")
    return int(math.ceil(p * 4294967296.0))


def keep_mask(b: int, h: int, rows, cols, dropout_p, seed: int) -> np.ndarray:
    """Bernoulli keep mask Z[r, c] for query rows `rows` and key columns `cols` of head (b, h).

    Returns a bool array of shape (len(rows), len(cols)); True means kept.
    """
    rows = np.asarray(rows, dtype=np.uint64).reshape(-1, 1)
    cols = np.asarray(cols, dtype=np.uint64).reshape(1, -1)
    thr = dropout_threshold(dropout_p)
    if thr == 0:
        return np.ones((rows.shape[0], cols.shape[1]), dtype=bool)
    k0, k1 = seed_to_key(seed)
    w0, _, _, _ = philox4x32_10(np.uint64(b), np.uint64(h), rows, cols, k0, k1)
    return w0 >= np.uint64(thr)
