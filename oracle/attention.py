"""Plain fp64 CPU oracle: standard (materialising) scaled dot-product attention.

TEST INFRASTRUCTURE. Only tests/, the smoke check in __graft_entry__.py and the
CPU-baseline leg of bench.py may import or run this module. It is slow and
obvious on purpose: it forms the full score and probability rows in fp64 and
uses library matmuls, with no tiling, fusion or reordering. It shares no code
with the GPU library.

What it computes
----------------
The pages state that the tiled, IO-aware method returns the same result as
standard attention up to ordinary floating-point differences (inferensys
glossary "FlashAttention", opening paragraph; DL0056 FlashAttention, answer
paragraph and point (3) "Exact Result"; emergent.sh "Flash Attention", section
"Flash Attention vs. Regular Attention"; mbrenndoerfer "FlashAttention (2022) >
The Solution", last paragraph). So the oracle is that plain definition:

* scores S_ij = s * <Q_i, K_j> with s = 1/sqrt(d) (DL0056, "Mathematical
  Formulation": the scaled score between query row i and key row j);
* causal masking: query i sees keys j <= i only (inferensys, paragraph on
  causal masking); a masked score takes no part in the softmax. When the
  query rows are the last Nq positions of a longer key sequence (new tokens
  against the key/value cache that inference servers keep; inferensys,
  paragraph on integration with inference servers), query i sits at key
  position key_offset + i and sees keys j <= key_offset + i;
* row softmax P = softmax(S) and O = P V (emergent.sh, section "Why Regular
  Attention Becomes a Bottleneck": scores, softmax weights, weighted values);
* the per-row statistic that the method keeps for the backward pass is the
  log-sum-exp LSE_i = m_i + ln(l_i), with m_i and l_i the final row maximum and
  denominator of the DL0056 recurrence;
* dropout (inverted): O = (P o Z / (1 - p)) V with Z the Bernoulli keep mask
  of oracle.philox; LSE excludes dropout.

Backward pass, given dO: D_i = <dO_i, O_i>; dV = (P o Z/(1-p))^T dO;
dP = (dO V^T) o Z/(1-p); dS = P o (dP - D); dQ = s dS K; dK = s dS^T Q. These
are the gradients of the forward above (chain rule through the softmax); the
pages only say that the backward gradients are fused into kernels (DL0056,
point (3)) and that the score and probability blocks are recomputed rather
than stored (inferensys, paragraph on recomputation).

Pins: tests/test_oracle.py checks these functions against pure-Python brute
force, PyTorch's float64 scaled_dot_product_attention and its autograd,
closed forms (uniform scores, one key, causal row 0, shift invariance),
central finite differences and the tiled recurrence of oracle.recurrence.
"""
from __future__ import annotations

import numpy as np

from .philox import keep_mask


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _dropout_p(dropout_p) -> float:
    # The probability is a float32 argument of the library; use that exact value.
    p = float(np.float32(dropout_p))
    if not (0.0 <= p < 1.0):
        raise ValueError("dropout probability must lie in [0, 1)")
    return p


def scores(q, k, scale: float, causal: bool, rows=None, key_offset: int = 0) -> np.ndarray:
    """Scaled scores of the given query rows against every key, masked entries = -inf.

    Causal: query row i sees keys j <= key_offset + i.
    """
    q, k = _f64(q), _f64(k)
    n = k.shape[0]
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    s = float(scale) * (q[rows] @ k.T)
    if causal:
        s[np.arange(n)[None, :] > rows[:, None] + int(key_offset)] = -np.inf
    return s


def forward(q, k, v, scale: float, causal: bool = False, dropout_p=0.0, seed: int = 0,
            b: int = 0, h: int = 0, rows=None, key_offset: int = 0):
    """Attention output and log-sum-exp for one head (b, h).

    q: [Nq, d], k, v: [Nk, d] arrays (any real dtype; widened exactly to fp64).
    rows: query rows to evaluate (default: all Nq).
    key_offset: key position of query row 0 for the causal mask (0 when the
    queries and keys are the same sequence; Nk - Nq for the last Nq positions).
    Returns (O [len(rows), d], LSE [len(rows)]), both fp64.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    n = k.shape[0]
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    p = _dropout_p(dropout_p)
    s = scores(q, k, scale, causal, rows, key_offset)
    m = s.max(axis=1)
    with np.errstate(under="ignore"):
        lse = m + np.log(np.exp(s - m[:, None]).sum(axis=1))
        prob = np.exp(s - lse[:, None])
    if p > 0.0:
        z = keep_mask(b, h, rows, np.arange(n), p, seed)
        prob = prob * z / (1.0 - p)
    return prob @ v, lse


def backward(q, k, v, do, scale: float, causal: bool = False, dropout_p=0.0, seed: int = 0,
             b: int = 0, h: int = 0):
    """Gradients (dQ, dK, dV) of one head, plus the oracle's own (O, LSE, D).

    The full N x N score and probability matrices are materialised (fp64).
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    n = k.shape[0]
    p = _dropout_p(dropout_p)
    s = scores(q, k, scale, causal)
    m = s.max(axis=1)
    with np.errstate(under="ignore"):
        lse = m + np.log(np.exp(s - m[:, None]).sum(axis=1))
        prob = np.exp(s - lse[:, None])
    if p > 0.0:
        zs = keep_mask(b, h, np.arange(n), np.arange(n), p, seed) / (1.0 - p)
    else:
        zs = np.ones_like(prob)
    pd = prob * zs
    o = pd @ v
    dsum = (do * o).sum(axis=1)
    dv = pd.T @ do
    dp = (do @ v.T) * zs
    ds = prob * (dp - dsum[:, None])
    dq = float(scale) * (ds @ k)
    dk = float(scale) * (ds.T @ q)
    return dq, dk, dv, (o, lse, dsum)
