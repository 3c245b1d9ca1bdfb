"""CPU oracle for exact scaled dot-product attention (fp64, NumPy).

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and the CPU-baseline
leg of bench.py may import anything from this package. The GPU library shares
no code with it and must never route a computation through it.

Contents
--------
attention   plain materialising forward/backward (the definition)
recurrence  the pages' tile-by-tile online-softmax recurrence (pins the reading)
philox      Philox-4x32-10 and the dropout keep mask
"""
from .attention import backward, forward, scores
from .philox import dropout_threshold, keep_mask, philox4x32_10, seed_to_key
from .recurrence import online_forward

__all__ = ["forward", "backward", "scores", "online_forward", "philox4x32_10",
           "keep_mask", "dropout_threshold", "seed_to_key"]
