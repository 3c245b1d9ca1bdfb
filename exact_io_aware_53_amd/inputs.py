"""Seeded synthetic inputs and the named workloads.

This module only draws random numbers and rounds them to the storage dtype; it
holds none of the attention arithmetic. Both the GPU library's tests/bench and
the CPU oracle consume what it returns, so the two sides always see the same
input values.

Recipe: i.i.d. standard normals from NumPy's PCG64 generator in float32, drawn
in the order Q, K, V, dO, then rounded to the workload dtype (bf16 by
round-to-nearest-even via torch on the CPU). A query multiplier (a power of
two, so exact in bf16) widens the score range for the softmax-stress workload.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str            # "bf16" or "f32"
    causal: bool
    dropout_p: float = 0.0
    q_mult: float = 1.0
    backward: bool = False
    data_seed: int = 0
    row_seed: int = 0     # seeds the sample of query rows checked at full size
    head_seed: int = 0    # seeds the sample of heads checked at full size
    dropout_seed: int = 0x0123456789ABCDEF

    @property
    def scale(self) -> float:
        return float(1.0 / np.sqrt(self.d))

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def fwd_flops(self) -> float:
        """Counted forward FLOPs: 4*B*H*N^2*d, halved when causal."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2 if self.causal else f

    def bwd_flops(self) -> float:
        """Counted backward FLOPs: 2.5x the forward count (five products against two)."""
        return 2.5 * self.fwd_flops()


# The five workloads the library is specified on; named by what they are.
WORKLOADS = {
    w.name: w for w in [
        Workload("fwd_f32_b1h1n128d64", 1, 1, 128, 64, "f32", causal=False,
                 data_seed=1001, row_seed=2001, head_seed=3001),
        Workload("fwd_causal_bf16_b4h16n2048d64", 4, 16, 2048, 64, "bf16", causal=True,
                 data_seed=1002, row_seed=2002, head_seed=3002),
        Workload("fwd_causal_q4_bf16_b2h32n8192d128", 2, 32, 8192, 128, "bf16", causal=True,
                 q_mult=4.0, data_seed=1003, row_seed=2003, head_seed=3003),
        Workload("fwdbwd_causal_dropout_bf16_b2h16n4096d64", 2, 16, 4096, 64, "bf16",
                 causal=True, dropout_p=0.1, backward=True,
                 data_seed=1004, row_seed=2004, head_seed=3004),
        Workload("fwd_causal_bf16_b1h16n32768d128", 1, 16, 32768, 128, "bf16", causal=True,
                 data_seed=1005, row_seed=2005, head_seed=3005),
    ]
}


@dataclass(frozen=True)
class DecodeWorkload:
    """Nq query rows (the newest positions) against an Nk-row key/value sequence."""
    name: str
    B: int
    H: int
    Nq: int
    Nk: int
    d: int
    causal: bool          # query i at key position Nk - Nq + i
    data_seed: int = 0
    head_seed: int = 0
    page: int = 0         # > 0: K/V stored in shuffled pages of this many rows

    @property
    def scale(self) -> float:
        return float(1.0 / np.sqrt(self.d))

    def io_bytes(self) -> float:
        """Algorithmic HBM bytes: Q, K, V read once; O and LSE written once (bf16, fp32 LSE)."""
        return 2.0 * self.B * self.H * self.d * (2 * self.Nq + 2 * self.Nk) + 4.0 * self.B * self.H * self.Nq


# Decode-shaped workloads (a new token, and a 16-token block, against a long cache).
DECODE_WORKLOADS = {
    w.name: w for w in [
        DecodeWorkload("decode_bf16_b4h32q1k16384d128", 4, 32, 1, 16384, 128, causal=True,
                       data_seed=1011, head_seed=3011),
        DecodeWorkload("decode_causal_bf16_b8h16q16k8192d64", 8, 16, 16, 8192, 64, causal=True,
                       data_seed=1012, head_seed=3012),
        DecodeWorkload("decode_paged128_bf16_b4h32q1k16384d128", 4, 32, 1, 16384, 128, causal=True,
                       data_seed=1011, head_seed=3011, page=128),
    ]
}


def make_decode_inputs(w: DecodeWorkload):
    """Q [B,H,Nq,d], K and V [B,H,Nk,d] bf16 CPU tensors (drawn in that order). Paged
    workloads also get the page pools k_pages, v_pages [B*Nk/page, H, page, d], holding
    the same rows in a seeded random page order, the block table [B, Nk/page] (int32)
    and seq_lens [B] (int32, all Nk)."""
    rng = np.random.Generator(np.random.PCG64(w.data_seed))
    out = {}
    for name, n in (("q", w.Nq), ("k", w.Nk), ("v", w.Nk)):
        x = rng.standard_normal((w.B, w.H, n, w.d), dtype=np.float32)
        out[name] = torch.from_numpy(x).to(torch.bfloat16)
    if w.page:
        nb = w.Nk // w.page
        perm = torch.from_numpy(rng.permutation(w.B * nb).astype(np.int64))
        table = perm.view(w.B, nb)
        for name in ("k", "v"):
            blocks = out[name].view(w.B, w.H, nb, w.page, w.d).permute(0, 2, 1, 3, 4).reshape(
                w.B * nb, w.H, w.page, w.d)
            pool = torch.empty_like(blocks)
            pool[table.reshape(-1)] = blocks
            out[name + "_pages"] = pool
        out["block_table"] = table.to(torch.int32).contiguous()
        out["seq_lens"] = torch.full((w.B,), w.Nk, dtype=torch.int32)
    return out


def normal_tensors(shape, seed: int, count: int, dtype, mults=None):
    """`count` tensors of i.i.d. N(0,1) values (CPU torch tensors of `dtype`)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    for t in range(count):
        x = rng.standard_normal(shape, dtype=np.float32)
        if mults is not None and mults[t] != 1.0:
            x *= np.float32(mults[t])
        out.append(torch.from_numpy(x).to(dtype))
    return out


def make_inputs(w: Workload, with_grad_out: bool | None = None):
    """Q, K, V (and dO for backward workloads) as contiguous [B,H,N,d] CPU tensors."""
    with_grad_out = w.backward if with_grad_out is None else with_grad_out
    shape = (w.B, w.H, w.N, w.d)
    count = 4 if with_grad_out else 3
    mults = [w.q_mult, 1.0, 1.0, 1.0][:count]
    ts = normal_tensors(shape, w.data_seed, count, w.torch_dtype, mults)
    names = ["q", "k", "v", "do"][:count]
    return dict(zip(names, ts))


def sample_heads(w, count: int):
    """`count` distinct (b, h) pairs drawn from the workload's head seed."""
    rng = np.random.Generator(np.random.PCG64(w.head_seed))
    flat = rng.choice(w.B * w.H, size=min(count, w.B * w.H), replace=False)
    return [(int(f) // w.H, int(f) % w.H) for f in flat]


def sample_rows(w: Workload, count: int, block_rows=(128,)):
    """Sorted query rows: the tile-boundary rows plus `count` seeded random rows."""
    rng = np.random.Generator(np.random.PCG64(w.row_seed))
    fixed = {0, 1, w.N - 1}
    for br in block_rows:
        fixed |= {br - 1, br, min(w.N - 1, 2 * br - 1)}
    fixed = {r for r in fixed if 0 <= r < w.N}
    rand = rng.choice(w.N, size=min(count, w.N), replace=False)
    return np.array(sorted(fixed | {int(r) for r in rand}), dtype=np.int64)


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact fp64 copy of a CPU tensor (bf16 and fp32 widen exactly)."""
    return t.detach().to("cpu", torch.float64).numpy()


# Coverage workloads: head sizes, fp16, [B, N, H, d] storage and packed
# variable-length batches, each at a size that fills the GPU.
@dataclass(frozen=True)
class CoverageWorkload:
    name: str
    B: int                # batch entries (sequences for "varlen")
    H: int
    N: int                # sequence length; for "varlen" the longest allowed
    d: int
    dtype: str            # "bf16" or "fp16"
    layout: str           # "bhsd", "bshd" or "varlen"
    causal: bool = True
    data_seed: int = 0
    len_lo: int = 0       # "varlen": lengths uniform in [len_lo, N]
    head_seed: int = 0

    @property
    def scale(self) -> float:
        return float(1.0 / np.sqrt(self.d))

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float16

    def lengths(self) -> np.ndarray:
        if self.layout != "varlen":
            return np.full(self.B, self.N, dtype=np.int64)
        rng = np.random.Generator(np.random.PCG64(self.data_seed + 1))
        return rng.integers(self.len_lo, self.N + 1, size=self.B)

    def fwd_flops(self) -> float:
        """4 * H * n^2 * d per sequence, halved when causal."""
        f = float(sum(4.0 * self.H * int(n) * int(n) * self.d for n in self.lengths()))
        return f / 2 if self.causal else f

    def bwd_flops(self) -> float:
        return 2.5 * self.fwd_flops()


COVERAGE_WORKLOADS = {
    w.name: w for w in [
        CoverageWorkload("cov_d256_bf16_b2h16n4096", 2, 16, 4096, 256, "bf16", "bhsd", data_seed=1101),
        CoverageWorkload("cov_d96_bf16_b2h16n4096", 2, 16, 4096, 96, "bf16", "bhsd", data_seed=1102),
        CoverageWorkload("cov_d32_bf16_b2h16n4096", 2, 16, 4096, 32, "bf16", "bhsd", data_seed=1103),
        CoverageWorkload("cov_fp16_b2h32n8192d128", 2, 32, 8192, 128, "fp16", "bhsd", data_seed=1104),
        CoverageWorkload("cov_bshd_bf16_b2h32n8192d128", 2, 32, 8192, 128, "bf16", "bshd", data_seed=1105),
        CoverageWorkload("cov_varlen_bf16_32seq_h16d128", 32, 16, 4096, 128, "bf16", "varlen",
                         data_seed=1106, len_lo=128),
    ]
}


def make_coverage_inputs(w: CoverageWorkload):
    """Q, K, V, dO as CPU tensors in the workload's storage: [B, H, N, d] ("bhsd"),
    [B, N, H, d] ("bshd"), or packed [total, H, d] with cu_seqlens [B+1] int32
    ("varlen"). Values drawn as in normal_tensors, in the storage shape."""
    if w.layout == "varlen":
        lens = w.lengths()
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        ts = normal_tensors((int(cu[-1]), w.H, w.d), w.data_seed, 4, w.torch_dtype)
        out = dict(zip(("q", "k", "v", "do"), ts))
        out["cu_seqlens"] = torch.from_numpy(cu)
        return out
    shape = (w.B, w.N, w.H, w.d) if w.layout == "bshd" else (w.B, w.H, w.N, w.d)
    return dict(zip(("q", "k", "v", "do"), normal_tensors(shape, w.data_seed, 4, w.torch_dtype)))
