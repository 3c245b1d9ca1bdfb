"""GPU parity of the general entry points fa_fwd_ex / fa_bwd_ex against the
fp64 oracle: head sizes 32, 96 and 256, fp16 next to bf16, strided layouts
([B, N, H, d] storage, views into a packed QKV projection) and packed
variable-length batches.

Bars (the bf16 ones, which fp16's 11-bit significand meets a fortiori):
O max|err| <= 1e-2 (plus half a storage ulp only where |O_ref| >= 4, see
parity_checks), LSE <= 1e-3, gradients max|g - g_ref| / max|g_ref| <= 2e-2. A strided
call must give exactly the bits of the same call on contiguous copies: the
kernels do the same arithmetic, only the addresses differ.
"""
import math

import numpy as np
import pytest
import torch

import exact_io_aware_53_amd as fa
import oracle
from exact_io_aware_53_amd.inputs import normal_tensors, to_f64
from parity_checks import Stats

pytestmark = pytest.mark.gpu

SEED = 0x5EED0F00D
DT = {"bf16": torch.bfloat16, "fp16": torch.float16}
GRAD_TOL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.lib()


def rel_to_max(g, ref, fallback):
    denom = np.abs(ref).max()
    if fallback and denom < 1e-9 * fallback:
        denom = fallback
    if denom == 0.0:
        denom = 1.0
    return float(np.abs(g - ref).max() / denom)


def check_head(q, k, v, o, lse, causal, p, b, h, dtype, do=None, grads=None, tag=""):
    """q, k, v, do: [n, d] CPU tensors of one head (one sequence); o, lse, grads: GPU results."""
    d = q.shape[-1]
    scale = 1.0 / math.sqrt(d)
    ro, rl = oracle.forward(to_f64(q), to_f64(k), to_f64(v), scale, causal, p, SEED, b, h)
    st = Stats(dtype)
    st.add(o.double().cpu().numpy(), ro, lse.double().cpu().numpy(), rl)
    st.check(f"{tag} b={b} h={h}")
    if grads is None:
        return
    rq, rk, rv, _ = oracle.backward(to_f64(q), to_f64(k), to_f64(v), to_f64(do), scale, causal, p,
                                    SEED, b, h)
    head_max = max(np.abs(r).max() for r in (rq, rk, rv))
    for name, g, r in zip(("dq", "dk", "dv"), grads, (rq, rk, rv)):
        e = rel_to_max(g.double().cpu().numpy(), r, head_max)
        assert e <= GRAD_TOL, f"{name} rel-to-max error {e:.3e} (b={b}, h={h})"


# ------------------------------------------------------------ head sizes, dtypes

SHAPES = [(1, 2, 1, 32), (2, 1, 300, 32), (1, 2, 257, 96), (1, 1, 700, 96), (1, 2, 129, 256),
          (1, 1, 333, 256), (2, 2, 200, 64), (1, 1, 300, 128)]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("p", [0.0, 0.1])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_fwd_bwd_head_sizes_and_dtypes(shape, causal, p, dtype):
    B, H, N, d = shape
    dt = DT[dtype]
    q, k, v, do = normal_tensors(shape, 3100 + N + d, 4, dt)
    gq, gk, gv, gdo = (t.cuda() for t in (q, k, v, do))
    o, lse = fa.fwd_ex(gq, gk, gv, causal=causal, dropout_p=p, seed=SEED)
    dq, dk, dv = fa.bwd_ex(gq, gk, gv, o, lse, gdo, causal=causal, dropout_p=p, seed=SEED)
    torch.cuda.synchronize()
    for b in range(B):
        for h in range(H):
            check_head(q[b, h], k[b, h], v[b, h], o[b, h], lse[b, h], causal, p, b, h, dt,
                       do[b, h], (dq[b, h], dk[b, h], dv[b, h]),
                       tag=f"fwd_ex {shape} {dtype} causal={causal} p={p}")


@pytest.mark.parametrize("d", [64, 128])
def test_ex_matches_plain_entry_points_bitwise(d):
    """fa_fwd_ex / fa_bwd_ex on contiguous bf16 tensors are fa_fwd / fa_bwd."""
    q, k, v, do = (t.cuda() for t in normal_tensors((2, 3, 300, d), 3300 + d, 4, torch.bfloat16))
    for p in (0.0, 0.1):
        o1, l1 = fa.fwd(q, k, v, causal=True, dropout_p=p, seed=SEED)
        o2, l2 = fa.fwd_ex(q, k, v, causal=True, dropout_p=p, seed=SEED)
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        g1 = fa.bwd(q, k, v, o1, l1, do, causal=True, dropout_p=p, seed=SEED, deterministic=True)
        g2 = fa.bwd_ex(q, k, v, o1, l1, do, causal=True, dropout_p=p, seed=SEED, deterministic=True)
        for a, b in zip(g1, g2):
            assert torch.equal(a, b)


# ------------------------------------------------------------------- layouts

@pytest.mark.parametrize("d", [64, 96, 128])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_bshd_layout_equals_contiguous(d, dtype):
    """Q, K, V, dO stored [B, N, H, d] (viewed as [B, H, N, d]); O and the
    gradients written into [B, N, H, d] buffers too."""
    B, H, N = 2, 3, 333
    dt = DT[dtype]
    q, k, v, do = normal_tensors((B, H, N, d), 3400 + d, 4, dt)
    cq, ck, cv, cdo = (t.cuda() for t in (q, k, v, do))
    sq, sk, sv, sdo = (t.transpose(1, 2).contiguous().cuda().transpose(1, 2) for t in (q, k, v, do))
    assert sq.stride(2) == H * d
    o_c, l_c = fa.fwd_ex(cq, ck, cv, causal=True, dropout_p=0.1, seed=SEED)
    o_s = torch.empty((B, N, H, d), dtype=dt, device="cuda").transpose(1, 2)
    o_s, l_s = fa.fwd_ex(sq, sk, sv, causal=True, dropout_p=0.1, seed=SEED, out=o_s)
    assert torch.equal(o_c, o_s) and torch.equal(l_c, l_s)
    g_c = fa.bwd_ex(cq, ck, cv, o_c, l_c, cdo, causal=True, dropout_p=0.1, seed=SEED,
                    deterministic=True)
    g_s = fa.bwd_ex(sq, sk, sv, o_s, l_s, sdo, causal=True, dropout_p=0.1, seed=SEED,
                    deterministic=True,
                    dq=torch.empty((B, N, H, d), dtype=dt, device="cuda").transpose(1, 2),
                    dk=torch.empty((B, N, H, d), dtype=dt, device="cuda").transpose(1, 2),
                    dv=torch.empty((B, N, H, d), dtype=dt, device="cuda").transpose(1, 2))
    for a, b in zip(g_c, g_s):
        assert torch.equal(a, b)
    torch.cuda.synchronize()
    check_head(q[1, 2], k[1, 2], v[1, 2], o_s[1, 2], l_s[1, 2], True, 0.1, 1, 2, dt, do[1, 2],
               (g_s[0][1, 2], g_s[1][1, 2], g_s[2][1, 2]), tag=f"[B,N,H,d] d={d} {dtype}")


def test_packed_qkv_views():
    """q, k, v as views into one [B, N, 3, H, d] projection output (row stride 3*H*d)."""
    B, H, N, d = 2, 4, 280, 64
    qkv = normal_tensors((B, N, 3, H, d), 3500, 1, torch.bfloat16)[0].cuda()
    q, k, v = (qkv[:, :, i].transpose(1, 2) for i in range(3))
    assert q.stride(2) == 3 * H * d
    o, lse = fa.fwd_ex(q, k, v, causal=True)
    ref_o, ref_l = fa.fwd_ex(q.contiguous(), k.contiguous(), v.contiguous(), causal=True)
    assert torch.equal(o, ref_o) and torch.equal(lse, ref_l)
    torch.cuda.synchronize()
    qc, kc, vc = (t.cpu() for t in (q, k, v))
    check_head(qc[1, 3], kc[1, 3], vc[1, 3], o[1, 3], lse[1, 3], True, 0.0, 1, 3, torch.bfloat16,
               tag="packed QKV views")


# ------------------------------------------------------------ packed batches

def packed(lengths, H, d, dtype, seed, count):
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    total = int(cu[-1])
    ts = normal_tensors((total, H, d), seed, count, dtype)
    return cu, total, ts


@pytest.mark.parametrize("d", [64, 128, 32])
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_forward_backward(d, causal):
    lengths = [1, 300, 0, 129, 64, 517]
    H, p = 2, 0.1
    dt = torch.bfloat16
    cu, total, (q, k, v, do) = packed(lengths, H, d, dt, 3600 + d, 4)
    gcu = torch.from_numpy(cu).cuda()
    gq, gk, gv, gdo = (t.cuda() for t in (q, k, v, do))
    pad = 2048
    obuf = torch.full((total * H * d + pad,), 7.0, dtype=dt, device="cuda")
    o = obuf[:total * H * d].view(total, H, d)
    o, lse = fa.fwd_varlen(gq, gk, gv, gcu, max(lengths), causal=causal, dropout_p=p, seed=SEED,
                           out=o)
    dq, dk, dv = fa.bwd_varlen(gq, gk, gv, o, lse, gdo, gcu, max(lengths), causal=causal,
                               dropout_p=p, seed=SEED)
    torch.cuda.synchronize()
    assert torch.all(obuf[total * H * d:] == 7.0), "write past the packed tokens"
    for b, n in enumerate(lengths):
        if n == 0:
            continue
        s = slice(int(cu[b]), int(cu[b + 1]))
        for h in range(H):
            check_head(q[s, h], k[s, h], v[s, h], o[s, h], lse[h, s], causal, p, b, h, dt,
                       do[s, h], (dq[s, h], dk[s, h], dv[s, h]),
                       tag=f"varlen d={d} causal={causal} len={n}")


def test_varlen_equals_padded_batch():
    """Equal-length packed sequences give the bits of the [B, H, N, d] call."""
    B, H, N, d = 3, 2, 200, 64
    q, k, v = (t.cuda() for t in normal_tensors((B, H, N, d), 3700, 3, torch.bfloat16))
    o, lse = fa.fwd_ex(q, k, v, causal=True, dropout_p=0.1, seed=SEED)
    pk = [t.transpose(1, 2).reshape(B * N, H, d) for t in (q, k, v)]
    cu = torch.arange(0, (B + 1) * N, N, dtype=torch.int32, device="cuda")
    o2, l2 = fa.fwd_varlen(*pk, cu, N, causal=True, dropout_p=0.1, seed=SEED)
    assert torch.equal(o2.view(B, N, H, d).transpose(1, 2), o)
    assert torch.equal(l2.view(H, B, N).transpose(0, 1), lse)


def test_varlen_clamps_oversized_offsets():
    """Offsets past total_tokens are clamped on the device: no access outside the
    packed tensors, sequences cut at the end."""
    H, d = 1, 64
    cu_np = np.array([0, 100, 5000], dtype=np.int32)    # second sequence runs past total
    total = 160
    q, k, v = normal_tensors((total, H, d), 3800, 3, torch.bfloat16)
    gq, gk, gv = (t.cuda() for t in (q, k, v))
    o, lse = fa.fwd_varlen(gq, gk, gv, torch.from_numpy(cu_np).cuda(), 256, causal=True)
    torch.cuda.synchronize()
    s = slice(100, 160)
    check_head(q[s, 0], k[s, 0], v[s, 0], o[s, 0], lse[0, s], True, 0.0, 1, 0, torch.bfloat16,
               tag="varlen clamped offsets")


# ------------------------------------------------------ full-size workloads

from exact_io_aware_53_amd.inputs import COVERAGE_WORKLOADS, make_coverage_inputs  # noqa: E402


@pytest.mark.parametrize("name", list(COVERAGE_WORKLOADS))
def test_coverage_workload_sampled_head(name):
    """The coverage workloads as bench.py runs them; one seeded head (and, for
    the packed batch, one seeded sequence) against the oracle's forward and
    backward."""
    w = COVERAGE_WORKLOADS[name]
    t = make_coverage_inputs(w)
    g = {n: x.cuda() for n, x in t.items()}
    rng = np.random.Generator(np.random.PCG64(w.data_seed + 7))
    h = int(rng.integers(w.H))
    if w.layout == "varlen":
        cu = t["cu_seqlens"].numpy()
        mx = int(w.lengths().max())
        o, lse = fa.fwd_varlen(g["q"], g["k"], g["v"], g["cu_seqlens"], mx, causal=w.causal)
        grads = fa.bwd_varlen(g["q"], g["k"], g["v"], o, lse, g["do"], g["cu_seqlens"], mx,
                              causal=w.causal)
        torch.cuda.synchronize()
        b = int(rng.integers(w.B))
        s = slice(int(cu[b]), int(cu[b + 1]))
        args = [t[n][s, h] for n in ("q", "k", "v")]
        res = (o[s, h], lse[h, s])
        gr = tuple(x[s, h] for x in grads)
        dout = t["do"][s, h]
    else:
        view = (lambda x: x.transpose(1, 2)) if w.layout == "bshd" else (lambda x: x)
        q, k, v, do = (view(g[n]) for n in ("q", "k", "v", "do"))
        o, lse = fa.fwd_ex(q, k, v, causal=w.causal)
        grads = fa.bwd_ex(q, k, v, o, lse, do, causal=w.causal)
        torch.cuda.synchronize()
        b = int(rng.integers(w.B))
        args = [view(t[n])[b, h] for n in ("q", "k", "v")]
        res = (o[b, h], lse[b, h])
        gr = tuple(x[b, h] for x in grads)
        dout = view(t["do"])[b, h]
    check_head(*args, *res, w.causal, 0.0, b, h, w.torch_dtype, dout, gr, tag=f"coverage workload {name}")
