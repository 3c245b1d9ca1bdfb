"""GPU parity: the HIP kernels (through the C ABI) against the fp64 CPU oracle.

Bars: fp32 tensors max |err| <= 1e-5 (O, LSE and gradients); bf16 tensors
O <= 1e-2 (plus half a storage ulp only where |O_ref| >= 4, see
parity_checks), LSE <= 1e-3, gradients max|g - g_ref| / max|g_ref| <= 2e-2;
dropout masks bit-exact. Small shapes are checked on every row of every
head; the full-size workloads on seeded heads and rows (full rows always).

A gradient whose reference is zero by the mathematics (one visible key, or a
dropped single key) has no "max": fp64 leaves it as rounding noise of order
1e-17. Such a reference (max below 1e-9 of the head's largest reference
gradient) is measured relative to that largest gradient, or absolutely if
all three are zero.
"""
import math

import numpy as np
import pytest
import torch

import exact_io_aware_53_amd as fa
import oracle
from exact_io_aware_53_amd.inputs import (WORKLOADS, make_inputs, normal_tensors, sample_heads,
                                          sample_rows, to_f64)
from parity_checks import Stats, p_rounding_bound

pytestmark = pytest.mark.gpu

TOL = {"bf16": dict(o=1e-2, lse=1e-3, grad=2e-2), "f32": dict(o=1e-5, lse=1e-5, grad=1e-5)}
DTYPES = {"bf16": torch.bfloat16, "f32": torch.float32}
SEED = 0x0123456789ABCDEF


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.lib()   # fails loudly when the library is missing


def upload(ts):
    return [t.to("cuda") for t in ts]


def check_forward_heads(q, k, v, o, lse, causal, p, seed, tol, heads, rows=None, tag="",
                        wide_scores=False):
    """Compare O and LSE of the given heads (all rows, or `rows`) with the oracle.
    wide_scores: the Q x16 stress inputs, where an element that misses the bar must
    lie within the bf16 P~ rounding bound (parity_checks)."""
    d = q.shape[-1]
    scale = 1.0 / math.sqrt(d)
    o_c, lse_c = o.float().cpu(), lse.cpu()
    st = Stats(o.dtype)
    for (b, h) in heads:
        qh, kh, vh = to_f64(q[b, h]), to_f64(k[b, h]), to_f64(v[b, h])
        ro, rl = oracle.forward(qh, kh, vh, scale, causal, p, seed, b, h, rows=rows)
        go = o_c[b, h].double().numpy()
        gl = lse_c[b, h].double().numpy()
        if rows is not None:
            go, gl = go[rows], gl[rows]
        pr = (p_rounding_bound(qh, kh, vh, ro, rl, scale, causal, p, seed, b, h, rows)
              if wide_scores else None)
        st.add(go, ro, gl, rl, p_round=pr)
    st.check(tag or f"{tuple(q.shape)} causal={causal} p={p}")
    return st.err_o, st.err_lse


def rel_to_max(g, ref, fallback=None):
    """max|g - ref| / max|ref|. A reference that the mathematics makes zero (one
    visible key: dS, hence dQ and dK, vanish) leaves fp64 as rounding noise;
    below 1e-9 of `fallback` (the head's largest reference gradient) the error
    is taken relative to `fallback`, and absolutely if that is zero as well."""
    denom = np.abs(ref).max()
    if fallback and denom < 1e-9 * fallback:
        denom = fallback
    if denom == 0.0:
        denom = 1.0
    return float(np.abs(g - ref).max() / denom)


def abs_err(g, ref):
    return float(np.abs(g - ref).max())


# The last two shapes have B*H = 8 and 32: workgroups are then dealt to XCDs by
# head, one head at a time and four heads at a time respectively.
SMALL = [(1, 2, 1, 64), (1, 2, 17, 64), (2, 1, 127, 128), (1, 1, 128, 64), (1, 2, 129, 128),
         (1, 1, 1000, 64), (2, 2, 300, 128), (1, 1, 64, 128), (3, 1, 257, 64),
         (1, 8, 300, 64), (2, 16, 520, 128)]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("p", [0.0, 0.1])
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
def test_forward_small(shape, causal, p, dtype):
    B, H, N, d = shape
    seed_data = 17 + N + 7 * d + B
    q, k, v = normal_tensors(shape, seed_data, 3, DTYPES[dtype])
    gq, gk, gv = upload((q, k, v))
    o, lse = fa.fwd(gq, gk, gv, causal=causal, dropout_p=p, seed=SEED)
    torch.cuda.synchronize()
    heads = [(b, h) for b in range(B) for h in range(H)]
    check_forward_heads(q, k, v, o, lse, causal, p, SEED, TOL[dtype], heads,
                        tag=f"forward {shape} {dtype} causal={causal} p={p}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("p", [0.0, 0.1])
@pytest.mark.parametrize("shape", [(1, 2, 17, 64), (2, 1, 129, 128), (1, 1, 256, 64),
                                   (1, 2, 300, 128), (1, 1, 1, 64)],
                         ids=lambda s: "x".join(map(str, s)))
def test_backward_small(shape, causal, p, dtype):
    B, H, N, d = shape
    q, k, v, do = normal_tensors(shape, 911 + N + d, 4, DTYPES[dtype])
    gq, gk, gv, gdo = upload((q, k, v, do))
    o, lse = fa.fwd(gq, gk, gv, causal=causal, dropout_p=p, seed=SEED)
    dq, dk, dv = fa.bwd(gq, gk, gv, o, lse, gdo, causal=causal, dropout_p=p, seed=SEED)
    torch.cuda.synchronize()
    scale = 1.0 / math.sqrt(d)
    worst = 0.0
    for b in range(B):
        for h in range(H):
            rq, rk, rv, _ = oracle.backward(to_f64(q[b, h]), to_f64(k[b, h]), to_f64(v[b, h]),
                                            to_f64(do[b, h]), scale, causal, p, SEED, b, h)
            head_max = max(np.abs(r).max() for r in (rq, rk, rv))
            for g, r in ((dq, rq), (dk, rk), (dv, rv)):
                got = g[b, h].double().cpu().numpy()
                worst = max(worst, abs_err(got, r) if dtype == "f32" else rel_to_max(got, r, head_max))
    assert worst <= TOL[dtype]["grad"], f"grad err {worst:.3e}"


# ------------------------------------------------------------ full workloads
def run_workload_forward(w):
    t = make_inputs(w)
    gq, gk, gv = upload((t["q"], t["k"], t["v"]))
    o, lse = fa.fwd(gq, gk, gv, causal=w.causal, dropout_p=w.dropout_p, seed=w.dropout_seed)
    torch.cuda.synchronize()
    return t, (gq, gk, gv), o, lse


def test_workload_f32_b1h1n128d64():
    w = WORKLOADS["fwd_f32_b1h1n128d64"]
    t, _, o, lse = run_workload_forward(w)
    check_forward_heads(t["q"], t["k"], t["v"], o, lse, w.causal, 0.0, 0, TOL["f32"], [(0, 0)],
                        tag="fwd_f32_b1h1n128d64 (all rows)")


def test_workload_causal_b4h16n2048d64():
    w = WORKLOADS["fwd_causal_bf16_b4h16n2048d64"]
    t, _, o, lse = run_workload_forward(w)
    check_forward_heads(t["q"], t["k"], t["v"], o, lse, True, 0.0, 0, TOL["bf16"],
                        sample_heads(w, 2), tag="fwd_causal_bf16_b4h16n2048d64 (2 heads, all rows)")


def test_workload_causal_q4_b2h32n8192d128():
    w = WORKLOADS["fwd_causal_q4_bf16_b2h32n8192d128"]
    t, _, o, lse = run_workload_forward(w)
    rows = sample_rows(w, 256, block_rows=(64, 128, 256))
    check_forward_heads(t["q"], t["k"], t["v"], o, lse, True, 0.0, 0, TOL["bf16"],
                        sample_heads(w, 2), rows=rows,
                        tag=f"fwd_causal_q4_bf16_b2h32n8192d128 (2 heads x {len(rows)} rows)")


def test_workload_causal_b1h16n32768d128():
    w = WORKLOADS["fwd_causal_bf16_b1h16n32768d128"]
    t, _, o, lse = run_workload_forward(w)
    rows = sample_rows(w, 64, block_rows=(64, 128, 256))
    check_forward_heads(t["q"], t["k"], t["v"], o, lse, True, 0.0, 0, TOL["bf16"],
                        sample_heads(w, 2), rows=rows,
                        tag=f"fwd_causal_bf16_b1h16n32768d128 (2 heads x {len(rows)} rows)")


def test_workload_dropout_fwd_bwd_b2h16n4096d64():
    w = WORKLOADS["fwdbwd_causal_dropout_bf16_b2h16n4096d64"]
    t = make_inputs(w)
    gq, gk, gv, gdo = upload((t["q"], t["k"], t["v"], t["do"]))
    o, lse = fa.fwd(gq, gk, gv, causal=True, dropout_p=w.dropout_p, seed=w.dropout_seed)
    dq, dk, dv = fa.bwd(gq, gk, gv, o, lse, gdo, causal=True, dropout_p=w.dropout_p,
                        seed=w.dropout_seed)
    torch.cuda.synchronize()
    (b, h), = sample_heads(w, 1)
    check_forward_heads(t["q"], t["k"], t["v"], o, lse, True, w.dropout_p, w.dropout_seed,
                        TOL["bf16"], [(b, h)], tag="fwdbwd_causal_dropout_bf16_b2h16n4096d64 (1 head)")
    rq, rk, rv, _ = oracle.backward(to_f64(t["q"][b, h]), to_f64(t["k"][b, h]),
                                    to_f64(t["v"][b, h]), to_f64(t["do"][b, h]), w.scale, True,
                                    w.dropout_p, w.dropout_seed, b, h)
    for name, g, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        e = rel_to_max(g[b, h].double().cpu().numpy(), r)
        assert e <= TOL["bf16"]["grad"], f"{name} rel-to-max err {e:.3e}"


# --------------------------------------------------------- dropout mask probes
def test_dropout_mask_bit_exact_one_head():
    w = WORKLOADS["fwdbwd_causal_dropout_bf16_b2h16n4096d64"]
    (b, h), = sample_heads(w, 1)
    m = fa.dropout_mask(w.B, w.H, w.N, b, h, w.dropout_p, w.dropout_seed).cpu().numpy()
    for i0 in range(0, w.N, 1024):
        rows = np.arange(i0, i0 + 1024)
        ref = oracle.keep_mask(b, h, rows, np.arange(w.N), w.dropout_p, w.dropout_seed)
        assert np.array_equal(m[rows].astype(bool), ref)


def test_dropout_mask_through_forward_kernel():
    """V = one-hot columns makes O[i, c] = P_{i j_c} Z_{i j_c} / (1-p): the forward kernel's
    mask for 64 keys per launch, compared bit-exactly with the oracle's."""
    B, H, N, d, p = 1, 2, 512, 64, 0.1
    q, k = normal_tensors((B, H, N, d), 5150, 2, torch.bfloat16)
    gq, gk = upload((q, k))
    for j0 in (0, 200, 448):
        v = torch.zeros((B, H, N, d), dtype=torch.bfloat16)
        cols = np.arange(j0, j0 + d)
        v[:, :, torch.as_tensor(cols), torch.arange(d)] = 1.0
        o, _ = fa.fwd(gq, gk, v.cuda(), causal=False, dropout_p=p, seed=SEED)
        got = (o.float().cpu().numpy() != 0)
        for h in range(H):
            ref = oracle.keep_mask(0, h, np.arange(N), cols, p, SEED)
            assert np.array_equal(got[0, h], ref), (j0, h)


def test_dropout_mask_through_backward_kernel():
    """dO rows i_c = e_c give dV_j[c] = P_{i_c j} Z_{i_c j} / (1-p): 64 mask rows per launch."""
    B, H, N, d, p = 1, 1, 384, 64, 0.1
    q, k, v = normal_tensors((B, H, N, d), 6160, 3, torch.bfloat16)
    gq, gk, gv = upload((q, k, v))
    o, lse = fa.fwd(gq, gk, gv, causal=False, dropout_p=p, seed=SEED)
    for i0 in (0, 130, 320):
        do = torch.zeros((B, H, N, d), dtype=torch.bfloat16)
        rows = np.arange(i0, i0 + d)
        do[:, :, torch.as_tensor(rows), torch.arange(d)] = 1.0
        _, _, dv = fa.bwd(gq, gk, gv, o, lse, do.cuda(), causal=False, dropout_p=p, seed=SEED)
        got = (dv.float().cpu().numpy()[0, 0] != 0).T        # [c, j]
        ref = oracle.keep_mask(0, 0, rows, np.arange(N), p, SEED)
        assert np.array_equal(got, ref), i0


# Probes on the kernel instances of the dropout workload itself (B2 H16 N4096
# d64, causal, p = 0.1): its grid takes the 8-wave causal dropout forward, the
# causal key-side backward with fused dQ atomics and, in the two-pass form, the
# chunked d = 64 key side and the query-side dQ pass. Each probe reads the mask
# out of a product whose element is a nonzero multiple of Z_ij, so any wrong
# counter shows as a mismatch with the oracle's mask; causal entries j > i must
# come out zero.
C4 = "fwdbwd_causal_dropout_bf16_b2h16n4096d64"
PROBE_HEADS = [(0, 0), (1, 15)]
PROBE_WINDOWS = (0, 1990, 4032)


def causal_keep(b, h, rows, cols, w):
    keep = oracle.keep_mask(b, h, rows, cols, w.dropout_p, w.dropout_seed)
    return keep & (np.asarray(cols)[None, :] <= np.asarray(rows)[:, None])


def test_dropout_mask_through_causal_forward_workload_kernel():
    """V = one-hot columns (V[j_c, c] = 1): O[i, c] = P_{i j_c} Z_{i j_c} / (1-p)."""
    w = WORKLOADS[C4]
    t = make_inputs(w)
    gq, gk = upload((t["q"], t["k"]))
    rows = np.arange(w.N)
    for j0 in PROBE_WINDOWS:
        cols = np.arange(j0, j0 + w.d)
        v = torch.zeros((w.B, w.H, w.N, w.d), dtype=torch.bfloat16)
        v[:, :, torch.as_tensor(cols), torch.arange(w.d)] = 1.0
        o, _ = fa.fwd(gq, gk, v.cuda(), causal=True, dropout_p=w.dropout_p, seed=w.dropout_seed)
        got = o.float().cpu().numpy() != 0
        for (b, h) in PROBE_HEADS:
            assert np.array_equal(got[b, h], causal_keep(b, h, rows, cols, w)), (j0, b, h)


@pytest.mark.parametrize("deterministic", [False, True], ids=["fused", "two_pass"])
def test_dropout_mask_through_causal_backward_dv(deterministic):
    """dO rows i_c = e_c: dV_j[c] = P_{i_c j} Z_{i_c j} / (1-p), 64 mask rows per launch,
    through the key-side kernel (fused dQ atomics, or the two-pass key side)."""
    w = WORKLOADS[C4]
    t = make_inputs(w)
    gq, gk, gv = upload((t["q"], t["k"], t["v"]))
    _, lse = fa.fwd(gq, gk, gv, causal=True)
    o = torch.zeros_like(gq)
    cols = np.arange(w.N)
    for i0 in PROBE_WINDOWS:
        rows = np.arange(i0, i0 + w.d)
        do = torch.zeros((w.B, w.H, w.N, w.d), dtype=torch.bfloat16)
        do[:, :, torch.as_tensor(rows), torch.arange(w.d)] = 1.0
        _, _, dv = fa.bwd(gq, gk, gv, o, lse, do.cuda(), causal=True, dropout_p=w.dropout_p,
                          seed=w.dropout_seed, deterministic=deterministic)
        got = dv.float().cpu().numpy() != 0
        for (b, h) in PROBE_HEADS:
            assert np.array_equal(got[b, h].T, causal_keep(b, h, rows, cols, w)), (i0, b, h)


@pytest.mark.parametrize("deterministic", [False, True], ids=["fused", "two_pass"])
def test_dropout_mask_through_causal_backward_dq(deterministic):
    """K and V one-hot on 64 keys j_c (K[j_c] = V[j_c] = e_c, every other row 0), dO all
    ones, and O = 0 given to the backward, so D = 0 and dS_ij = P_ij Z_ij / (1-p) on the
    probed keys and 0 elsewhere: dQ_i[c] = scale P_{i j_c} Z_{i j_c} / (1-p). That is the
    fused kernel's dQ atomics, or the two-pass form's query-side pass."""
    w = WORKLOADS[C4]
    t = make_inputs(w)
    gq = t["q"].cuda()
    rows = np.arange(w.N)
    do = torch.ones((w.B, w.H, w.N, w.d), dtype=torch.bfloat16, device="cuda")
    for j0 in PROBE_WINDOWS:
        cols = np.arange(j0, j0 + w.d)
        kv = torch.zeros((w.B, w.H, w.N, w.d), dtype=torch.bfloat16)
        kv[:, :, torch.as_tensor(cols), torch.arange(w.d)] = 1.0
        kv = kv.cuda()
        _, lse = fa.fwd(gq, kv, kv, causal=True)
        o = torch.zeros_like(gq)
        dq, _, _ = fa.bwd(gq, kv, kv, o, lse, do, causal=True, dropout_p=w.dropout_p,
                          seed=w.dropout_seed, deterministic=deterministic)
        got = dq.float().cpu().numpy() != 0
        for (b, h) in PROBE_HEADS:
            assert np.array_equal(got[b, h], causal_keep(b, h, rows, cols, w)), (j0, b, h)


@pytest.mark.parametrize("deterministic", [False, True], ids=["fused", "two_pass"])
def test_dropout_mask_through_d128_backward(deterministic):
    """d = 128, causal, p = 0.1: in the two-pass form the key side is split over two
    waves per SIMD, one applying Z to P for dV, the other reading Z back from the sign
    of the P it receives for dS. dO rows i_c = e_c give dV_j[c] = P_{i_c j} Z'_{i_c j}
    (the first wave's mask); Q rows i_c = e_c with every other Q row 0, V and dO all
    ones and O = 0 (so D = 0 and dP = d) give dK_j[c] = scale d P_{i_c j} Z'_{i_c j}
    (the second wave's)."""
    B, H, N, d, p = 1, 2, 512, 128, 0.1
    q, k, v = normal_tensors((B, H, N, d), 6262, 3, torch.bfloat16)
    gk = k.cuda()
    cols = np.arange(N)
    for i0 in (0, 200, 384):
        rows = np.arange(i0, i0 + d)
        ref = [oracle.keep_mask(0, h, rows, cols, p, SEED) & (cols[None, :] <= rows[:, None]) for h in range(H)]
        # dV: the P side
        gq, gv = q.cuda(), v.cuda()
        _, lse = fa.fwd(gq, gk, gv, causal=True)
        do = torch.zeros((B, H, N, d), dtype=torch.bfloat16)
        do[:, :, torch.as_tensor(rows), torch.arange(d)] = 1.0
        _, _, dv = fa.bwd(gq, gk, gv, torch.zeros_like(gq), lse, do.cuda(), causal=True, dropout_p=p,
                          seed=SEED, deterministic=deterministic)
        got = dv.float().cpu().numpy() != 0
        for h in range(H):
            assert np.array_equal(got[0, h].T, ref[h]), ("dV", i0, h)
        # dK: the dS side
        q1 = torch.zeros((B, H, N, d), dtype=torch.bfloat16)
        q1[:, :, torch.as_tensor(rows), torch.arange(d)] = 1.0
        gq1 = q1.cuda()
        ones = torch.ones((B, H, N, d), dtype=torch.bfloat16, device="cuda")
        _, lse1 = fa.fwd(gq1, gk, ones, causal=True)
        _, dk, _ = fa.bwd(gq1, gk, ones, torch.zeros_like(gq1), lse1, ones, causal=True, dropout_p=p,
                          seed=SEED, deterministic=deterministic)
        got = dk.float().cpu().numpy() != 0
        for h in range(H):
            assert np.array_equal(got[0, h].T, ref[h]), ("dK", i0, h)


# ------------------------------------------------------------ other properties
def test_forward_is_deterministic():
    shape = (2, 4, 1000, 128)
    q, k, v = upload(normal_tensors(shape, 7007, 3, torch.bfloat16))
    outs = [fa.fwd(q, k, v, causal=True, dropout_p=0.1, seed=SEED) for _ in range(3)]
    for o, l in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(l, outs[0][1])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_outputs_stay_in_bounds(dtype):
    """Canary words around every output buffer are untouched."""
    B, H, N, d = 1, 3, 333, 64
    dt = DTYPES[dtype]
    q, k, v, do = upload(normal_tensors((B, H, N, d), 8118, 4, dt))
    n = B * H * N * d
    pad = 4096

    def guarded(count, tdt):
        buf = torch.full((count + 2 * pad,), 7.0, dtype=tdt, device="cuda")
        return buf, buf[pad:pad + count]

    ob, o = guarded(n, dt)
    lb, lse = guarded(B * H * N, torch.float32)
    fa.fwd(q, k, v, causal=True, dropout_p=0.1, seed=SEED, out=o.view(B, H, N, d),
           lse=lse.view(B, H, N))
    grads = [guarded(n, dt) for _ in range(3)]
    fa.bwd(q, k, v, o.view(B, H, N, d), lse.view(B, H, N), do, causal=True, dropout_p=0.1,
           seed=SEED, dq=grads[0][1].view(B, H, N, d), dk=grads[1][1].view(B, H, N, d),
           dv=grads[2][1].view(B, H, N, d))
    torch.cuda.synchronize()
    for buf, _ in [(ob, o), (lb, lse)] + grads:
        assert torch.all(buf[:pad] == 7.0) and torch.all(buf[-pad:] == 7.0)


def test_uniform_scores_and_causal_row0_on_gpu():
    """Closed forms through the kernels: Q = 0 gives O_i = mean of visible V rows and
    LSE_i = ln(i+1) (causal); causal row 0 returns V_0 exactly."""
    B, H, N, d = 1, 1, 300, 128
    k, v = normal_tensors((B, H, N, d), 9119, 2, torch.bfloat16)
    q = torch.zeros_like(k)
    o, lse = fa.fwd(*upload((q, k, v)), causal=True)
    vv = to_f64(v[0, 0])
    mean = np.cumsum(vv, axis=0) / np.arange(1, N + 1)[:, None]
    assert np.abs(o[0, 0].double().cpu().numpy() - mean).max() <= 1e-2
    assert np.abs(lse[0, 0].double().cpu().numpy() - np.log(np.arange(1, N + 1))).max() <= 1e-3
    q2 = normal_tensors((B, H, N, d), 9120, 1, torch.bfloat16)[0]
    o2, _ = fa.fwd(*upload((q2, k, v)), causal=True)
    assert torch.equal(o2[0, 0, 0].cpu(), v[0, 0, 0])


@pytest.mark.parametrize("p", [0.0, 0.1])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_forward_wide_score_range(d, causal, p):
    """Q scaled by 16 (exact in bf16): scores spread over tens of log2 units, so a
    row's maximum jumps between key tiles, weights taken against the reference
    maximum of earlier tiles overflow fp32, and the forward's rescale path runs on
    most rows of most tiles. O and LSE still match the oracle on every row."""
    B, H, N = 1, 2, 700
    q, k, v = normal_tensors((B, H, N, d), 7331 + d, 3, torch.bfloat16)
    q = (q.float() * 16.0).to(torch.bfloat16)
    o, lse = fa.fwd(*upload((q, k, v)), causal=causal, dropout_p=p, seed=SEED)
    torch.cuda.synchronize()
    check_forward_heads(q, k, v, o, lse, causal, p, SEED, TOL["bf16"], [(0, 0), (0, 1)],
                        tag=f"wide scores (Q x16) d={d} causal={causal} p={p}", wide_scores=True)


# d = 64 grids of at least 512 workgroups (two per CU) run the forward with
# 64-key tiles and two workgroups per CU; smaller grids keep 128-key tiles.
# B*H = 64 heads; 256 query rows per workgroup, causal grids pair two blocks.
TWO_PER_CU = [(1, 64, 2048, 64, False, 1.0), (1, 64, 1999, 64, False, 16.0),
              (1, 64, 4096, 64, True, 1.0), (1, 64, 3969, 64, True, 16.0)]


@pytest.mark.parametrize("case", TWO_PER_CU, ids=lambda c: "x".join(map(str, c[:4])) + f"-causal{int(c[4])}-q{c[5]:g}")
def test_forward_d64_two_workgroups_per_cu(case):
    """The 64-key-tile forward against the oracle, on sampled heads spread over
    the XCD groups, with a ragged tail and (Q x 16) the rescale path."""
    B, H, N, d, causal, qmul = case
    q, k, v = normal_tensors((B, H, N, d), 4100 + N, 3, torch.bfloat16)
    q = (q.float() * qmul).to(torch.bfloat16)
    o, lse = fa.fwd(*upload((q, k, v)), causal=causal, dropout_p=0.0, seed=SEED)
    torch.cuda.synchronize()
    check_forward_heads(q, k, v, o, lse, causal, 0.0, SEED, TOL["bf16"], [(0, 0), (0, 9), (0, 38), (0, 63)],
                        tag=f"64-key forward {case}", wide_scores=qmul > 4.0)


# A grid that fits 256 workgroups of 128 query rows (one per CU) runs the
# forward with 4-wave workgroups: the small shapes above all take that path.
# These shapes give more workgroups than that, so they run the 8-wave kernel
# (256 rows per workgroup) on ragged tails, with and without dropout.
EIGHT_WAVE = [(1, 160, 300, 128), (2, 80, 257, 64), (1, 160, 300, 64)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("p", [0.0, 0.1])
@pytest.mark.parametrize("shape", EIGHT_WAVE, ids=lambda s: "x".join(map(str, s)))
def test_forward_eight_wave_grids(shape, causal, p):
    B, H, N, d = shape
    q, k, v = normal_tensors(shape, 5200 + N + d, 3, torch.bfloat16)
    o, lse = fa.fwd(*upload((q, k, v)), causal=causal, dropout_p=p, seed=SEED)
    torch.cuda.synchronize()
    heads = [(0, 0), (0, 1), (0, 37), (B - 1, H - 2), (B - 1, H - 1)]
    check_forward_heads(q, k, v, o, lse, causal, p, SEED, TOL["bf16"], heads,
                        tag=f"8-wave forward {shape} causal={causal} p={p}")


# d = 128 without dropout on the 8-wave grid runs the two-group forward (waves
# 0-3 and 4-7 alternate products and softmax half steps). B*H = 80 heads of
# N = 1000 give 160 causal workgroups (more than the 4-wave grid can fit in
# one round), four 128-key tiles per 256-row block, a ragged last tile and
# causal block pairs of unequal length; Q x 16 drives the rescale path.
TWO_GROUP = [(1, 80, 1000, 128, True, 1.0), (1, 80, 1000, 128, False, 1.0),
             (1, 80, 1000, 128, True, 16.0), (2, 40, 777, 128, False, 16.0)]


@pytest.mark.parametrize("case", TWO_GROUP, ids=lambda c: "x".join(map(str, c[:4])) + f"-causal{int(c[4])}-q{c[5]:g}")
def test_forward_two_group_kernel(case):
    B, H, N, d, causal, qmul = case
    q, k, v = normal_tensors((B, H, N, d), 6100 + N + int(qmul), 3, torch.bfloat16)
    q = (q.float() * qmul).to(torch.bfloat16)
    o, lse = fa.fwd(*upload((q, k, v)), causal=causal, dropout_p=0.0, seed=SEED)
    torch.cuda.synchronize()
    heads = [(0, 0), (0, 7), (0, 38), (B - 1, H - 1)]
    check_forward_heads(q, k, v, o, lse, causal, 0.0, SEED, TOL["bf16"], heads,
                        tag=f"two-group forward {case}", wide_scores=qmul > 1.0)


# Very short sequences over many heads still take the 8-wave grid (640 heads,
# so the 4-wave grid would not fit one round): one key tile, most waves own
# only rows past N and skip every tile.
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 33])
def test_two_group_forward_short_sequences(N, causal):
    B, H, d = 1, 640, 128
    q, k, v = normal_tensors((B, H, N, d), 6300 + N, 3, torch.bfloat16)
    o, lse = fa.fwd(*upload((q, k, v)), causal=causal, dropout_p=0.0, seed=SEED)
    torch.cuda.synchronize()
    check_forward_heads(q, k, v, o, lse, causal, 0.0, SEED, TOL["bf16"], [(0, 0), (0, 255), (0, 639)],
                        tag=f"two-group forward short N={N} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("qmul", [1.0, 16.0])
def test_two_group_forward_bitwise_equal_to_one_group(causal, qmul):
    """Each row's arithmetic is the same in both forward kernels, so two heads
    computed in an 80-head grid (the two-group kernel) and on their own (a grid
    small enough for the 4-wave one-group kernel) give the same bits."""
    B, H, N, d = 1, 80, 1000, 128
    q, k, v = normal_tensors((B, H, N, d), 6200 + int(qmul), 3, torch.bfloat16)
    q = (q.float() * qmul).to(torch.bfloat16)
    o, lse = fa.fwd(*upload((q, k, v)), causal=causal, dropout_p=0.0, seed=SEED)
    heads = [3, 41]
    sub = [t[:, heads].contiguous() for t in (q, k, v)]
    o2, lse2 = fa.fwd(*upload(sub), causal=causal, dropout_p=0.0, seed=SEED)
    torch.cuda.synchronize()
    assert torch.equal(o[:, heads].cpu(), o2.cpu())
    assert torch.equal(lse[:, heads].cpu(), lse2.cpu())


def test_forward_four_wave_grid_at_the_limit():
    """B1 H16 N4096 d128 causal: 16 heads x 16 pairs of 128-row blocks = 256
    workgroups, the largest grid that takes the 4-wave kernel."""
    B, H, N, d = 1, 16, 4096, 128
    q, k, v = normal_tensors((B, H, N, d), 5301, 3, torch.bfloat16)
    o, lse = fa.fwd(*upload((q, k, v)), causal=True, dropout_p=0.0, seed=SEED)
    torch.cuda.synchronize()
    check_forward_heads(q, k, v, o, lse, True, 0.0, SEED, TOL["bf16"], [(0, 0), (0, 15)], tag="b1h16n4096d128")


def test_forward_takes_no_device_memory_and_inputs_grow_linearly():
    """The forward needs no workspace: with outputs preallocated, free device
    memory is the same before and after a call at every N; the tensors a call
    touches grow linearly in N (no N x N buffer exists anywhere)."""
    B, H, d = 1, 4, 128
    sizes = []
    for N in (1024, 4096, 16384):
        q, k, v = (t.cuda() for t in normal_tensors((B, H, N, d), 9300 + N, 3, torch.bfloat16))
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
        fa.fwd(q, k, v, causal=True, out=o, lse=lse)
        torch.cuda.synchronize()
        free0 = torch.cuda.mem_get_info()[0]
        for _ in range(3):
            fa.fwd(q, k, v, causal=True, out=o, lse=lse)
        torch.cuda.synchronize()
        assert torch.cuda.mem_get_info()[0] == free0
        sizes.append(sum(t.numel() * t.element_size() for t in (q, k, v, o, lse)))
        del q, k, v, o, lse
    assert sizes[1] == 4 * sizes[0] and sizes[2] == 4 * sizes[1]
