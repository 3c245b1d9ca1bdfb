"""Pins for the CPU oracle (no GPU). Each check ties the oracle to something other
than itself: pure-Python brute force, PyTorch's float64 attention and autograd,
closed forms, central finite differences, the tiled recurrence the pages print,
and AMD's rocRAND Philox engine. The mutation tests at the end plant plausible
mistakes in copies of the oracle's arithmetic and show that some pin fails.
"""
import math
import os
import shutil
import subprocess

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as A
from oracle import philox as PH
from oracle.recurrence import online_forward

HERE = os.path.dirname(os.path.abspath(__file__))


def randn(shape, seed, scale=1.0):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape) * scale


# ---------------------------------------------------------------- brute force
def brute_forward(q, k, v, scale, causal, keep=None, p=0.0, key_offset=0):
    """Scalar loops with math.fsum; keep[i][j] is the dropout keep mask; causal query i
    sits at key position key_offset + i."""
    q, k, v = q.tolist(), k.tolist(), v.tolist()
    n, d = len(k), len(k[0])
    outs, lses = [], []
    for i in range(len(q)):
        js = [j for j in range(n) if (not causal or j <= key_offset + i)]
        s = [scale * math.fsum(q[i][t] * k[j][t] for t in range(d)) for j in js]
        m = max(s)
        l = math.fsum(math.exp(x - m) for x in s)
        lse = m + math.log(l)
        w = [math.exp(x - lse) for x in s]
        if keep is not None:
            w = [wj * (1.0 if keep[i][j] else 0.0) / (1.0 - p) for wj, j in zip(w, js)]
        outs.append([math.fsum(wj * v[j][c] for wj, j in zip(w, js)) for c in range(len(v[0]))])
        lses.append(lse)
    return np.array(outs), np.array(lses)


def pin_bruteforce(fwd):
    err = 0.0
    for (n, d, causal, p, seed) in [(1, 1, False, 0.0, 1), (5, 3, False, 0.0, 2), (7, 4, True, 0.0, 3),
                                    (8, 2, True, 0.5, 4), (6, 4, False, 0.25, 5), (8, 4, True, 0.0, 6)]:
        q, k, v = randn((n, d), seed), randn((n, d), seed + 100), randn((n, d), seed + 200)
        s = 1 / math.sqrt(d)
        keep = PH.keep_mask(0, 1, np.arange(n), np.arange(n), p, 99 + seed) if p else None
        o_ref, l_ref = brute_forward(q, k, v, s, causal, keep, float(np.float32(p)))
        o, l = fwd(q, k, v, s, causal, dropout_p=p, seed=99 + seed, b=0, h=1)
        err = max(err, np.abs(o - o_ref).max(), np.abs(l - l_ref).max())
    return err


def pin_sdpa(fwd):
    """Against torch.nn.functional.scaled_dot_product_attention in float64 (dropout 0)."""
    err = 0.0
    for (n, d, causal, seed) in [(1, 4, True, 10), (33, 16, False, 11), (64, 8, True, 12), (50, 32, True, 13)]:
        q, k, v = randn((n, d), seed, 2.0), randn((n, d), seed + 1), randn((n, d), seed + 2)
        s = 1 / math.sqrt(d)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
            is_causal=causal, scale=s)[0].numpy()
        o, _ = fwd(q, k, v, s, causal)
        err = max(err, np.abs(o - ref).max())
    return err


def pin_closed_forms(fwd):
    """Worst deviation from closed-form results (uniform scores, one key, causal row 0, shifts)."""
    errs = []
    n, d = 40, 8
    s = 1 / math.sqrt(d)
    v = randn((n, d), 21)
    k = randn((n, d), 22)
    # Uniform scores (Q = 0): O_i = mean of the visible V rows, LSE_i = ln(count).
    for causal in (False, True):
        o, l = fwd(np.zeros((n, d)), k, v, s, causal)
        cnt = np.arange(1, n + 1) if causal else np.full(n, n)
        mean = np.cumsum(v, axis=0) / cnt[:, None] if causal else np.broadcast_to(v.mean(0), v.shape)
        errs += [np.abs(o - mean).max(), np.abs(l - np.log(cnt)).max()]
    # One key: O = V, LSE = s q.k.
    q1, k1, v1 = randn((1, d), 23), randn((1, d), 24), randn((1, d), 25)
    o, l = fwd(q1, k1, v1, s, False)
    errs += [np.abs(o - v1).max(), abs(l[0] - s * float(q1[0] @ k1[0]))]
    # Causal row 0 sees only key 0.
    q = randn((n, d), 26)
    o, l = fwd(q, k, v, s, True)
    errs += [np.abs(o[0] - v[0]).max(), abs(l[0] - s * float(q[0] @ k[0]))]
    # Shift invariance: K_j + w for all j leaves O unchanged and adds s q_i.w to LSE;
    # |w| puts raw scores near 1e3, which would overflow a softmax without the max shift.
    w = randn((d,), 27)
    w *= 1.0e3 / np.abs(q @ w).max() / s
    o0, l0 = fwd(q, k, v, s, False)
    o1, l1 = fwd(q, k + w, v, s, False)
    errs += [np.abs(o1 - o0).max(), np.abs((l1 - l0) - s * (q @ w)).max() / 1e3]
    return max(float(e) for e in errs)


def loss_and_grads_fd(q, k, v, do, s, causal, p, seed, h=1e-6):
    """Central finite differences of L = sum(dO * O) with the dropout mask held fixed."""
    def loss(qq, kk, vv):
        o, _ = A.forward(qq, kk, vv, s, causal, p, seed, 0, 0)
        return float((do * o).sum())
    grads = []
    for which in range(3):
        base = [q.copy(), k.copy(), v.copy()]
        g = np.zeros_like(base[which])
        for idx in np.ndindex(g.shape):
            plus = [x.copy() for x in base]
            minus = [x.copy() for x in base]
            plus[which][idx] += h
            minus[which][idx] -= h
            g[idx] = (loss(*plus) - loss(*minus)) / (2 * h)
        grads.append(g)
    return grads


def pin_finite_differences(bwd):
    worst = 0.0
    for (n, d, causal, p, seed) in [(5, 3, False, 0.0, 31), (6, 4, True, 0.0, 32), (6, 4, True, 0.3, 33),
                                    (4, 2, False, 0.5, 34)]:
        q, k, v, do = (randn((n, d), seed + 10 * t) for t in range(4))
        s = 1 / math.sqrt(d)
        fd = loss_and_grads_fd(q, k, v, do, s, causal, p, 7 + seed)
        an = bwd(q, k, v, do, s, causal, p, 7 + seed, 0, 0)[:3]
        for g_fd, g_an in zip(fd, an):
            worst = max(worst, np.abs(g_fd - g_an).max() / max(np.abs(g_fd).max(), 1e-3))
    return worst


def pin_autograd(bwd):
    worst = 0.0
    for (n, d, causal, seed) in [(17, 8, False, 41), (32, 16, True, 42)]:
        q, k, v, do = (randn((n, d), seed + 10 * t) for t in range(4))
        s = 1 / math.sqrt(d)
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        out = torch.nn.functional.scaled_dot_product_attention(tq[None], tk[None], tv[None],
                                                               is_causal=causal, scale=s)[0]
        out.backward(torch.from_numpy(do))
        an = bwd(q, k, v, do, s, causal, 0.0, 0, 0, 0)[:3]
        for t, g in zip((tq, tk, tv), an):
            worst = max(worst, np.abs(t.grad.numpy() - g).max())
    return worst


# ------------------------------------------------------------------ the pins
def test_forward_matches_bruteforce():
    assert pin_bruteforce(A.forward) <= 1e-13


def test_forward_matches_torch_sdpa_float64():
    assert pin_sdpa(A.forward) <= 1e-12


def _maxdiff(a, b):
    """Largest absolute difference; a NaN anywhere counts as an infinite error."""
    d = np.abs(np.asarray(a, dtype=np.float64) - np.asarray(b, dtype=np.float64))
    return float("inf") if np.isnan(d).any() else float(d.max())


def pin_key_offset(fwd):
    """Query blocks placed at an offset in a longer key sequence (decode shape):
    brute force, torch SDPA on the visible keys of each row, and agreement with the
    same-sequence causal rows that the offset stands for."""
    err = 0.0
    for (nq, nk, d, causal, seed) in [(1, 9, 4, True, 40), (3, 11, 2, True, 41), (4, 4, 3, True, 42),
                                      (2, 7, 4, False, 43), (5, 12, 3, True, 44)]:
        q, k, v = randn((nq, d), seed, 2.0), randn((nk, d), seed + 1), randn((nk, d), seed + 2)
        s = 1 / math.sqrt(d)
        off = nk - nq
        o, l = fwd(q, k, v, s, causal, key_offset=off)
        o_ref, l_ref = brute_forward(q, k, v, s, causal, key_offset=off)
        err = max(err, _maxdiff(o, o_ref), _maxdiff(l, l_ref))
        for i in range(nq):
            vis = off + i + 1 if causal else nk
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(q[i:i + 1])[None], torch.from_numpy(k[:vis])[None],
                torch.from_numpy(v[:vis])[None], scale=s)[0].numpy()
            err = max(err, _maxdiff(o[i], ref[0]))
        # the last nq rows of a same-sequence problem
        qa = np.concatenate([randn((off, d), seed + 3), q]) if off else q
        o_rows, l_rows = fwd(qa, k, v, s, causal, rows=np.arange(off, nk))
        err = max(err, _maxdiff(o, o_rows), _maxdiff(l, l_rows))
    return err


def test_forward_key_offset():
    assert pin_key_offset(A.forward) <= 1e-12


def test_single_query_at_end_sees_every_key():
    q, k, v = randn((1, 8), 50, 2.0), randn((37, 8), 51), randn((37, 8), 52)
    o_c, l_c = A.forward(q, k, v, 0.3, True, key_offset=36)
    o_n, l_n = A.forward(q, k, v, 0.3, False)
    assert np.array_equal(o_c, o_n) and np.array_equal(l_c, l_n)


def test_forward_closed_forms():
    assert pin_closed_forms(A.forward) <= 1e-12


def test_backward_finite_differences():
    assert pin_finite_differences(A.backward) <= 1e-6


def test_backward_matches_torch_autograd_float64():
    assert pin_autograd(A.backward) <= 1e-12


def test_rows_of_p_sum_to_one():
    n = 24
    q, k = randn((n, 8), 51), randn((n, 8), 52)
    for causal in (False, True):
        o, _ = A.forward(q, k, np.eye(n), 0.35, causal)   # V = I gives O = P
        assert np.abs(o.sum(axis=1) - 1).max() <= 1e-14
        if causal:
            assert np.all(np.triu(o, 1) == 0)


def test_key_value_permutation_equivariance():
    n, d = 30, 8
    q, k, v = randn((n, d), 61), randn((n, d), 62), randn((n, d), 63)
    perm = np.random.Generator(np.random.PCG64(64)).permutation(n)
    o0, l0 = A.forward(q, k, v, 0.3, False)
    o1, l1 = A.forward(q, k[perm], v[perm], 0.3, False)
    assert np.abs(o0 - o1).max() <= 1e-13 and np.abs(l0 - l1).max() <= 1e-13


def test_row_subset_matches_full():
    n, d = 45, 8
    q, k, v = randn((n, d), 71), randn((n, d), 72), randn((n, d), 73)
    rows = np.array([0, 3, 17, 44])
    for causal, p in ((False, 0.0), (True, 0.0), (True, 0.2)):
        of, lf = A.forward(q, k, v, 0.3, causal, p, 5, 1, 2)
        os_, ls = A.forward(q, k, v, 0.3, causal, p, 5, 1, 2, rows=rows)
        assert np.array_equal(of[rows], os_) and np.array_equal(lf[rows], ls)


def test_causal_row0_with_dropout():
    n, d, p, seed = 16, 4, 0.5, 77
    q, k, v = randn((n, d), 81), randn((n, d), 82), randn((n, d), 83)
    o, _ = A.forward(q, k, v, 0.5, True, p, seed, 0, 3)
    z00 = PH.keep_mask(0, 3, [0], [0], p, seed)[0, 0]
    assert np.abs(o[0] - (1.0 if z00 else 0.0) * v[0] / (1 - p)).max() <= 1e-15


def test_inverted_dropout_is_unbiased():
    """E_seed[O_dropout] = O: the average over seeds converges (inverted dropout)."""
    n, d, p = 6, 3, 0.3
    q, k, v = randn((n, d), 91), randn((n, d), 92), randn((n, d), 93)
    o_ref, _ = A.forward(q, k, v, 0.5, True)
    seeds = 4000
    acc = np.zeros_like(o_ref)
    acc2 = np.zeros_like(o_ref)
    for sd in range(seeds):
        o, _ = A.forward(q, k, v, 0.5, True, p, 1000 + sd, 0, 0)
        acc += o
        acc2 += o * o
    mean = acc / seeds
    sem = np.sqrt(np.maximum(acc2 / seeds - mean ** 2, 1e-30) / seeds)
    assert np.all(np.abs(mean - o_ref) <= 5 * sem + 1e-12)


def test_backward_invariants():
    n, d = 20, 8
    q, k, v, do = (randn((n, d), 101 + t) for t in range(4))
    for causal, p in ((False, 0.0), (True, 0.0), (True, 0.25)):
        dq, dk, dv, _ = A.backward(q, k, v, do, 0.35, causal, p, 9, 1, 1)
        # Rows of dS sum to zero, so the key gradients sum to zero.
        assert np.abs(dk.sum(axis=0)).max() <= 1e-12
    # All keys equal: the scores of a row are equal, dS rows sum to 0, so dQ = 0.
    k_eq = np.broadcast_to(randn((1, d), 109), (n, d)).copy()
    dq, _, _, _ = A.backward(q, k_eq, v, do, 0.35, False, 0.0)
    assert np.abs(dq).max() <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("p", [0.0, 0.1])
@pytest.mark.parametrize("block", [1, 3, 16, 37])
def test_tiled_recurrence_equals_plain_softmax(causal, p, block):
    """The pages' online recurrence, tile by tile, reproduces the materialising oracle."""
    n, d = 37, 8
    q, k, v = randn((n, d), 111, 3.0), randn((n, d), 112), randn((n, d), 113)
    o0, l0 = A.forward(q, k, v, 0.35, causal, p, 12345, 1, 0)
    o1, l1 = online_forward(q, k, v, 0.35, causal, block, p, 12345, 1, 0)
    assert np.abs(o0 - o1).max() <= 1e-12
    assert np.abs(l0 - l1).max() <= 1e-12


# ------------------------------------------------------------------- Philox
def _rocrand_ref_binary(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available to build the rocRAND reference")
    out = str(tmp_path_factory.mktemp("rocrand") / "philox_ref")
    subprocess.run([hipcc, "-O1", os.path.join(HERE, "rocrand_philox_ref.cpp"), "-o", out],
                   check=True, capture_output=True)
    return out


@pytest.fixture(scope="module")
def rocrand_ref(tmp_path_factory):
    return _rocrand_ref_binary(tmp_path_factory)


def _rocrand_words(binary, tuples):
    text = "\n".join(" ".join(str(x) for x in t) for t in tuples) + "\n"
    res = subprocess.run([binary], input=text, capture_output=True, text=True, check=True)
    return np.array([[int(w) for w in line.split()] for line in res.stdout.strip().splitlines()],
                    dtype=np.uint64)


def test_philox_matches_rocrand_engine(rocrand_ref):
    rng = np.random.Generator(np.random.PCG64(121))
    # rocRAND takes counter words (0, 1) through a 64-bit offset of 4 * (b + 2^32 h),
    # so h stays below 2^30 here; the other words span their full 32-bit range.
    tuples = [(0, 0, 0, 0, 0), (2**64 - 1, 2**32 - 1, 2**30 - 1, 2**32 - 1, 2**32 - 1),
              (0x0123456789ABCDEF, 1, 15, 4095, 17)]
    for _ in range(500):
        b, i, j = (int(x) for x in rng.integers(0, 2**32, size=3))
        tuples.append((int(rng.integers(0, 2**63)) * 2 + int(rng.integers(0, 2)),
                       b, int(rng.integers(0, 2**30)), i, j))
    ref = _rocrand_words(rocrand_ref, tuples)
    arr = np.array(tuples, dtype=np.uint64)
    got = []
    for t in tuples:
        k0, k1 = PH.seed_to_key(t[0])
        got.append([int(w) for w in PH.philox4x32_10(t[1], t[2], t[3], t[4], k0, k1)])
    assert np.array_equal(np.array(got, dtype=np.uint64), ref)
    # Vectorised form over many counters at once agrees too.
    k0, k1 = PH.seed_to_key(tuples[2][0])
    w = PH.philox4x32_10(arr[:, 1], arr[:, 2], arr[:, 3], arr[:, 4], k0, k1)
    ref2 = _rocrand_words(rocrand_ref, [(tuples[2][0], *t[1:]) for t in tuples])
    assert np.array_equal(np.stack(w, axis=1), ref2)


def test_keep_mask_matches_rocrand_engine(rocrand_ref):
    seed, b, h, p = 0x0123456789ABCDEF, 1, 7, 0.1
    rows, cols = np.arange(40, 72), np.arange(0, 48)
    z = PH.keep_mask(b, h, rows, cols, p, seed)
    ref = _rocrand_words(rocrand_ref, [(seed, b, h, i, j) for i in rows for j in cols])
    thr = PH.dropout_threshold(p)
    assert np.array_equal(z.reshape(-1), ref[:, 0] >= thr)


def test_dropout_threshold_values():
    assert PH.dropout_threshold(0.0) == 0
    assert PH.dropout_threshold(0.5) == 2**31
    # float32(0.1) = 0.100000001490116..., times 2^32 = 429496735.6 -> 429496736
    assert PH.dropout_threshold(0.1) == 429496736
    assert PH.dropout_threshold(np.float32(0.1)) == 429496736
    with pytest.raises(ValueError):
        PH.dropout_threshold(1.0)


def test_keep_fraction_one_head():
    """Dropped fraction over the causal triangle of one 4096-row head is thr/2^32 within 5 sigma."""
    n, p = 4096, 0.1
    thr = PH.dropout_threshold(p)
    dropped, total = 0, 0
    for i0 in range(0, n, 512):
        rows = np.arange(i0, i0 + 512)
        z = PH.keep_mask(0, 0, rows, np.arange(n), p, 0x0123456789ABCDEF)
        live = np.arange(n)[None, :] <= rows[:, None]
        dropped += int((~z & live).sum())
        total += int(live.sum())
    q = thr / 2**32
    assert abs(dropped / total - q) <= 5 * math.sqrt(q * (1 - q) / total)
    assert PH.keep_mask(0, 0, np.arange(8), np.arange(8), 0.0, 1).all()


# ------------------------------------------------- planted mistakes fail a pin
def _mutant_forward(kind):
    def fwd(q, k, v, scale, causal=False, dropout_p=0.0, seed=0, b=0, h=0, rows=None, key_offset=0):
        q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
        n = k.shape[0]
        rows_ = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
        q = q[rows_]
        sc = 1.0 if kind == "no_scale" else scale
        s = sc * (q @ k.T)
        off = {"offset_ignored": 0, "offset_negated": -key_offset}.get(kind, key_offset)
        if causal:
            bad = (np.arange(n)[None, :] < rows_[:, None] + off) if kind == "anti_causal" else \
                  (np.arange(n)[None, :] > rows_[:, None] + off)
            s[bad] = -np.inf
        m = s.max(axis=1)
        l = np.exp(s - m[:, None]).sum(axis=1)
        lse = m + (l if kind == "lse_no_log" else np.log(l))
        prob = np.exp(s - lse[:, None]) if kind != "lse_no_log" else np.exp(s - m[:, None]) / l[:, None]
        p = float(np.float32(dropout_p))
        if p > 0:
            z = PH.keep_mask(b, h, rows_, np.arange(n), p, seed)
            prob = prob * z if kind == "dropout_unscaled" else prob * z / (1 - p)
        o = (prob.T @ v) if kind == "transposed_p" else prob @ v
        return o, lse
    return fwd


def _mutant_backward(kind):
    def bwd(q, k, v, do, scale, causal=False, dropout_p=0.0, seed=0, b=0, h=0):
        dq, dk, dv, aux = A.backward(q, k, v, do, scale, causal, dropout_p, seed, b, h)
        q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
        if kind == "no_D":
            s = A.scores(q, k, scale, causal)
            prob = np.exp(s - aux[1][:, None])
            p = float(np.float32(dropout_p))
            zs = PH.keep_mask(b, h, np.arange(len(k)), np.arange(len(k)), p, seed) / (1 - p) if p else 1.0
            ds = prob * ((do @ v.T) * zs)
            dq, dk = scale * ds @ k, scale * ds.T @ q
        elif kind == "dk_unscaled":
            dk = dk / scale
        elif kind == "dv_transposed":
            s = A.scores(q, k, scale, causal)
            dv = np.exp(s - aux[1][:, None]) @ do
        return dq, dk, dv, aux
    return bwd


@pytest.mark.parametrize("kind", ["no_scale", "anti_causal", "lse_no_log", "transposed_p"])
def test_planted_forward_mistakes_are_caught(kind):
    fwd = _mutant_forward(kind)
    caught = [pin_bruteforce(fwd) > 1e-6, pin_sdpa(fwd) > 1e-6, pin_closed_forms(fwd) > 1e-6]
    assert any(caught), kind


def test_planted_dropout_scaling_mistake_is_caught():
    fwd = _mutant_forward("dropout_unscaled")
    assert pin_bruteforce(fwd) > 1e-6


@pytest.mark.parametrize("kind", ["offset_ignored", "offset_negated", "no_scale"])
def test_planted_key_offset_mistakes_are_caught(kind):
    assert pin_key_offset(_mutant_forward(kind)) > 1e-6, kind


@pytest.mark.parametrize("kind", ["no_D", "dk_unscaled", "dv_transposed"])
def test_planted_backward_mistakes_are_caught(kind):
    bwd = _mutant_backward(kind)
    assert pin_finite_differences(bwd) > 1e-3 or pin_autograd(bwd) > 1e-6
