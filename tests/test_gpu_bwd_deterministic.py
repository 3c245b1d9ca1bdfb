"""GPU parity of the deterministic backward (fa_bwd_deterministic): dQ from a
pass of its own over the query blocks, no atomics.

Bars: the gradients meet the bf16 tolerance against the fp64 oracle (max|g -
g_ref| / max|g_ref| <= 2e-2); dK and dV are bit-identical to fa_bwd's (the
key-side pass is the fused kernel without its dQ products); dQ is
bit-identical across repeated calls, and within the bf16 tolerance of the
atomically accumulated dQ that fa_bwd computes with dropout. Without dropout
fa_bwd takes this same path, so all three gradients are bit-identical.
"""
import math

import numpy as np
import pytest
import torch

import exact_io_aware_53_amd as fa
import oracle
from exact_io_aware_53_amd.inputs import WORKLOADS, make_inputs, normal_tensors, sample_heads, to_f64

pytestmark = pytest.mark.gpu

GRAD_TOL = 2e-2
SEED = 0x0123456789ABCDEF


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.lib()


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


def run_both(q, k, v, do, causal, p, seed):
    gq, gk, gv, gdo = (t.cuda() for t in (q, k, v, do))
    o, lse = fa.fwd(gq, gk, gv, causal=causal, dropout_p=p, seed=seed)
    det = fa.bwd(gq, gk, gv, o, lse, gdo, causal=causal, dropout_p=p, seed=seed,
                 deterministic=True)
    ato = fa.bwd(gq, gk, gv, o, lse, gdo, causal=causal, dropout_p=p, seed=seed)
    torch.cuda.synchronize()
    return det, ato


def check_heads(q, k, v, do, grads, heads, causal, p, seed, more=()):
    """Worst relative-to-max gradient error over the heads, for `grads` and any
    further (dQ, dK, dV) sets in `more` (one oracle call per head)."""
    d = q.shape[-1]
    worst = 0.0
    for b, h in heads:
        rq, rk, rv, _ = oracle.backward(to_f64(q[b, h]), to_f64(k[b, h]), to_f64(v[b, h]),
                                        to_f64(do[b, h]), 1.0 / math.sqrt(d), causal, p, seed, b, h)
        head_max = max(np.abs(r).max() for r in (rq, rk, rv))
        for gs in (grads,) + tuple(more):
            for g, r in zip(gs, (rq, rk, rv)):
                worst = max(worst, rel_to_max(g[b, h].double().cpu().numpy(), r, head_max))
    return worst


# Ragged ends, one row, several 64- and 128-row tiles, B*H = 8 and 32 (the
# XCD-grouped workgroup order).
SHAPES = [(1, 2, 17, 64), (2, 1, 129, 128), (1, 1, 256, 64), (1, 2, 300, 128), (1, 1, 1, 64),
          (1, 8, 300, 64), (2, 16, 520, 128)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("p", [0.0, 0.1])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_deterministic_backward_small(shape, causal, p):
    B, H, N, d = shape
    q, k, v, do = normal_tensors(shape, 4242 + N + d, 4, torch.bfloat16)
    det, ato = run_both(q, k, v, do, causal, p, SEED)
    assert torch.equal(det[1], ato[1]), "dK differs from fa_bwd's"
    assert torch.equal(det[2], ato[2]), "dV differs from fa_bwd's"
    heads = [(b, h) for b in range(B) for h in range(H)]
    worst = check_heads(q, k, v, do, det, heads, causal, p, SEED)
    assert worst <= GRAD_TOL, f"grad err {worst:.3e}"


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("p", [0.0, 0.1])
def test_dq_pass_eight_wave_grid(d, causal, p):
    """B4 H32 N2000: the dQ pass's grid reaches 512 workgroups of eight waves, so
    it runs 256-row query blocks (the smaller shapes above run 128-row ones),
    with a ragged last block of 208 rows; two heads against the oracle."""
    shape = (4, 32, 2000, d)
    q, k, v, do = normal_tensors(shape, 7070 + d, 4, torch.bfloat16)
    det, ato = run_both(q, k, v, do, causal, p, SEED)
    assert torch.equal(det[1], ato[1]) and torch.equal(det[2], ato[2])
    worst = check_heads(q, k, v, do, det, [(0, 0), (3, 31)], causal, p, SEED)
    assert worst <= GRAD_TOL, f"grad err {worst:.3e}"


def test_deterministic_dq_is_bitwise_repeatable():
    shape = (2, 4, 1000, 128)
    q, k, v, do = (t.cuda() for t in normal_tensors(shape, 5151, 4, torch.bfloat16))
    o, lse = fa.fwd(q, k, v, causal=True, dropout_p=0.1, seed=SEED)
    runs = [fa.bwd(q, k, v, o, lse, do, causal=True, dropout_p=0.1, seed=SEED,
                   deterministic=True) for _ in range(3)]
    for r in runs[1:]:
        for a, b in zip(r, runs[0]):
            assert torch.equal(a, b)


def test_deterministic_dq_close_to_atomic_dq():
    shape = (1, 4, 700, 64)
    q, k, v, do = normal_tensors(shape, 6161, 4, torch.bfloat16)
    det, ato = run_both(q, k, v, do, True, 0.1, SEED)
    a, b = det[0].float(), ato[0].float()
    assert (a - b).abs().max().item() <= GRAD_TOL * b.abs().max().item()


def test_without_dropout_fa_bwd_is_the_two_pass_form():
    q, k, v, do = normal_tensors((2, 3, 333, 128), 6262, 4, torch.bfloat16)
    det, plain = run_both(q, k, v, do, True, 0.0, SEED)
    for a, b in zip(det, plain):
        assert torch.equal(a, b)


def test_deterministic_rejects_f32():
    q = torch.zeros(1, 1, 8, 64, device="cuda")
    with pytest.raises(ValueError):
        fa.bwd(q, q, q, q, torch.zeros(1, 1, 8, device="cuda"), q, deterministic=True)


def test_deterministic_workload_dropout_b2h16n4096d64():
    w = WORKLOADS["fwdbwd_causal_dropout_bf16_b2h16n4096d64"]
    t = make_inputs(w)
    det, ato = run_both(t["q"], t["k"], t["v"], t["do"], True, w.dropout_p, w.dropout_seed)
    assert torch.equal(det[1], ato[1]) and torch.equal(det[2], ato[2])
    worst = check_heads(t["q"], t["k"], t["v"], t["do"], det, sample_heads(w, 1), True,
                        w.dropout_p, w.dropout_seed)
    assert worst <= GRAD_TOL, f"grad err {worst:.3e}"


def test_backward_both_paths_b2h32n8192d128_q4():
    """The backward at the long softmax-stress shape (Q scaled by 4), the
    two-pass form without dropout and the fused atomic form with p = 0.1, one
    seeded head each against the oracle's full backward."""
    w = WORKLOADS["fwd_causal_q4_bf16_b2h32n8192d128"]
    t = make_inputs(w, with_grad_out=True)
    (b, h), = sample_heads(w, 1)
    for p in (0.0, 0.1):
        det, ato = run_both(t["q"], t["k"], t["v"], t["do"], True, p, SEED)
        assert torch.equal(det[1], ato[1]) and torch.equal(det[2], ato[2])
        more = (ato,) if p > 0 else ()
        worst = check_heads(t["q"], t["k"], t["v"], t["do"], det, [(b, h)], True, p, SEED,
                            more=more)
        assert worst <= GRAD_TOL, f"p={p}: grad err {worst:.3e}"
