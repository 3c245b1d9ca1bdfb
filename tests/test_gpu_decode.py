"""GPU parity of the decode-shaped forward (fa_fwd_decode) against the fp64 oracle.

Nq query rows sit at key positions Nk - Nq .. Nk - 1 of an Nk-row key/value
sequence; causal rows see the keys up to their own position. Every row of every
head is checked on the small shapes, every row of two seeded heads on the full
decode workloads. Tolerances as for the forward: bf16 O <= 1e-2 (widened only
where bf16 storage alone exceeds it), LSE <= 1e-3.
"""
import math

import numpy as np
import pytest
import torch

import exact_io_aware_53_amd as fa
import oracle
from exact_io_aware_53_amd.inputs import DECODE_WORKLOADS, make_decode_inputs, sample_heads, to_f64
from parity_checks import Stats

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.lib()


def decode_inputs(B, H, Nq, Nk, d, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    return [torch.from_numpy(rng.standard_normal((B, H, n, d), dtype=np.float32)).to(torch.bfloat16)
            for n in (Nq, Nk, Nk)]


def check_decode(q, k, v, o, lse, causal, heads, tag=""):
    Nq, Nk, d = q.shape[2], k.shape[2], q.shape[3]
    scale = 1.0 / math.sqrt(d)
    o_c, l_c = o.float().cpu(), lse.cpu()
    st = Stats(torch.bfloat16)
    for (b, h) in heads:
        ro, rl = oracle.forward(to_f64(q[b, h]), to_f64(k[b, h]), to_f64(v[b, h]), scale, causal,
                                key_offset=Nk - Nq)
        st.add(o_c[b, h].double().numpy(), ro, l_c[b, h].double().numpy(), rl)
    st.check(f"decode {tag}")


# (B, H, Nq, Nk, d): one key; one chunk (Nk <= 128); many chunks with a ragged
# last one; several 32-row query blocks; Nq = Nk (the full causal square);
# causal blocks whose early rows see none of the last chunks.
SHAPES = [(1, 1, 1, 1, 64), (1, 2, 1, 100, 128), (2, 2, 5, 3000, 64), (1, 1, 32, 4099, 128),
          (1, 2, 33, 777, 64), (1, 1, 70, 70, 128), (2, 1, 17, 5000, 128), (1, 3, 64, 129, 64),
          (1, 1, 96, 2000, 64)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_decode_small(shape, causal):
    B, H, Nq, Nk, d = shape
    q, k, v = decode_inputs(B, H, Nq, Nk, d, 4400 + Nq + Nk + d)
    o, lse = fa.fwd_decode(q.cuda(), k.cuda(), v.cuda(), causal=causal)
    torch.cuda.synchronize()
    check_decode(q, k, v, o, lse, causal, [(b, h) for b in range(B) for h in range(H)], str(shape))


@pytest.mark.parametrize("name", list(DECODE_WORKLOADS))
def test_decode_workload(name):
    w = DECODE_WORKLOADS[name]
    t = make_decode_inputs(w)
    if w.page:
        o, lse = fa.fwd_decode_paged(t["q"].cuda(), t["k_pages"].cuda(), t["v_pages"].cuda(),
                                     t["block_table"].cuda(), t["seq_lens"].cuda(), causal=w.causal)
    else:
        o, lse = fa.fwd_decode(t["q"].cuda(), t["k"].cuda(), t["v"].cuda(), causal=w.causal)
    torch.cuda.synchronize()
    check_decode(t["q"], t["k"], t["v"], o, lse, w.causal, sample_heads(w, 2), name)


def test_decode_is_deterministic():
    q, k, v = (x.cuda() for x in decode_inputs(2, 4, 3, 6000, 128, 4501))
    outs = [fa.fwd_decode(q, k, v, causal=True) for _ in range(3)]
    for o, l in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(l, outs[0][1])


def test_decode_single_query_equals_last_row_of_forward():
    """A one-row decode against the whole sequence is the forward's last causal row."""
    B, H, N, d = 1, 2, 700, 64
    q, k, v = (x.cuda() for x in decode_inputs(B, H, N, N, d, 4502))
    o_f, l_f = fa.fwd(q, k, v, causal=True)
    o_d, l_d = fa.fwd_decode(q[:, :, -1:].contiguous(), k, v, causal=True)
    assert (o_d[:, :, 0].float() - o_f[:, :, -1].float()).abs().max().item() <= 2e-2
    assert (l_d[:, :, 0] - l_f[:, :, -1]).abs().max().item() <= 2e-3


def test_decode_outputs_stay_in_bounds():
    B, H, Nq, Nk, d = 1, 3, 5, 3000, 128
    q, k, v = (x.cuda() for x in decode_inputs(B, H, Nq, Nk, d, 4503))
    pad = 4096
    ob = torch.full((B * H * Nq * d + 2 * pad,), 7.0, dtype=torch.bfloat16, device="cuda")
    lb = torch.full((B * H * Nq + 2 * pad,), 7.0, dtype=torch.float32, device="cuda")
    need = fa.decode_workspace_size(B, H, Nq, Nk, d)
    assert need > 0
    wb = torch.full((need + 2 * 4096,), 7, dtype=torch.uint8, device="cuda")
    fa.fwd_decode(q, k, v, causal=True, out=ob[pad:-pad].view(B, H, Nq, d),
                  lse=lb[pad:-pad].view(B, H, Nq), workspace=wb[4096:-4096])
    torch.cuda.synchronize()
    for buf, p_ in ((ob, pad), (lb, pad), (wb, 4096)):
        assert torch.all(buf[:p_] == 7) and torch.all(buf[-p_:] == 7)


# ------------------------------------------------------------ paged key/value
def make_paged(k, v, lens, page, rng, spare=3):
    """Scatter each sequence's rows [0, len) into pages of a shuffled pool.
    Returns (k_pages, v_pages [num_pages, H, page, d], block_table [B, max_blocks])."""
    B, H, Nk, d = k.shape
    max_blocks = -(-Nk // page)
    used = [-(-int(n) // page) for n in lens]
    num_pages = sum(used) + spare
    perm = rng.permutation(num_pages)
    kp = torch.zeros((num_pages, H, page, d), dtype=k.dtype)
    vp = torch.zeros_like(kp)
    table = np.full((B, max_blocks), -1, dtype=np.int32)        # unused slots hold -1
    nxt = 0
    for b in range(B):
        for blk in range(used[b]):
            pid = int(perm[nxt]); nxt += 1
            table[b, blk] = pid
            rows = slice(blk * page, min((blk + 1) * page, int(lens[b])))
            n = rows.stop - rows.start
            kp[pid, :, :n] = k[b, :, rows]
            vp[pid, :, :n] = v[b, :, rows]
    return kp, vp, torch.from_numpy(table)


def check_paged(q, k, v, lens, o, lse, causal, tag):
    """Oracle on each sequence's own keys; rows that see no key must give O = 0, LSE = -inf."""
    B, H, Nq, d = q.shape
    scale = 1.0 / math.sqrt(d)
    o_c, l_c = o.float().cpu(), lse.cpu()
    for b in range(B):
        n = int(lens[b])
        off = n - Nq
        for h in range(H):
            go, gl = o_c[b, h].double().numpy(), l_c[b, h].double().numpy()
            rows = [i for i in range(Nq) if (off + i >= 0 if causal else n > 0)]
            dead = [i for i in range(Nq) if i not in rows]
            if dead:
                assert np.all(go[dead] == 0) and np.all(np.isneginf(gl[dead])), f"{tag} empty rows"
            if not rows:
                continue
            ro, rl = oracle.forward(to_f64(q[b, h]), to_f64(k[b, h, :n]), to_f64(v[b, h, :n]), scale,
                                    causal, rows=np.array(rows), key_offset=off)
            st = Stats(torch.bfloat16)
            st.add(go[rows], ro, gl[rows], rl)
            st.check(f"paged decode {tag} b{b} h{h}")


PAGED_CASES = [  # (H, Nq, lens, page, d)
    (2, 1, [1, 37, 300, 1024], 32, 64),
    (1, 4, [4, 129, 2000], 64, 128),
    (3, 40, [40, 90, 700], 256, 64),
    (2, 3, [0, 2, 5000], 128, 128),      # an empty sequence and one shorter than Nq
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", PAGED_CASES, ids=lambda c: f"h{c[0]}q{c[1]}p{c[3]}d{c[4]}")
def test_decode_paged(case, causal):
    H, Nq, lens, page, d = case
    B, Nk = len(lens), max(lens)
    q, k, v = decode_inputs(B, H, Nq, Nk, d, 4600 + Nq + page + d)
    rng = np.random.Generator(np.random.PCG64(4700 + page))
    kp, vp, table = make_paged(k, v, lens, page, rng)
    o, lse = fa.fwd_decode_paged(q.cuda(), kp.cuda(), vp.cuda(), table.cuda(),
                                 torch.tensor(lens, dtype=torch.int32).cuda(), causal=causal)
    torch.cuda.synchronize()
    check_paged(q, k, v, lens, o, lse, causal, f"{case}")


def test_decode_paged_matches_contiguous_decode():
    """Identity block table with full-length sequences: the paged kernel gives the
    contiguous kernel's result bit for bit (same work split, same tiles)."""
    B, H, Nq, Nk, d, page = 2, 4, 3, 4096, 128, 128
    q, k, v = (x.cuda() for x in decode_inputs(B, H, Nq, Nk, d, 4801))
    nb = Nk // page
    kp = k.view(B, H, nb, page, d).permute(0, 2, 1, 3, 4).reshape(B * nb, H, page, d).contiguous()
    vp = v.view(B, H, nb, page, d).permute(0, 2, 1, 3, 4).reshape(B * nb, H, page, d).contiguous()
    table = torch.arange(B * nb, dtype=torch.int32, device="cuda").view(B, nb)
    lens = torch.full((B,), Nk, dtype=torch.int32, device="cuda")
    o1, l1 = fa.fwd_decode(q, k, v, causal=True)
    o2, l2 = fa.fwd_decode_paged(q, kp, vp, table, lens, causal=True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_decode_paged_bad_table_entry_reads_zeros():
    """A block-table entry outside the pool reads as zero keys and values."""
    H, Nq, d, page = 1, 1, 64, 32
    lens = [96]
    q, k, v = decode_inputs(1, H, Nq, 96, d, 4901)
    rng = np.random.Generator(np.random.PCG64(4902))
    kp, vp, table = make_paged(k, v, lens, page, rng)
    table[0, 1] = 10_000                                      # the middle page: out of range
    o, lse = fa.fwd_decode_paged(q.cuda(), kp.cuda(), vp.cuda(), table.cuda(),
                                 torch.tensor(lens, dtype=torch.int32).cuda())
    torch.cuda.synchronize()
    k0, v0 = k.clone(), v.clone()
    k0[0, :, 32:64] = 0
    v0[0, :, 32:64] = 0
    check_paged(q, k0, v0, lens, o, lse, False, "bad entry")
