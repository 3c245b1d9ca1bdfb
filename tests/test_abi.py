"""The C ABI library on the CPU: it loads, exports every symbol include/fa.h
declares, and rejects invalid arguments before any HIP call (no GPU needed,
no kernel is launched by these tests)."""
import ctypes
import os
import re

import pytest

import exact_io_aware_53_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")
FAKE = 4096   # a non-null, 16-byte aligned address; never dereferenced on these paths


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(fa.LIB_PATH):
        pytest.fail("libfa.so is not built (run __graft_entry__.build())")
    return fa.lib()


def test_exports_every_declared_symbol(L):
    declared = header_functions()
    assert declared == sorted(fa.SIGNATURES), declared
    for name in declared:
        assert isinstance(getattr(L, name), ctypes._CFuncPtr)


def test_noalloc_rejects_invalid_arguments(L):
    """fa_bwd_noalloc validates like fa_bwd, and rejects a problem whose workspace
    would not fit its scratch, all before any HIP call."""
    inv, uns = fa.FA_ERR_INVALID_ARG, fa.FA_ERR_UNSUPPORTED
    assert fa.NOALLOC_SCRATCH_BYTES == 128 << 20

    def call(B=1, H=2, N=100, d=64, ptr=FAKE, scale=0.125, p=0.0):
        return L.fa_bwd_noalloc(*([ptr] * 9), B, H, N, d, scale, 1, p, 0, None)
    assert call(ptr=None) == inv
    assert call(ptr=FAKE + 8) == inv
    assert call(d=96) == uns
    assert call(N=0) == inv
    assert call(scale=float("nan")) == inv
    assert call(p=1.0) == inv
    # B*H*N rows: the largest that fits the scratch at d = 128, and one past it
    rows_fit = max(r for r in range(258000, 258200) if L.fa_bwd_workspace_size(1, 1, r, 128) <= fa.NOALLOC_SCRATCH_BYTES)
    assert L.fa_bwd_workspace_size(1, 1, rows_fit + 1, 128) > fa.NOALLOC_SCRATCH_BYTES
    assert call(B=1, H=1, N=rows_fit + 1, d=128) == inv
    assert call(B=2, H=32, N=8192, d=128) == inv


def test_status_strings(L):
    for code in range(4):
        assert L.fa_status_string(code).startswith(b"FA_")
    assert L.fa_status_string(99) == b"unknown fa_status"


def test_workspace_size(L):
    B, H, N, d = 2, 16, 4096, 64
    rows = B * H * N
    rnd = lambda x: (x + 255) // 256 * 256
    assert L.fa_bwd_workspace_size(B, H, N, d) == rnd(rows * d * 4) + 2 * rnd(rows * 4)
    assert L.fa_bwd_workspace_size(0, 1, 1, 64) == 0
    assert L.fa_bwd_workspace_size(1024, 1024, 1024, 128) == 0   # above 2^31 - 1 elements


def fwd_call(L, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=1, N=128, d=64, scale=0.125,
             causal=0, p=0.0, seed=0)
    a.update(kw)
    return [L.fa_fwd, L.fa_fwd_f32][a.pop("f32", 0)](
        a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"], a["d"], a["scale"],
        a["causal"], a["p"], a["seed"], None)


@pytest.mark.parametrize("f32", [0, 1])
def test_forward_rejects_invalid_arguments(L, f32):
    inv, uns = fa.FA_ERR_INVALID_ARG, fa.FA_ERR_UNSUPPORTED
    for name in ("q", "k", "v", "o", "lse"):
        assert fwd_call(L, f32=f32, **{name: None}) == inv
        assert fwd_call(L, f32=f32, **{name: FAKE + 8}) == inv       # misaligned
    for name in ("B", "H", "N"):
        assert fwd_call(L, f32=f32, **{name: 0}) == inv
        assert fwd_call(L, f32=f32, **{name: -3}) == inv
    assert fwd_call(L, f32=f32, scale=float("inf")) == inv
    assert fwd_call(L, f32=f32, scale=float("nan")) == inv
    assert fwd_call(L, f32=f32, scale=0.0) == inv
    assert fwd_call(L, f32=f32, scale=-0.125) == inv
    for p in (-0.1, 1.0, 1.5, float("nan")):
        assert fwd_call(L, f32=f32, p=p) == inv
    assert fwd_call(L, f32=f32, B=4096, H=4096, N=4096, d=64) == inv   # too many elements
    for d in (0, 32, 96, 256):
        assert fwd_call(L, f32=f32, d=d) == (inv if d == 0 else uns)


@pytest.mark.parametrize("f32", [0, 1])
def test_backward_rejects_invalid_arguments(L, f32):
    fn = [L.fa_bwd, L.fa_bwd_f32][f32]
    need = L.fa_bwd_workspace_size(1, 2, 256, 64)

    def call(ws=FAKE * 16, ws_bytes=need, d=64, p=0.0, nulls=()):
        ptr = [None if i in nulls else FAKE for i in range(9)]
        return fn(*ptr, 1, 2, 256, d, 0.125, 1, p, 7, ws, ws_bytes, None)

    assert call(ws_bytes=need - 1) == fa.FA_ERR_INVALID_ARG
    assert call(ws=None) == fa.FA_ERR_INVALID_ARG
    assert call(ws=FAKE * 16 + 16) == fa.FA_ERR_INVALID_ARG         # workspace not 256-aligned
    for i in range(9):
        assert call(nulls=(i,)) == fa.FA_ERR_INVALID_ARG
    assert call(p=1.0) == fa.FA_ERR_INVALID_ARG
    assert call(d=80) == fa.FA_ERR_UNSUPPORTED


def test_decode_rejects_invalid_arguments(L):
    inv, uns = fa.FA_ERR_INVALID_ARG, fa.FA_ERR_UNSUPPORTED

    def call(Nq=1, Nk=4096, d=128, scale=0.1, ws=FAKE * 16, ws_bytes=None, nulls=()):
        need = L.fa_fwd_decode_workspace_size(2, 4, Nq, Nk, d)
        ptr = [None if i in nulls else FAKE for i in range(5)]
        return L.fa_fwd_decode(*ptr, 2, 4, Nq, Nk, d, scale, 1, ws,
                               need if ws_bytes is None else ws_bytes, None)

    for i in range(5):
        assert call(nulls=(i,)) == inv
    assert call(Nq=5, Nk=4) == inv                 # more queries than keys
    assert call(Nq=0) == inv
    assert call(scale=0.0) == inv and call(scale=-1.0) == inv and call(scale=float("nan")) == inv
    assert call(d=96) == uns
    assert call(ws=None) == inv                     # this shape is split, so it needs scratch
    assert call(ws_bytes=1) == inv
    assert call(ws=FAKE * 16 + 64) == inv           # not 256-aligned


def test_decode_paged_rejects_invalid_arguments(L):
    inv = fa.FA_ERR_INVALID_ARG

    def call(page=64, max_blocks=64, nulls=(), ws_bytes=None, Nq=1):
        need = L.fa_fwd_decode_paged_workspace_size(2, 4, Nq, max_blocks, page, 128)
        ptr = [None if i in nulls else FAKE for i in range(7)]
        return L.fa_fwd_decode_paged(*ptr, 2, 4, Nq, max_blocks, page, 100, 128, 0.1, 1, FAKE * 16,
                                     need if ws_bytes is None else ws_bytes, None)

    for i in range(7):
        assert call(nulls=(i,)) == inv
    assert call(page=48) == inv and call(page=16) == inv     # not a multiple of 32
    assert call(max_blocks=0) == inv
    assert call(Nq=64 * 64 + 1) == inv                          # more queries than the table reaches
    assert call(ws_bytes=1) == inv


def test_decode_workspace_size(L):
    assert L.fa_fwd_decode_workspace_size(1, 1, 1, 100, 64) == 0        # one key chunk: no scratch
    assert L.fa_fwd_decode_workspace_size(2, 4, 3, 5000, 128) > 0
    assert L.fa_fwd_decode_workspace_size(1, 1, 5, 4, 64) == 0          # invalid: Nq > Nk


def test_dropout_mask_rejects_invalid_arguments(L):
    inv = fa.FA_ERR_INVALID_ARG
    assert L.fa_dropout_mask(None, 1, 1, 8, 0, 0, 0.1, 1, None) == inv
    assert L.fa_dropout_mask(FAKE, 1, 1, 8, 1, 0, 0.1, 1, None) == inv   # b out of range
    assert L.fa_dropout_mask(FAKE, 1, 2, 8, 0, 2, 0.1, 1, None) == inv   # h out of range
    assert L.fa_dropout_mask(FAKE, 1, 1, 8, 0, 0, 1.0, 1, None) == inv
    assert L.fa_dropout_mask(FAKE, 1, 1, 65536, 0, 0, 0.1, 1, None) == inv  # N*N too large


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(fa, "_lib", None)
    monkeypatch.setattr(fa, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        fa.lib()


def problem(**kw):
    """A valid contiguous bf16 problem, then the overrides."""
    B, H, N, d = kw.pop("B", 2), kw.pop("H", 3), kw.pop("N", 100), kw.pop("d", 64)
    lay = fa.Layout(H * N * d, N * d, d)
    pb = fa.Problem(B=B, H=H, N=N, d=d, dtype=kw.pop("dtype", 0), cu_seqlens=kw.pop("cu", None),
                    total_tokens=kw.pop("total", 0))
    for name in ("q", "k", "v", "o", "dout", "dq", "dk", "dv"):
        setattr(pb, name, lay)
    pb.lse = fa.Layout(H * N, N, 1)
    for name, val in kw.items():
        setattr(pb, name, val)
    return pb


def fwd_ex(L, pb, scale=0.125, p=0.0, lse=FAKE):
    return L.fa_fwd_ex(ctypes.byref(pb), FAKE, FAKE, FAKE, FAKE, lse, scale, 1, p, 0, None)


def bwd_ex(L, pb, ws_bytes=None, ws=FAKE * 16):
    need = L.fa_bwd_ex_workspace_size(ctypes.byref(pb))
    return L.fa_bwd_ex(ctypes.byref(pb), *([FAKE] * 9), 0.125, 1, 0.0, 0, 1, ws,
                       need if ws_bytes is None else ws_bytes, None)


def test_ex_rejects_invalid_problems(L):
    inv, uns = fa.FA_ERR_INVALID_ARG, fa.FA_ERR_UNSUPPORTED
    assert L.fa_fwd_ex(None, FAKE, FAKE, FAKE, FAKE, FAKE, 0.1, 0, 0.0, 0, None) == inv
    for d in (16, 48, 80, 160, 512):
        assert fwd_ex(L, problem(d=d)) == uns
    assert fwd_ex(L, problem(dtype=2)) == uns
    for bad in (dict(B=0), dict(H=-1), dict(N=0)):
        assert fwd_ex(L, problem(**bad)) == inv
    N, d = 100, 64
    assert fwd_ex(L, problem(q=fa.Layout(0, N * d, d - 8))) == inv            # rows overlap
    assert fwd_ex(L, problem(k=fa.Layout(0, N * d + 4, d))) == inv            # head stride not 16-byte
    assert fwd_ex(L, problem(v=fa.Layout(-8, N * d, d))) == inv               # negative stride
    assert fwd_ex(L, problem(o=fa.Layout(0, N * d, d + 4))) == inv            # row stride not 16-byte
    assert fwd_ex(L, problem(lse=fa.Layout(0, N, 0))) == inv                  # LSE rows overlap
    assert fwd_ex(L, problem(N=2**20, q=fa.Layout(0, 0, 4096))) == inv        # head past 32-bit offsets
    assert fwd_ex(L, problem(cu=FAKE, total=0)) == inv                        # packed, no token count
    assert fwd_ex(L, problem(cu=FAKE + 2, total=10)) == inv                   # misaligned offsets
    assert fwd_ex(L, problem(), scale=0.0) == inv
    assert fwd_ex(L, problem(), p=1.0) == inv
    assert fwd_ex(L, problem(), lse=FAKE + 2) == inv                          # fp32 LSE misaligned


def test_ex_accepts_valid_layouts_on_the_host(L):
    """Every check above passes for these; the calls then stop at the launch,
    which needs a GPU, so only the validation result is compared."""
    for d in (32, 64, 96, 128, 256):
        pb = problem(d=d)
        assert L.fa_bwd_ex_workspace_size(ctypes.byref(pb)) > 0
    N, H, d = 100, 3, 64
    bshd = fa.Layout(N * H * d, d, H * d)
    pb = problem(q=bshd, k=bshd, v=bshd, o=bshd)
    assert L.fa_bwd_ex_workspace_size(ctypes.byref(pb)) > 0


def test_bwd_ex_workspace(L):
    inv = fa.FA_ERR_INVALID_ARG
    rnd = lambda x: (x + 255) // 256 * 256
    for d, dc in ((32, 64), (64, 64), (96, 128), (128, 128), (256, 256)):
        pb = problem(B=2, H=3, N=100, d=d)
        rows = 2 * 3 * 100
        assert L.fa_bwd_ex_workspace_size(ctypes.byref(pb)) == rnd(rows * dc * 4) + 2 * rnd(rows * 4)
    pb = problem()
    assert bwd_ex(L, pb, ws_bytes=1) == inv
    assert bwd_ex(L, pb, ws=None) == inv
    assert bwd_ex(L, pb, ws=FAKE * 16 + 8) == inv
    assert bwd_ex(L, problem(dq=fa.Layout(0, 0, 8))) == inv                   # dq rows overlap
    # one head's fp32 dQ accumulator past 32-bit byte offsets (its bf16 rows are not)
    big = problem(B=1, H=1, N=2**23, d=128)
    assert L.fa_bwd_ex_workspace_size(ctypes.byref(big)) == 0
    assert bwd_ex(L, big, ws_bytes=1 << 40) == inv
    assert L.fa_bwd_ex_workspace_size(ctypes.byref(problem(B=1, H=1, N=2**22, d=128))) > 0
    assert L.fa_bwd_ex_workspace_size(None) == 0
