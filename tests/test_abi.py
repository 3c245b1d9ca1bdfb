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
