"""Wait states around the inline assembly of the kernels (CPU only).

Two kinds of inline assembly are checked, because the compiler's hazard
recognizer does not see into either.

The tile copies are issued as inline assembly so that the compiler's wait-count
tracking does not serialise them with the LDS reads of the other buffer. The
compiler's hazard checks do not see into inline assembly either: a vector
instruction that writes an SGPR (v_readlane reloading a spilled resource word,
v_readfirstlane into M0) must be at least five wait states ahead of a
vector-memory instruction that reads that SGPR, or the copy can read a stale
buffer resource. This test compiles every kernel source to gfx950 assembly with
the library's own flags and checks that distance in front of every inline copy.

Matrix-core products written as inline assembly need the same care: a vector
instruction that writes a source register of a product (its A, B or C
operand) must be at least MFMA_SRC_WAIT_STATES wait states ahead of it, and an
instruction other than the next product of the same accumulator that reads the
product's result must come at least MFMA_RESULT_WAIT_STATES wait states after
it. The kernels issue every product through the compiler's builtins today, so
the scan over them finds none; it still runs over every kernel, so that an
inline product added later is checked, and the detector itself is tested on
hand-written snippets. The scan follows straight-line code only: it stops at
labels and branches.
"""
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from exact_io_aware_53_amd import build as fabuild

VMEM_SGPR_WAIT_STATES = 5
MFMA_SRC_WAIT_STATES = 2
MFMA_RESULT_WAIT_STATES = 18


def _sregs(tok):
    tok = tok.strip().rstrip(",")
    m = re.match(r"s\[(\d+):(\d+)\]$", tok)
    if m:
        return {f"s{i}" for i in range(int(m.group(1)), int(m.group(2)) + 1)}
    return {tok} if re.match(r"(s\d+|m0|vcc|vcc_lo|vcc_hi)$", tok) else set()


def _vector_sgpr_writes(inst):
    """SGPRs a vector instruction writes: its destination, or the carry/compare
    mask of the instructions that also produce one."""
    op, _, rest = inst.partition(" ")
    dst = rest.split(",")
    w = _sregs(dst[0])
    if re.match(r"v_(cmp|cmpx|mad_u64|mad_i64|add_co|sub_co|subrev_co|addc_co|subb_co|div_scale)", op):
        for d in dst[:2]:
            w |= _sregs(d)
    return w


def inline_copy_hazards(asm_text):
    """(copies checked, [(line, writer, wait states, copy)]) for every
    `buffer_load_* ... lds` inside an inline-assembly block."""
    lines = asm_text.split("\n")
    found, checked = [], 0
    for i, raw in enumerate(lines):
        t = raw.strip()
        if not (t.startswith("buffer_load") and t.endswith(" lds")):
            continue
        j = i - 1
        while j >= 0 and lines[j].strip().startswith("s_nop"):
            j -= 1
        if "ASMSTART" not in lines[j]:
            continue
        checked += 1
        reads = _sregs(t.split(None, 1)[1].split(",")[1]) | {"m0"}
        ws, k = 0, i - 1
        while k >= 0 and ws < VMEM_SGPR_WAIT_STATES:
            u = lines[k].strip()
            k -= 1
            if not u or u.startswith(";") or u.startswith(".") or u.endswith(":"):
                continue
            m = re.match(r"s_nop (\d+)", u)
            if m:
                ws += int(m.group(1)) + 1
                continue
            if u.startswith("v_") and _vector_sgpr_writes(u) & reads:
                found.append((i + 1, u, ws, t))
            ws += 1
    return checked, found


def _regs(tok):
    """Register names of one operand: v[4:7] -> {v4..v7}, a3 -> {a3}."""
    tok = tok.strip().rstrip(",")
    m = re.match(r"([va])\[(\d+):(\d+)\]$", tok)
    if m:
        return {f"{m.group(1)}{i}" for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    return {tok} if re.match(r"[va]\d+$", tok) else set()


def _operands(inst):
    op, _, rest = inst.partition(" ")
    return op, [t.strip() for t in rest.split(",")] if rest else []


def _wait_states(u):
    m = re.match(r"s_nop (\d+)", u)
    return int(m.group(1)) + 1 if m else 1


def _is_code(u):
    return bool(u) and not u.startswith(";") and not u.startswith(".") and not u.endswith(":")


def _in_asm_block(lines, i):
    j = i - 1
    while j >= 0 and "ASMSTART" not in lines[j] and "ASMEND" not in lines[j]:
        j -= 1
    return j >= 0 and "ASMSTART" in lines[j]


def inline_mfma_hazards(asm_text):
    """(products checked, [(line, kind, other instruction, wait states, product)]) for
    every v_mfma inside an inline-assembly block: vector writes of its sources too
    close before it, and reads of its AGPR result too close after it."""
    lines = asm_text.split("\n")
    found, checked = [], 0
    for i, raw in enumerate(lines):
        t = raw.strip()
        if not t.startswith("v_mfma") or not _in_asm_block(lines, i):
            continue
        checked += 1
        op, ops = _operands(t)
        dst = _regs(ops[0])
        srcs = set().union(*(_regs(x) for x in ops[1:4]))
        # vector writes of a source before the product
        ws, k = 0, i - 1
        while k >= 0 and ws < MFMA_SRC_WAIT_STATES:
            u = lines[k].strip()
            k -= 1
            if u.endswith(":") or u.startswith("s_cbranch") or u.startswith("s_branch"):
                break
            if not _is_code(u):
                continue
            if u.startswith("v_") and not u.startswith("v_mfma"):
                _, uops = _operands(u)
                if uops and _regs(uops[0]) & srcs:
                    found.append((i + 1, "source written", u, ws, t))
            ws += _wait_states(u)
        # reads of the AGPR result after the product
        ws, k = 0, i + 1
        while k < len(lines) and ws < MFMA_RESULT_WAIT_STATES:
            u = lines[k].strip()
            k += 1
            if u.endswith(":") or u.startswith("s_cbranch") or u.startswith("s_branch") or u.startswith("s_endpgm"):
                break
            if not _is_code(u):
                continue
            uop, uops = _operands(u)
            if uop.startswith("v_mfma"):
                # the next product of the same accumulator reads it as C, exactly overlapped
                if _regs(uops[0]) == dst and len(uops) > 3 and _regs(uops[3]) == dst and not (
                        set().union(*(_regs(x) for x in uops[1:3])) & dst):
                    ws += _wait_states(u)
                    continue
                reads = set().union(*(_regs(x) for x in uops[1:]))
            else:
                reads = set().union(*(_regs(x) for x in uops[1:])) if uops else set()
            if reads & dst:
                found.append((i + 1, "result read", u, ws, t))
            ws += _wait_states(u)
    return checked, found


def _device_asm(src, out_dir):
    out = os.path.join(out_dir, os.path.basename(src) + ".s")
    cmd = [fabuild.hipcc(), "-x", "hip", *fabuild.flags(src), "--cuda-device-only", "-S", src, "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    with open(out) as f:
        return f.read()


def test_detector_flags_a_close_sgpr_reload():
    """The scan itself: a reload one wait state ahead is flagged, five are not."""
    close = ("\tv_readlane_b32 s7, v225, 19\n\t;;#ASMSTART\n\ts_nop 0\n"
             "\tbuffer_load_dwordx4 v1, s[4:7], 0 offen lds\n\t;;#ASMEND\n")
    far = close.replace("s_nop 0", "s_nop 4")
    m0 = ("\tv_readfirstlane_b32 m0, v3\n\t;;#ASMSTART\n\ts_nop 2\n"
          "\tbuffer_load_dword v1, s[8:11], 0 offen lds\n\t;;#ASMEND\n")
    assert len(inline_copy_hazards(close)[1]) == 1
    assert inline_copy_hazards(far) == (1, [])
    assert len(inline_copy_hazards(m0)[1]) == 1


@pytest.fixture(scope="module")
def kernel_asm(tmp_path_factory):
    """gfx950 assembly of every kernel source, compiled once with the library's flags."""
    if shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("needs hipcc")
    out = str(tmp_path_factory.mktemp("asm"))
    srcs = [s for s in fabuild.sources() if s.endswith(".hip")]
    with ThreadPoolExecutor(max_workers=min(len(srcs), 8)) as ex:
        return list(zip(srcs, ex.map(lambda s: _device_asm(s, out), srcs)))


def test_inline_lds_copies_keep_sgpr_wait_states(kernel_asm):
    total, problems = 0, []
    for src, text in kernel_asm:
        n, found = inline_copy_hazards(text)
        total += n
        problems += [(os.path.basename(src),) + f for f in found]
    print(f"inline LDS copies checked: {total}")
    assert total > 0, "no inline LDS copies found: the scan no longer matches the generated code"
    assert not problems, "\n".join(f"{s}:{ln}: '{w}' {ws} wait states before '{c}'" for s, ln, w, ws, c in problems[:10])


def test_detector_flags_inline_product_hazards():
    """The scan itself on hand-written snippets: a source written one wait state
    before a product and an AGPR result read 8 wait states after it are flagged;
    two and 24 wait states, and back-to-back accumulation, are not."""
    prod = "v_mfma_f32_32x32x16_bf16 a[0:15], v[4:7], v[8:11], a[0:15]"
    close_src = f"\tv_mov_b32 v5, v1\n\t;;#ASMSTART\n\ts_nop 0\n\t{prod}\n\t;;#ASMEND\n"
    far_src = close_src.replace("s_nop 0", "s_nop 1")
    acc_w = f"\tv_accvgpr_write_b32 a3, 0\n\t;;#ASMSTART\n\t{prod}\n\t;;#ASMEND\n"
    close_res = (f"\t;;#ASMSTART\n\ts_nop 1\n\t{prod}\n\t;;#ASMEND\n\t;;#ASMSTART\n\ts_nop 7\n\t;;#ASMEND\n"
                 "\tv_accvgpr_read_b32 v20, a3\n")
    far_res = close_res.replace("s_nop 7\n", "s_nop 7\n\ts_nop 7\n\ts_nop 7\n")
    chain = (f"\t;;#ASMSTART\n\ts_nop 1\n\t{prod}\n\t;;#ASMEND\n\t;;#ASMSTART\n\ts_nop 1\n"
             "\tv_mfma_f32_32x32x16_bf16 a[0:15], v[12:15], v[16:19], a[0:15]\n\t;;#ASMEND\n"
             "\t;;#ASMSTART\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\t;;#ASMEND\n\tv_accvgpr_read_b32 v20, a0\n")
    assert [f[1] for f in inline_mfma_hazards(close_src)[1]] == ["source written"]
    assert inline_mfma_hazards(far_src) == (1, [])
    assert [f[1] for f in inline_mfma_hazards(acc_w)[1]] == ["source written"]
    assert [f[1] for f in inline_mfma_hazards(close_res)[1]] == ["result read"]
    assert inline_mfma_hazards(far_res) == (1, [])
    assert inline_mfma_hazards(chain) == (2, [])


def test_inline_products_keep_wait_states(kernel_asm):
    total, problems = 0, []
    for src, text in kernel_asm:
        n, found = inline_mfma_hazards(text)
        total += n
        problems += [(os.path.basename(src),) + f for f in found]
    print(f"inline products checked: {total}")
    assert not problems, "\n".join(f"{s}:{ln}: {kind}: '{u}' {ws} wait states from '{c}'"
                                    for s, ln, kind, u, ws, c in problems[:10])
