"""The prefill attention kernels issue their LDS operand reads in one
inline-asm block and wait for them in a second one, with the tile copies in
between (tile_ops.h: read_k_issue / read_k_wait, read_v_issue / read_v_wait).
That is correct only while no instruction between the two blocks reads or
writes a destination register of the reads: such an instruction would see the
register before the LDS data has arrived. The compiler schedules other
independent work into that gap, so this test compiles attn_kernels.hip to
gfx950 assembly with the library's own flags (cross-compiled, no GPU) and checks
every split read of every kernel instantiation.
"""
import os
import re
import subprocess

import pytest

from learned_block_sparse_attngate_amd import build as seer_build


def _vregs(text):
    out = set()
    for m in re.finditer(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b", text):
        if m.group(3):
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def _asm_blocks(lines):
    """(start, end, body) of each inline-asm block, indices into `lines`."""
    i = 0
    while i < len(lines):
        if ";;#ASMSTART" in lines[i]:
            j = i + 1
            while ";;#ASMEND" not in lines[j]:
                j += 1
            yield i, j, [ln.strip() for ln in lines[i + 1:j]]
            i = j
        i += 1


@pytest.fixture(scope="module")
def kernel_asm(tmp_path_factory):
    try:
        cc = seer_build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "attn_kernels.s"
    flags = [f for f in seer_build.HIPCC_FLAGS if f != "-fPIC"]
    cmd = [cc, *flags, f"-I{seer_build.CSRC}", "--cuda-device-only", "-S",
           os.path.join(seer_build.CSRC, "attn_kernels.hip"), "-o", str(out)]
    subprocess.run(cmd, check=True, stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
    return out.read_text()


def _check_kernel(name, kernel_asm):
    """Number of split reads in kernel `name`; fails on a violation.

    From each issuing block, every control-flow path (fall-through and branch
    targets, as laid out in the assembly) is followed up to the next non-empty
    inline-asm block, which must be the wait; the instructions on the way must
    not name a destination register of the reads."""
    body = kernel_asm[kernel_asm.index(name + ":"):]
    # the function's end label: the compiler may lay out an early s_endpgm
    # (an exit path) or a loop's wait before its issue
    lines = body[:body.index(".Lfunc_end")].split("\n")
    labels = {}
    for i, ln in enumerate(lines):
        m = re.match(r"^(\.?\w+):", ln.strip())
        if m:
            labels[m.group(1)] = i
    blocks = list(_asm_blocks(lines))
    block_at = {b[0]: b for b in blocks}
    splits = 0
    for start, end, text in blocks:
        reads = [t for t in text if t.startswith("ds_read")]
        if not reads or any(t.startswith("s_waitcnt") for t in text):
            continue
        splits += 1
        dst = set()
        for t in reads:
            dst |= _vregs(t.split(",")[0])
        todo, seen = [end + 1], set()
        while todo:
            i = todo.pop()
            while True:
                assert i < len(lines), f"{name}: a path from a split read runs off the function"
                if i in seen:
                    break
                seen.add(i)
                if i in block_at:
                    _, bend, btext = block_at[i]
                    if not btext:            # empty block: a register-opacity marker
                        i = bend + 1
                        continue
                    assert btext == ["s_waitcnt lgkmcnt(0)"], (name, btext)
                    break
                ins = lines[i].split(";")[0].strip()
                if ins and not re.match(r"^\.?\w+:", ins):
                    assert not (_vregs(ins) & dst), f"{name}: '{ins}' touches a register the LDS reads are filling"
                    assert not ins.startswith("s_endpgm"), f"{name}: a split read reaches the end unwaited"
                    m = re.match(r"s_(c?)branch\w*\s+(\S+)", ins)
                    if m:
                        todo.append(labels[m.group(2)])
                        if not m.group(1):   # unconditional: no fall-through
                            break
                i += 1
    return splits


def test_no_instruction_touches_a_split_read_destination(kernel_asm):
    names = re.findall(
        r"^(_ZN4seer\S*(?:attn_sparse_xcd_kernel|attn_sparse_rows_kernel|attn_fwd_kernel|"
        r"attn_varlen_kernel)\S*):",
        kernel_asm, re.M)
    # D = 64 and 128: the XCD-owned chunks in both phases (chunks past the
    # row, the row's diagonal chunk with the merge); the
    # persistent rows (D = 128); the row kernels in block-sparse, dense and
    # ground-truth mode
    assert len(names) == 2 + 2 + 1 + 6 + 6, names
    for name in names:
        # every kernel reads K and V of at least two inlined tile bodies (the
        # diagonal tile and the others) through the split form
        assert _check_kernel(name, kernel_asm) >= 4, name
    # the GQA dense kernel splits its K reads (diagonal tile and the others)
    gqa = re.findall(r"^(_ZN4seer\S*attn_dense_gqa_kernel\S*):", kernel_asm, re.M)
    assert len(gqa) == 4, gqa
    for name in gqa:
        assert _check_kernel(name, kernel_asm) >= 2, name


_SYNTH = """_ZN4seer3fooEv:
\t;;#ASMSTART
\tds_read_b128 v[0:3], v10
\t;;#ASMEND
\ts_cbranch_scc1 .LBB0_2
\tv_mov_b32 v20, v21
.LBB0_1:                                ; %tail
\t;;#ASMSTART
\ts_waitcnt lgkmcnt(0)
\t;;#ASMEND
\ts_endpgm
.LBB0_2:
\tv_add_f32_e32 v{reg}, v12, v13
\ts_branch .LBB0_1
.Lfunc_end0:
"""


@pytest.mark.parametrize("reg,bad", [(14, False), (2, True)])
def test_checker_follows_branches(reg, bad):
    """The checker follows a branch taken between the two blocks (a loop's
    wait laid out before its issue) and finds a destination register named on
    that path only."""
    asm = _SYNTH.format(reg=reg)
    if bad:
        with pytest.raises(AssertionError):
            _check_kernel("_ZN4seer3fooEv", asm)
    else:
        assert _check_kernel("_ZN4seer3fooEv", asm) == 1
