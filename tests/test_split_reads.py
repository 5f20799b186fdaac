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
    """Number of split reads in kernel `name`; fails on a violation."""
    body = kernel_asm[kernel_asm.index(name + ":"):]
    lines = body[:body.index("s_endpgm")].split("\n")
    blocks = list(_asm_blocks(lines))
    splits = 0
    for n, (start, end, text) in enumerate(blocks):
        reads = [t for t in text if t.startswith("ds_read")]
        if not reads or any(t.startswith("s_waitcnt") for t in text):
            continue
        splits += 1
        dst = set()
        for t in reads:
            dst |= _vregs(t.split(",")[0])
        # empty inline-asm blocks (register-opacity markers) may sit between
        # the two; the instructions around them are checked like the others
        nxt = n + 1
        while not blocks[nxt][2]:
            nxt += 1
        nxt_start, _, nxt_text = blocks[nxt]
        assert nxt_text == ["s_waitcnt lgkmcnt(0)"], (name, nxt_text)
        for ln in lines[end + 1:nxt_start]:
            ins = ln.split(";")[0].strip()
            if ins and not ins.endswith(":"):
                assert not (_vregs(ins) & dst), f"{name}: '{ins}' touches a register the LDS reads are filling"
    return splits


def test_no_instruction_touches_a_split_read_destination(kernel_asm):
    names = re.findall(
        r"^(_ZN4seer\S*(?:attn_sparse_xcd_kernel|attn_sparse_rows_kernel|attn_fwd_kernel|attn_varlen_kernel)\S*):",
        kernel_asm, re.M)
    # D = 64 and 128; the persistent rows (D = 128); the row kernels in
    # block-sparse, dense and ground-truth mode
    assert len(names) == 2 + 1 + 6 + 6, names
    for name in names:
        # every kernel reads K and V of at least two inlined tile bodies (the
        # diagonal tile and the others) through the split form
        assert _check_kernel(name, kernel_asm) >= 4, name
    # the GQA dense kernel splits its K reads (diagonal tile and the others)
    gqa = re.findall(r"^(_ZN4seer\S*attn_dense_gqa_kernel\S*):", kernel_asm, re.M)
    assert len(gqa) == 4, gqa
    for name in gqa:
        assert _check_kernel(name, kernel_asm) >= 2, name
