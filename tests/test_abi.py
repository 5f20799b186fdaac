"""C ABI checks that need no GPU: the library loads, exports every function
include/seer.h declares, sizes its workspaces as documented, and rejects bad
arguments on the host before any HIP call (fake device pointers are passed;
they are never dereferenced because validation fails first)."""
import ctypes
import math
import os
import re
import subprocess

import pytest

import learned_block_sparse_attngate_amd as seer
from learned_block_sparse_attngate_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "seer.h")

pytestmark = pytest.mark.skipif(not os.path.exists(B.LIB_PATH), reason="libseer.so not built")

FAKE = ctypes.c_void_p(0x10000)       # 16-byte aligned, never dereferenced
FAKE_ODD = ctypes.c_void_p(0x10002)


def _lib():
    return seer.load_library()


def _shape(b=1, hq=4, hkv=2, s=256, d=128, blk=64):
    return seer.make_shape(b, hq, hkv, s, d, blk)


def _attn(shape, q=FAKE, k=FAKE, v=FAKE, mask=None, out=FAKE, dt=B.SEER_F32, lse=None, ws=None, ws_bytes=0):
    return _lib().seer_block_sparse_attn_fwd(ctypes.byref(shape) if shape is not None else None, q, k, v, mask,
                                             out, dt, lse, ws, ws_bytes, None)


def _gate(shape, dg=128, per_kv=0, mode=B.SEER_MASK_THRESHOLD, T=5e-4, k=4, per_head=None, scores=None,
          mask=FAKE, ws=FAKE, ws_bytes=1 << 40, rope=0.0):
    return _lib().seer_gate_fwd(ctypes.byref(shape), dg, per_kv, rope, FAKE, FAKE, FAKE, FAKE, mode, T, k, per_head,
                                scores, mask, ws, ws_bytes, None)


def _distill(shape, dg=128, per_kv=0, rope=0.0, gt=FAKE, loss=FAKE, gq=FAKE, gk=FAKE, ws=FAKE, ws_bytes=1 << 40):
    return _lib().seer_gate_distill_bwd(ctypes.byref(shape), dg, per_kv, rope, FAKE, FAKE, FAKE, FAKE, gt, loss,
                                        gq, gk, ws, ws_bytes, None)


def test_exports_every_declared_symbol():
    src = open(HEADER).read()
    declared = set(re.findall(r"\b(seer_[a-z_]+)\s*\(", src))
    assert declared == set(seer.EXPORTED)
    lib = _lib()
    for name in declared:
        assert hasattr(lib, name), name
    nm = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True).stdout
    for name in declared:
        assert re.search(rf"\bT {name}$", nm, re.M), f"{name} not exported as a text symbol"


def test_status_strings_and_version():
    lib = _lib()
    for code, name in [(0, b"SEER_OK"), (1, b"SEER_ERR_INVALID_ARG"), (2, b"SEER_ERR_SHAPE"),
                       (3, b"SEER_ERR_UNSUPPORTED"), (4, b"SEER_ERR_WORKSPACE"), (5, b"SEER_ERR_HIP")]:
        assert lib.seer_status_string(code) == name
    assert b"gfx950" in lib.seer_version()


def test_shape_validation():
    assert _attn(None) == B.SEER_ERR_INVALID_ARG
    assert _attn(_shape(s=-1)) == B.SEER_ERR_SHAPE
    assert b"negative" in _lib().seer_last_error()
    assert _attn(_shape(blk=32)) == B.SEER_ERR_SHAPE
    assert _attn(_shape(hq=6, hkv=4)) == B.SEER_ERR_SHAPE
    assert _attn(_shape(hq=4, hkv=0)) == B.SEER_ERR_SHAPE
    assert _attn(_shape(d=96)) == B.SEER_ERR_UNSUPPORTED
    assert _attn(_shape(s=(1 << 22) + 1)) == B.SEER_ERR_UNSUPPORTED
    assert _attn(_shape(b=4096, hq=4096, hkv=1, s=1 << 20)) == B.SEER_ERR_SHAPE


def test_empty_problem_is_a_noop():
    # nothing to do: OK even with NULL tensors, and no HIP call is made
    assert _attn(_shape(s=0), q=None, k=None, v=None, out=None) == B.SEER_OK
    assert _attn(_shape(b=0), q=None, k=None, v=None, out=None) == B.SEER_OK
    assert _lib().seer_last_error() == b""


def test_pointer_validation():
    assert _attn(_shape(), q=None) == B.SEER_ERR_INVALID_ARG
    assert _attn(_shape(), v=None) == B.SEER_ERR_INVALID_ARG
    assert _attn(_shape(), k=FAKE_ODD) == B.SEER_ERR_INVALID_ARG
    assert _attn(_shape(), out=None) == B.SEER_ERR_INVALID_ARG
    assert _attn(_shape(), dt=7) == B.SEER_ERR_INVALID_ARG
    assert _attn(_shape(), out=ctypes.c_void_p(0x10008), dt=B.SEER_F32) == B.SEER_ERR_INVALID_ARG


def test_sparse_workspace_validation():
    s = _shape(s=64 * 1200)                      # 1200 blocks: rows span up to three key chunks
    need = _lib().seer_attn_workspace_size(ctypes.byref(s))
    assert need > 0
    assert _attn(s, mask=FAKE) == B.SEER_ERR_WORKSPACE
    assert b"workspace" in _lib().seer_last_error()
    assert _attn(s, mask=FAKE, ws=FAKE, ws_bytes=need - 1) == B.SEER_ERR_WORKSPACE
    assert _attn(s, mask=FAKE, ws=ctypes.c_void_p(0x10008), ws_bytes=need) == B.SEER_ERR_WORKSPACE
    # dense attention takes no workspace
    assert _attn(s) != B.SEER_ERR_WORKSPACE


def test_gate_rope_and_distill_validation():
    s = _shape()
    for bad in (-1.0, math.inf, math.nan):
        assert _gate(s, rope=bad) == B.SEER_ERR_INVALID_ARG
        assert b"rope_theta" in _lib().seer_last_error()
        assert _distill(s, rope=bad) == B.SEER_ERR_INVALID_ARG
    assert _distill(s, dg=100) == B.SEER_ERR_UNSUPPORTED
    assert _distill(s, loss=None) == B.SEER_ERR_INVALID_ARG
    assert _distill(s, gt=None) == B.SEER_ERR_INVALID_ARG
    assert _distill(s, gk=None) == B.SEER_ERR_INVALID_ARG
    need = _lib().seer_gate_distill_workspace_size(ctypes.byref(s), 128, 0)
    assert _distill(s, ws_bytes=need - 1) == B.SEER_ERR_WORKSPACE
    assert _distill(_shape(s=0), gt=None, loss=FAKE) != B.SEER_ERR_WORKSPACE


def test_distill_workspace_size():
    # gate segments (pooled Q, pooled K, Q', K', logits) + dQ', dK' + row losses, 256-byte aligned
    lib = _lib()
    s = _shape(b=2, hq=4, hkv=2, s=200, d=64)
    nb = 4
    align = lambda x: (x + 255) // 256 * 256
    gate = (align(2 * 4 * nb * 64 * 4) + align(2 * 2 * nb * 192 * 4) + align(2 * 4 * nb * 32 * 4)
            + align(2 * 4 * nb * 32 * 4) + align(2 * 4 * nb * nb * 4))
    want = gate + 2 * align(2 * 4 * nb * 32 * 4) + align(2 * 4 * nb * 4)
    assert lib.seer_gate_distill_workspace_size(ctypes.byref(s), 32, 0) == want


def test_decode_validation():
    lib = _lib()
    s = _shape(hq=4, hkv=2, s=1000)                 # 16 blocks
    assert lib.seer_decode_compress_k(ctypes.byref(s), 0, FAKE, FAKE, -1, FAKE, 16, None) == B.SEER_ERR_INVALID_ARG
    assert lib.seer_decode_compress_k(ctypes.byref(s), 0, FAKE, FAKE, 17, FAKE, 16, None) == B.SEER_ERR_INVALID_ARG
    assert lib.seer_decode_compress_k(ctypes.byref(s), 0, FAKE, FAKE, 0, FAKE, 15, None) == B.SEER_ERR_INVALID_ARG
    assert b"kcomp_blocks" in lib.seer_last_error()
    assert lib.seer_decode_compress_k(ctypes.byref(s), 0, FAKE, FAKE, 16, FAKE, 16, None) == B.SEER_OK  # nothing to do
    assert lib.seer_decode_gate_fwd(ctypes.byref(s), 0, FAKE, FAKE, 16, 7, 0.1, 1, None, None, FAKE,
                                    None) == B.SEER_ERR_INVALID_ARG
    assert lib.seer_decode_gate_fwd(ctypes.byref(s), 0, FAKE, FAKE, 16, B.SEER_MASK_TOPK, 0.1, 0, None, None, FAKE,
                                    None) == B.SEER_ERR_INVALID_ARG
    assert lib.seer_decode_gate_fwd(ctypes.byref(s), 0, FAKE, FAKE, 16, B.SEER_MASK_THRESHOLD, 0.1, 1, None, FAKE,
                                    None, None) == B.SEER_ERR_INVALID_ARG
    assert lib.seer_decode_gate_fwd(ctypes.byref(s), 0, FAKE, FAKE, 16, B.SEER_MASK_THRESHOLD, 0.1, 1, None, None,
                                    FAKE, None) == B.SEER_ERR_INVALID_ARG          # scores hold the logits
    assert lib.seer_decode_gate_fwd(ctypes.byref(s), 0, ctypes.c_void_p(0x10008), FAKE, 16, B.SEER_MASK_THRESHOLD, 0.1, 1, None,
                                    FAKE, FAKE, None) == B.SEER_ERR_INVALID_ARG    # q not 16-byte aligned
    assert b"16-byte aligned" in lib.seer_last_error()
    big = _shape(hq=32, hkv=2, s=1000)              # 16 query heads per KV head
    need = lib.seer_decode_attn_workspace_size(ctypes.byref(s))
    assert need > 0
    args = (FAKE, FAKE, FAKE, None, FAKE, B.SEER_F32, None, None, FAKE, need, None)
    assert lib.seer_decode_attn_fwd(ctypes.byref(big), *args) == B.SEER_ERR_UNSUPPORTED
    assert lib.seer_decode_attn_fwd(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, B.SEER_F32, None, FAKE, FAKE,
                                    need, None) == B.SEER_ERR_INVALID_ARG          # gt with a mask
    assert lib.seer_decode_attn_fwd(ctypes.byref(s), FAKE, FAKE, FAKE, None, FAKE, B.SEER_F32, None, None, FAKE,
                                    need - 1, None) == B.SEER_ERR_WORKSPACE
    # partials: one (D + 2)-float record per query head and key split (padded
    # to 16 bytes), then per KV head a compacted list of the 16 blocks and its count
    lists = 2 * (16 + 1) * 4
    part = need - lists
    splits = part // (4 * 4 * (128 + 2))
    assert part == (4 * 4 * splits * (128 + 2) + 15) // 16 * 16 and 1 <= splits <= 16


def test_varlen_validation_and_sizes():
    lib = _lib()
    V = B.make_varlen
    assert lib.seer_varlen_map_elements(ctypes.byref(V([0, 100, 300, 300, 1000], 4, 2, 128))) == 4 * (4 + 16 + 0 + 121)
    bad = [V([1, 100], 4, 2, 128), V([0, 100, 50], 4, 2, 128)]
    for vl in bad:
        assert lib.seer_block_sparse_attn_varlen_fwd(ctypes.byref(vl), FAKE, FAKE, FAKE, None, FAKE, B.SEER_F32,
                                                     None, None, 0, None) == B.SEER_ERR_SHAPE
    assert lib.seer_block_sparse_attn_varlen_fwd(None, FAKE, FAKE, FAKE, None, FAKE, B.SEER_F32, None, None, 0,
                                                 None) == B.SEER_ERR_INVALID_ARG
    # the workspace is the largest one sequence needs
    vl = V([0, 64 * 1100, 64 * 1100 + 500], 4, 2, 128)
    one = lib.seer_attn_workspace_size(ctypes.byref(_shape(b=1, hq=4, hkv=2, s=64 * 1100, d=128)))
    assert one > 0 and lib.seer_attn_varlen_workspace_size(ctypes.byref(vl)) == one
    assert lib.seer_block_sparse_attn_varlen_fwd(ctypes.byref(vl), FAKE, FAKE, FAKE, FAKE, FAKE, B.SEER_F32, None,
                                                 FAKE, one - 1, None) == B.SEER_ERR_WORKSPACE
    # the ground-truth map runs both sequences in one launch: the scratch of both
    # ([Hq][nb(nb+1)/2][64] fp32 each), rounded up to 256 bytes
    raw = sum(4 * (nb * (nb + 1) // 2) * 64 * 4 for nb in (1100, 8))
    assert lib.seer_gt_varlen_workspace_size(ctypes.byref(vl)) == (raw + 255) // 256 * 256
    g1 = lib.seer_gt_workspace_size(ctypes.byref(_shape(b=1, hq=4, hkv=2, s=64 * 1100, d=128)))
    assert lib.seer_gt_varlen_workspace_size(ctypes.byref(vl)) > g1
    # nothing is enqueued when a later sequence is invalid: a bad head_dim fails before any launch
    assert lib.seer_gate_varlen_fwd(ctypes.byref(V([0, 64, 128], 4, 2, 96)), 128, 0, 0.0, FAKE, FAKE, FAKE, FAKE,
                                    B.SEER_MASK_THRESHOLD, 0.1, 1, None, None, FAKE, FAKE, 1 << 40,
                                    None) == B.SEER_ERR_UNSUPPORTED
    # an all-empty batch is a no-op
    assert lib.seer_block_sparse_attn_varlen_fwd(ctypes.byref(V([0, 0, 0], 4, 2, 128)), None, None, None, None,
                                                 None, B.SEER_F32, None, None, 0, None) == B.SEER_OK


def test_varlen_gate_workspace():
    """The packed gate runs consecutive sequences of up to 4096 blocks in one
    launch per stage: its workspace holds a run's pooled, projected (and,
    without scores, logits) parts side by side; a longer sequence runs alone
    and needs its own batch-1 workspace."""
    lib = _lib()
    hq, hkv, d, dg = 32, 8, 128, 128
    al = lambda n: (n + 255) // 256 * 256
    nbs = [32, 32, 30]
    vl = B.make_varlen([0, 2048, 4096, 4096, 6000], hq, hkv, d)     # an empty sequence inside the run
    inter = al(hq * d * 4 * sum(nbs)) + al(hkv * 3 * d * 4 * sum(nbs)) + 2 * al(hq * dg * 4 * sum(nbs))
    assert lib.seer_gate_varlen_workspace_size(ctypes.byref(vl), dg, 0, 1) == inter
    assert lib.seer_gate_varlen_workspace_size(ctypes.byref(vl), dg, 0, 0) == inter + al(hq * sum(n * n for n in nbs) * 4)
    # a sequence of 4097 blocks ends the run and runs on its own
    long_len = 64 * 4097
    vl2 = B.make_varlen([0, 2048, 2048 + long_len, 2 * 2048 + long_len], hq, hkv, d)
    one = lib.seer_gate_workspace_size(ctypes.byref(_shape(b=1, hq=hq, hkv=hkv, s=long_len, d=d)), dg, 0, 0)
    assert lib.seer_gate_varlen_workspace_size(ctypes.byref(vl2), dg, 0, 0) == one
    # too small a workspace is refused before any launch
    need = lib.seer_gate_varlen_workspace_size(ctypes.byref(vl), dg, 0, 0)
    assert lib.seer_gate_varlen_fwd(ctypes.byref(vl), dg, 0, 0.0, FAKE, FAKE, FAKE, FAKE, B.SEER_MASK_THRESHOLD,
                                    0.1, 1, None, None, FAKE, FAKE, need - 256, None) == B.SEER_ERR_WORKSPACE


def test_gate_validation():
    s = _shape()
    assert _gate(s, dg=100) == B.SEER_ERR_UNSUPPORTED
    assert _gate(s, dg=512) == B.SEER_ERR_UNSUPPORTED
    assert _gate(s, mode=5) == B.SEER_ERR_INVALID_ARG
    assert _gate(s, T=math.nan) == B.SEER_ERR_INVALID_ARG
    assert _gate(s, T=math.inf) == B.SEER_ERR_INVALID_ARG
    assert _gate(s, mode=B.SEER_MASK_TOPK, k=0) == B.SEER_ERR_INVALID_ARG
    ph = (ctypes.c_int32 * 4)(3, 3, 0, 3)
    assert _gate(s, mode=B.SEER_MASK_TOPK, per_head=ph) == B.SEER_ERR_INVALID_ARG
    assert b"head 2" in _lib().seer_last_error()
    assert _gate(s, mask=None) == B.SEER_ERR_INVALID_ARG
    assert _gate(s, ws=None) == B.SEER_ERR_WORKSPACE
    need = _lib().seer_gate_workspace_size(ctypes.byref(s), 128, 0, 0)
    assert _gate(s, ws_bytes=need - 1) == B.SEER_ERR_WORKSPACE
    big = _shape(s=64 * 16385)
    assert _gate(big) == B.SEER_ERR_UNSUPPORTED


def test_gt_validation():
    s = _shape()
    lib = _lib()
    need = lib.seer_gt_workspace_size(ctypes.byref(s))
    assert lib.seer_attn_maxpool_gt(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, B.SEER_F32, None, None, FAKE, need,
                                    None) == B.SEER_ERR_INVALID_ARG
    assert lib.seer_attn_maxpool_gt(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, B.SEER_F32, None, FAKE, FAKE,
                                    need - 1, None) == B.SEER_ERR_WORKSPACE


def test_workspace_sizes():
    lib = _lib()
    s = _shape(b=2, hq=4, hkv=2, s=200, d=64)
    nb = 4
    align = lambda x: (x + 255) // 256 * 256
    # every row within one key chunk; 8 heads over the 8 XCDs: the per-XCD
    # counts of the XCD-major order (8 ints in 256 bytes)
    assert lib.seer_attn_workspace_size(ctypes.byref(s)) == 256
    for b0, hq0, s0, d0 in ((1, 12, 200, 64), (1, 8, 64 * 257, 128), (1, 8, 64 * 513, 64)):
        assert lib.seer_attn_workspace_size(ctypes.byref(_shape(b=b0, hq=hq0, hkv=hq0 // 4, s=s0, d=d0))) == 0
    assert lib.seer_attn_workspace_size(ctypes.byref(_shape(b=1, hq=8, hkv=2, s=64 * 256, d=128))) == 256
    assert lib.seer_attn_workspace_size(ctypes.byref(_shape(b=1, hq=8, hkv=2, s=64 * 512, d=64))) == 256
    # one-item rows over 256 blocks at D = 128 with >= 8 rows per resident
    # workgroup (8 x 1024): the persistent launch's 8 queue counters
    assert lib.seer_attn_workspace_size(ctypes.byref(_shape(b=1, hq=32, hkv=8, s=64 * 300, d=128))) == 256
    assert lib.seer_attn_workspace_size(ctypes.byref(_shape(b=1, hq=32, hkv=8, s=64 * 959, d=128))) == 256
    assert lib.seer_attn_workspace_size(ctypes.byref(_shape(b=1, hq=8, hkv=2, s=64 * 300, d=128))) == 0
    assert lib.seer_attn_workspace_size(ctypes.byref(_shape(b=1, hq=32, hkv=8, s=64 * 600, d=64))) == 0
    # rows of more than 1024 blocks are cut into key chunks of 512 blocks: chunk
    # c holds the rows with query block >= 512 c (1100 + 588 + 76 rows per query
    # head); each (row, chunk) item reserves a 64 x (D + 1) fp32 partial
    s2 = _shape(b=2, hq=4, hkv=2, s=64 * 1100, d=128)
    assert lib.seer_attn_workspace_size(ctypes.byref(s2)) == 2 * 4 * (1100 + 588 + 76) * 64 * 129 * 4
    s3 = _shape(b=1, hq=2, hkv=1, s=64 * 1024, d=64)
    assert lib.seer_attn_workspace_size(ctypes.byref(s3)) == 0
    s4 = _shape(b=1, hq=2, hkv=1, s=64 * 1024 + 1, d=64)
    assert lib.seer_attn_workspace_size(ctypes.byref(s4)) == 2 * (1025 + 513 + 1) * 64 * 65 * 4
    # rows of >= 960 blocks with >= 64 (batch, KV group, 128-block chunk) jobs
    # take the XCD-owned path: rows qb >= 128 own qb // 128 + 1 slots of a
    # 64 x D bf16 partial and 64 fp32 log-sum-exps; 256 bytes of item counters
    for nb5, d5 in ((1300, 128), (2048, 64), (960, 128), (1024, 128)):
        s5 = _shape(b=1, hq=16, hkv=8, s=64 * nb5 - 3, d=d5)
        slots = sum(q // 128 + 1 for q in range(128, nb5))
        assert lib.seer_attn_workspace_size(ctypes.byref(s5)) == 16 * slots * 64 * (2 * d5 + 4) + 256
    s6 = _shape(b=1, hq=4, hkv=2, s=64 * 1300, d=128)             # 2 x 11 jobs: the other path
    assert lib.seer_attn_workspace_size(ctypes.byref(s6)) == 4 * (1300 + 788 + 276) * 64 * 129 * 4
    assert lib.seer_gt_workspace_size(ctypes.byref(s)) == align(2 * 4 * (nb * (nb + 1) // 2) * 64 * 4)
    want = (align(2 * 4 * nb * 64 * 4) + align(2 * 2 * nb * 192 * 4) + align(2 * 4 * nb * 32 * 4)
            + align(2 * 4 * nb * 32 * 4))
    assert lib.seer_gate_workspace_size(ctypes.byref(s), 32, 0, 1) == want
    assert lib.seer_gate_workspace_size(ctypes.byref(s), 32, 0, 0) == want + align(2 * 4 * nb * nb * 4)
    want_kv = (align(2 * 4 * nb * 64 * 4) + align(2 * 2 * nb * 192 * 4) + align(2 * 4 * nb * 32 * 4)
               + align(2 * 2 * nb * 32 * 4))
    assert lib.seer_gate_workspace_size(ctypes.byref(s), 32, 1, 1) == want_kv
