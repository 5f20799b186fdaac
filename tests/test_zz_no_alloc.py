"""The allocation-free decode attention entry point (seer_decode_attn_fwd_noalloc),
called through the C ABI, against the workspace entry point seer_decode_attn_fwd:
two calls in a row on one device, the second with a smaller input, each equal
bit for bit to the workspace call on the same inputs (the same kernels run on
the library's fixed scratch instead of a caller workspace), and a shape whose
scratch exceeds the fixed size rejected before anything is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

import synth
from synth import Shape
from gpu_util import dev_bf16, dev_u8, say

pytestmark = pytest.mark.gpu


def _lib():
    import learned_block_sparse_attngate_amd as seer
    return seer, seer.load_library()


def _case(shape, seed, dens):
    q, k, v = synth.gen_qkv(shape, seed)
    qd = q[:, :, -1]                                     # the newest token's query per head
    rng = np.random.default_rng(seed + 1)
    mask = (rng.random((shape.batch, shape.heads_q, shape.nb)) < dens).astype(np.uint8)
    if shape.heads_q > 1:
        mask[0, 1, :] = 0                                # a head with no active block
    return dev_bf16(np.ascontiguousarray(qd)), dev_bf16(k), dev_bf16(v), dev_u8(mask)


def _noalloc(lib, seer, shape, q, k, v, mask, out_dtype, want_gt=False):
    """Direct C-ABI call; outputs allocated here by the test, none by the library."""
    B, Hq, S, D = shape.batch, shape.heads_q, shape.seq_len, shape.head_dim
    out = torch.full((B, Hq, D), float("nan"), dtype=out_dtype, device="cuda")
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda")
    gt = torch.full((B, Hq, shape.nb), float("nan"), dtype=torch.float32, device="cuda") if want_gt else None
    shp = seer.make_shape(B, Hq, shape.heads_kv, S, D)
    dt = seer.SEER_BF16 if out_dtype == torch.bfloat16 else seer.SEER_F32
    st = lib.seer_decode_attn_fwd_noalloc(ctypes.byref(shp), ctypes.c_void_p(q.data_ptr()),
                                          ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
                                          None if mask is None else ctypes.c_void_p(mask.data_ptr()),
                                          ctypes.c_void_p(out.data_ptr()), dt, ctypes.c_void_p(lse.data_ptr()),
                                          None if gt is None else ctypes.c_void_p(gt.data_ptr()),
                                          ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == seer.SEER_OK, lib.seer_last_error().decode()
    return out, lse, gt


def test_noalloc_matches_workspace_call_twice():
    seer, lib = _lib()
    # first a large call (sparse, bf16 out), then a smaller one (dense + 1D map, fp32 out):
    # the second reuses the scratch the first left behind
    cases = [(Shape(2, 32, 8, 64 * 700 - 9, 128), 0.3, None, torch.bfloat16),
             (Shape(1, 8, 2, 64 * 40 + 3, 64), None, True, torch.float32)]
    for n, (shape, dens, gt, dt) in enumerate(cases):
        say(f"[noalloc call {n}] shape={shape} mask={'dense' if dens is None else dens} out={dt}")
        q, k, v, mask = _case(shape, 500 + n, dens or 1.0)
        if dens is None:
            mask = None
        out_n, lse_n, gt_n = _noalloc(lib, seer, shape, q, k, v, mask, dt, want_gt=bool(gt))
        out_w, lse_w, gt_w = seer.seer_decode_attn_fwd(q, k, v, mask, out_dtype=dt, want_lse=True,
                                                       want_gt=bool(gt))
        torch.cuda.synchronize()
        assert torch.equal(out_n, out_w), "out differs from the workspace call"
        assert torch.equal(lse_n, lse_w), "lse differs from the workspace call"
        if gt:
            assert torch.equal(gt_n, gt_w), "1D map differs from the workspace call"
        assert torch.isfinite(out_n).all()
        say(f"  call {n}: out, lse{', gt' if gt else ''} bitwise equal to the workspace call")


def test_noalloc_rejects_shapes_beyond_scratch():
    seer, lib = _lib()
    shape = Shape(256, 32, 8, 64 * 2048, 128)            # needs about 48 MiB of scratch
    need = seer.decode_attn_workspace_bytes(shape.batch, shape.heads_q, shape.heads_kv, shape.seq_len,
                                            shape.head_dim)
    assert need > seer.NOALLOC_SCRATCH_BYTES
    shp = seer.make_shape(shape.batch, shape.heads_q, shape.heads_kv, shape.seq_len, shape.head_dim)
    fake = ctypes.c_void_p(1 << 40)                      # never dereferenced: rejected on the host
    st = lib.seer_decode_attn_fwd_noalloc(ctypes.byref(shp), fake, fake, fake, None, fake, seer.SEER_F32, None,
                                          None, None)
    assert st == seer.SEER_ERR_UNSUPPORTED
    assert "allocation-free" in lib.seer_last_error().decode()
