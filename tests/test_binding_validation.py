"""The Python binding validates every tensor before a pointer reaches the C ABI.

The C calls take raw pointers and trust their extents, so a short K/V cache,
a small output or a wrong dtype would make the kernels read or write past an
allocation. These CPU tests use `meta` tensors (shape and dtype only, no
memory): every malformed case must raise TypeError / ValueError from the
binding, and a well-formed call on non-GPU tensors must still raise before
anything is launched.
"""
import pytest
import torch

import learned_block_sparse_attngate_amd as seer

META = torch.device("meta")
B, HQ, HKV, S, D, DG = 1, 4, 2, 300, 128, 64
NB = -(-S // 64)


def t(*shape, dtype=torch.bfloat16):
    return torch.empty(shape, dtype=dtype, device=META)


def qkv():
    return t(B, HQ, S, D), t(B, HKV, S, D), t(B, HKV, S, D)


def gate_w(per_kv=False):
    return t(HQ, D, DG, dtype=torch.float32), t(HKV if per_kv else HQ, 3 * D, DG, dtype=torch.float32)


def raises(exc, fn, *a, **kw):
    with pytest.raises(exc):
        fn(*a, **kw)


def test_attention_inputs():
    q, k, v = qkv()
    raises(TypeError, seer.seer_block_sparse_attn_fwd, q, k, v)                      # not on a GPU
    raises(ValueError, seer.seer_block_sparse_attn_fwd, q, t(B, HKV, S - 1, D), v)    # short K
    raises(ValueError, seer.seer_block_sparse_attn_fwd, q, k, t(B, HKV, S - 64, D))   # short V
    raises(ValueError, seer.seer_block_sparse_attn_fwd, q, k, t(B, HKV, S, 64))       # V head dim
    raises(ValueError, seer.seer_block_sparse_attn_fwd, q, t(2, HKV, S, D), t(2, HKV, S, D))   # batch
    raises(ValueError, seer.seer_block_sparse_attn_fwd, q, t(B, 3, S, D), t(B, 3, S, D))       # 4 % 3 heads
    raises(ValueError, seer.seer_block_sparse_attn_fwd, t(HQ, S, D), k, v)            # rank
    raises(TypeError, seer.seer_block_sparse_attn_fwd, q.float(), k, v)               # dtype
    raises(TypeError, seer.seer_block_sparse_attn_fwd, q, k.half(), v)
    raises(ValueError, seer.seer_block_sparse_attn_fwd, q, k.transpose(2, 3).contiguous().transpose(2, 3), v)


def test_attention_mask_and_outputs():
    q, k, v = qkv()
    good = t(B, HQ, NB, NB, dtype=torch.uint8)
    raises(ValueError, seer.seer_block_sparse_attn_fwd, q, k, v, t(B, HQ, NB - 1, NB, dtype=torch.uint8))
    raises(TypeError, seer.seer_block_sparse_attn_fwd, q, k, v, t(B, HQ, NB, NB, dtype=torch.bool))
    raises(TypeError, seer.seer_block_sparse_attn_fwd, q, k, v, good, out=t(B, HQ, S, D, dtype=torch.float16))
    raises(TypeError, seer.seer_block_sparse_attn_fwd, q, k, v, good, out_dtype=torch.float16)
    raises(ValueError, seer.seer_block_sparse_attn_fwd, q, k, v, good, out=t(B, HQ, S - 1, D, dtype=torch.float32))
    raises(ValueError, seer.seer_block_sparse_attn_fwd, q, k, v, good, lse=t(B, HQ, S - 1, dtype=torch.float32))
    raises(TypeError, seer.seer_block_sparse_attn_fwd, q, k, v, good, lse=t(B, HQ, S, dtype=torch.bfloat16))
    raises(TypeError, seer.seer_block_sparse_attn_fwd, q, k, v, good, out=t(B, HQ, S, D, dtype=torch.float32),
           lse=t(B, HQ, S, dtype=torch.float32))                                   # well formed, not on a GPU


def test_ground_truth_outputs():
    q, k, v = qkv()
    raises(ValueError, seer.seer_attn_maxpool_gt, q, k, t(B, HKV, S, 64))
    raises(ValueError, seer.seer_attn_maxpool_gt, q, k, v, gt=t(B, HQ, NB, NB - 1, dtype=torch.float32))
    raises(TypeError, seer.seer_attn_maxpool_gt, q, k, v, gt=t(B, HQ, NB, NB, dtype=torch.float16))
    raises(TypeError, seer.seer_attn_maxpool_gt, q, k, v, out=t(B, HQ, S, D, dtype=torch.float16))
    raises(TypeError, seer.seer_attn_maxpool_gt, q, k, v, gt=t(B, HQ, NB, NB, dtype=torch.float32))


def test_gate_inputs_and_outputs():
    q, k, _ = qkv()
    wq, wk = gate_w()
    raises(ValueError, seer.seer_gate_fwd, q, k, wq, t(HQ, 2 * D, DG, dtype=torch.float32))   # W_k rows
    raises(ValueError, seer.seer_gate_fwd, q, k, wq, t(HKV, 3 * D, DG, dtype=torch.float32))  # per-KV W_k, flag off
    raises(ValueError, seer.seer_gate_fwd, q, k, t(HQ, D, DG + 16, dtype=torch.float32), wk)  # gate dims differ
    raises(TypeError, seer.seer_gate_fwd, q, k, wq.half(), wk)
    raises(ValueError, seer.seer_gate_fwd, q, t(B, HKV, S + 64, D), wq, wk)
    raises(ValueError, seer.seer_gate_fwd, q, k, wq, wk, block_mask=t(B, HQ, NB, NB + 1, dtype=torch.uint8))
    raises(ValueError, seer.seer_gate_fwd, q, k, wq, wk, scores=t(B, HQ - 1, NB, NB, dtype=torch.float32))
    raises(ValueError, seer.seer_gate_fwd, q, k, wq, wk, mode="topk")                          # no k
    raises(ValueError, seer.seer_gate_fwd, q, k, wq, wk, mode="topk", topk=[1, 2])             # per-head count
    raises(ValueError, seer.seer_gate_fwd, q, k, wq, wk, mode="bogus")
    wq2, wk2 = gate_w(per_kv=True)
    raises(TypeError, seer.seer_gate_fwd, q, k, wq2, wk2, wk_per_kv_head=True)                  # not on a GPU


def test_distillation_inputs():
    q, k, _ = qkv()
    wq, wk = gate_w()
    gt = t(B, HQ, NB, NB, dtype=torch.float32)
    raises(ValueError, seer.seer_gate_distill_bwd, q, k, wq, wk, t(B, HQ, NB - 1, NB - 1, dtype=torch.float32))
    raises(ValueError, seer.seer_gate_distill_bwd, q, k, wq, wk, gt, grad_wq=t(HQ, D, DG - 1, dtype=torch.float32))
    raises(ValueError, seer.seer_gate_distill_bwd, q, k, wq, wk, gt, grad_wk=t(HQ, D, DG, dtype=torch.float32))
    raises(ValueError, seer.seer_gate_distill_bwd, q, k, wq, wk, gt, loss=t(2, dtype=torch.float32))
    raises(TypeError, seer.seer_gate_distill_bwd, q, k, wq, wk, gt)


def test_decode_inputs():
    qd = t(B, HQ, D)
    kc, vc = t(B, HKV, S, D), t(B, HKV, S, D)
    raises(ValueError, seer.seer_decode_attn_fwd, qd, kc, t(B, HKV, S - 1, D))
    raises(ValueError, seer.seer_decode_attn_fwd, t(B, HQ, 64), kc, vc)
    raises(ValueError, seer.seer_decode_attn_fwd, qd, kc, vc, t(B, HQ, NB + 1, dtype=torch.uint8))
    raises(ValueError, seer.seer_decode_attn_fwd, qd, kc, vc, out=t(B, HQ - 1, D, dtype=torch.float32))
    raises(TypeError, seer.seer_decode_attn_fwd, qd, kc, vc, out=t(B, HQ, D, dtype=torch.float16))
    raises(ValueError, seer.seer_decode_attn_fwd, qd, kc, vc, gt=t(B, HQ, NB - 1, dtype=torch.float32))
    raises(TypeError, seer.seer_decode_attn_fwd, qd, kc, vc)
    wk = t(HQ, 3 * D, D, dtype=torch.float32)
    raises(ValueError, seer.seer_decode_compress_k, kc, t(HQ, 3 * D, DG, dtype=torch.float32), HQ)
    raises(ValueError, seer.seer_decode_compress_k, kc, wk, HQ, kcomp=t(B, HQ, NB, 64, dtype=torch.float32))
    raises(ValueError, seer.seer_decode_compress_k, kc, wk, 3)
    raises(TypeError, seer.seer_decode_compress_k, kc, wk, HQ)
    kcomp = t(B, HQ, NB, D, dtype=torch.float32)
    raises(ValueError, seer.seer_decode_gate_fwd, qd, t(B, HQ - 1, NB, D, dtype=torch.float32), S, HKV)
    raises(ValueError, seer.seer_decode_gate_fwd, qd, kcomp, S, HKV, scores=t(B, HQ, NB + 1, dtype=torch.float32))
    raises(ValueError, seer.seer_decode_gate_fwd, qd, kcomp, S, 3)
    raises(TypeError, seer.seer_decode_gate_fwd, qd, kcomp, S, HKV)


def test_varlen_inputs():
    cu = [0, 100, 300]
    T = cu[-1]
    q, k, v = t(HQ, T, D), t(HKV, T, D), t(HKV, T, D)
    _, n_map = seer.varlen_map_offsets(cu, HQ)
    raises(ValueError, seer.seer_block_sparse_attn_varlen_fwd, q, k, v, [0, 100, 299])
    raises(ValueError, seer.seer_block_sparse_attn_varlen_fwd, q, k, v, [0, 200, 100, 300])
    raises(ValueError, seer.seer_block_sparse_attn_varlen_fwd, q, t(HKV, T - 1, D), v, cu)
    raises(ValueError, seer.seer_block_sparse_attn_varlen_fwd, q, k, v, cu, t(n_map - 1, dtype=torch.uint8))
    raises(ValueError, seer.seer_block_sparse_attn_varlen_fwd, q, k, v, cu, out=t(HQ, T, 64, dtype=torch.float32))
    raises(TypeError, seer.seer_block_sparse_attn_varlen_fwd, q, k, v, cu, t(n_map, dtype=torch.uint8))
    raises(ValueError, seer.seer_attn_maxpool_gt_varlen, q, k, v, cu, gt=t(n_map + 1, dtype=torch.float32))
    raises(TypeError, seer.seer_attn_maxpool_gt_varlen, q, k, v, cu)
    wq, wk = gate_w()
    raises(ValueError, seer.seer_gate_varlen_fwd, q, k, wq, wk, cu, scores=t(n_map - 1, dtype=torch.float32))
    raises(TypeError, seer.seer_gate_varlen_fwd, q, k, wq, wk, cu)
