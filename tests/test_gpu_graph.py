"""HIP graph capture of the hot path: a decode step (compressed-K update,
decode gate, block-sparse decode attention) and prefill steps (gate, then
block-sparse attention on the XCD-owned persistent path, and on short rows in
the XCD-major order with its balance pre-pass) captured once and replayed
several times, with eager work between the replays; every replay
must give the eager call's bits (the kernels are deterministic and clear
their own counters with a kernel, not a memset)."""
import numpy as np
import pytest
import torch

import synth
from synth import Shape
from gpu_util import dev_bf16, dev_f32, say

pytestmark = pytest.mark.gpu


def _seer():
    import learned_block_sparse_attngate_amd as seer
    seer.load_library()
    return seer


def _replay_and_check(step, outs, label):
    step()
    torch.cuda.synchronize()
    refs = [o.clone() for o in outs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for r in range(3):
        for o in outs:
            o.zero_()
        graph.replay()
        torch.cuda.synchronize()
        for o, ref in zip(outs, refs):
            assert torch.equal(o, ref), f"{label}: replay {r} differs from the eager call"
        step()                                       # eager work between replays
        torch.cuda.synchronize()
        for o, ref in zip(outs, refs):
            assert torch.equal(o, ref), f"{label}: eager call after replay {r} differs"
    say(f"[graph {label}] 3 replays identical to eager")


def test_graph_decode_step():
    seer = _seer()
    shape = Shape(1, 32, 8, 64 * 1024, 128)
    say(f"[graph decode] shape={shape}")
    q, k, v = synth.gen_qkv(shape, 301)
    _, wk = synth.gen_gate_weights(shape.heads_q, shape.head_dim, shape.head_dim, 302)
    qd, kk, vv, wkd = dev_bf16(np.ascontiguousarray(q[:, :, -1])), dev_bf16(k), dev_bf16(v), dev_f32(wk)
    nb = shape.nb
    kc = seer.seer_decode_compress_k(kk, wkd, shape.heads_q)
    mask = torch.empty((1, shape.heads_q, nb), dtype=torch.uint8, device="cuda")
    scores = torch.empty((1, shape.heads_q, nb), dtype=torch.float32, device="cuda")
    out = torch.empty((1, shape.heads_q, shape.head_dim), dtype=torch.float32, device="cuda")
    ws = torch.empty(seer.decode_attn_workspace_bytes(1, shape.heads_q, shape.heads_kv, shape.seq_len, shape.head_dim),
                     dtype=torch.uint8, device="cuda")

    def step():
        seer.seer_decode_compress_k(kk, wkd, shape.heads_q, kcomp=kc, block_begin=nb - 1)
        seer.seer_decode_gate_fwd(qd, kc, shape.seq_len, shape.heads_kv, mode="topk", topk=nb // 10,
                                  scores=scores, block_mask=mask)
        seer.seer_decode_attn_fwd(qd, kk, vv, mask, out=out, workspace=ws)

    _replay_and_check(step, [mask, scores, out], "decode")


def test_graph_prefill_step_xcd_path():
    seer = _seer()
    shape = Shape(1, 16, 8, 64 * 1300, 64)            # 1300 blocks, 88 (KV group, chunk) jobs: XCD-owned path
    say(f"[graph prefill] shape={shape}")
    q, k, v = synth.gen_qkv(shape, 303)
    wq, wk = synth.gen_gate_weights(shape.heads_q, shape.head_dim, 64, 304)
    qq, kk, vv = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    wqd, wkd = dev_f32(wq), dev_f32(wk)
    nb = shape.nb
    mask = torch.empty((1, shape.heads_q, nb, nb), dtype=torch.uint8, device="cuda")
    scores = torch.empty((1, shape.heads_q, nb, nb), dtype=torch.float32, device="cuda")
    gws = torch.empty(seer.gate_workspace_bytes(1, shape.heads_q, shape.heads_kv, shape.seq_len, shape.head_dim, 64),
                      dtype=torch.uint8, device="cuda")
    out = torch.empty_like(qq)
    aws = torch.empty(max(seer.attn_workspace_bytes(1, shape.heads_q, shape.heads_kv, shape.seq_len, shape.head_dim), 16),
                      dtype=torch.uint8, device="cuda")

    def step():
        seer.seer_gate_fwd(qq, kk, wqd, wkd, rope_theta=500000.0, mode="topk", topk=nb // 10, scores=scores,
                           block_mask=mask, workspace=gws)
        seer.seer_block_sparse_attn_fwd(qq, kk, vv, mask, out=out, workspace=aws)

    _replay_and_check(step, [mask, scores, out], "prefill")


def test_graph_prefill_step_xcd_major_rows():
    """Short rows (128 blocks, 32 heads): the gate's uniform top-k mask gives
    every head the same work, so the pre-pass's per-XCD counts are balanced
    and the rows run in the XCD-major order; the counts are cleared by a
    kernel inside the captured step."""
    seer = _seer()
    shape = Shape(1, 32, 8, 8192, 128)
    say(f"[graph prefill xcd-major] shape={shape}")
    assert seer.attn_workspace_bytes(1, shape.heads_q, shape.heads_kv, shape.seq_len, shape.head_dim) == 256
    q, k, v = synth.gen_qkv(shape, 305)
    wq, wk = synth.gen_gate_weights(shape.heads_q, shape.head_dim, 128, 306)
    qq, kk, vv = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    wqd, wkd = dev_f32(wq), dev_f32(wk)
    nb = shape.nb
    mask = torch.empty((1, shape.heads_q, nb, nb), dtype=torch.uint8, device="cuda")
    gws = torch.empty(seer.gate_workspace_bytes(1, shape.heads_q, shape.heads_kv, shape.seq_len, shape.head_dim, 128,
                                                want_scores=False), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(qq)
    aws = torch.empty(256, dtype=torch.uint8, device="cuda")

    def step():
        seer.seer_gate_fwd(qq, kk, wqd, wkd, rope_theta=500000.0, mode="topk", topk=nb // 4, want_scores=False,
                           block_mask=mask, workspace=gws)
        seer.seer_block_sparse_attn_fwd(qq, kk, vv, mask, out=out, workspace=aws)

    _replay_and_check(step, [mask, out], "prefill xcd-major")
