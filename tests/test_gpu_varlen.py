"""GPU parity of varlen (packed, unpadded) prefill batches: gate, block-sparse
and dense attention and the 2D-maxpooled map, each sequence against the fp64
oracle on that sequence alone, and bitwise against the batch-1 calls."""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth import Shape
from gpu_util import MASK_BAND, check_close, check_lse, dev_bf16, dev_f32, dev_u8, host, say

pytestmark = pytest.mark.gpu

HQ, HKV = 4, 2


def _seer():
    import learned_block_sparse_attngate_amd as seer
    seer.load_library()
    return seer


def _pack(lens, D, seed, hq=HQ, hkv=HKV):
    """Per-sequence bf16 q, k, v ([1, H, len, D]) and their packed [H, T, D] forms."""
    seqs = []
    for i, n in enumerate(lens):
        if n == 0:
            seqs.append(None)
            continue
        q, k, v = synth.gen_qkv(Shape(1, hq, hkv, n, D), seed + i)
        seqs.append((q, k, v))
    def cat(idx, H):
        parts = [s[idx][0] for s in seqs if s is not None]
        return np.ascontiguousarray(np.concatenate(parts, axis=1)) if parts else np.zeros((H, 0, D), np.uint16)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(int).tolist()
    return seqs, cat(0, hq), cat(1, hkv), cat(2, hkv), cu


def _masks(lens, seed, p):
    rng = np.random.default_rng(seed)
    out = []
    for n in lens:
        nb = synth.Shape(1, HQ, HKV, max(n, 1), 64).nb if n else 0
        m = (rng.random((HQ, nb, nb)) < p).astype(np.uint8)
        if nb:
            m[:, np.arange(nb), np.arange(nb)] = 1
        out.append(m)
    return out


LENS = [1, 130, 0, 1000, 64 * 20 - 5, 64]


@pytest.mark.parametrize("D,dt", [(128, torch.float32), (64, torch.bfloat16)], ids=["d128_f32", "d64_bf16"])
def test_varlen_sparse_and_dense_attention(D, dt):
    seer = _seer()
    seqs, qp, kp, vp, cu = _pack(LENS, D, 100 + D)
    say(f"[varlen attn D={D}] lens={LENS}")
    masks = _masks(LENS, 7, 0.4)
    flat = np.concatenate([m.reshape(-1) for m in masks])
    dq, dk, dv = dev_bf16(qp), dev_bf16(kp), dev_bf16(vp)
    out, lse = seer.seer_block_sparse_attn_varlen_fwd(dq, dk, dv, cu, dev_u8(flat), out_dtype=dt, want_lse=True)
    outd, lsed = seer.seer_block_sparse_attn_varlen_fwd(dq, dk, dv, cu, None, out_dtype=dt, want_lse=True)
    torch.cuda.synchronize()
    o_h, l_h, od_h, ld_h = host(out), host(lse), host(outd), host(lsed)
    for i, n in enumerate(LENS):
        if n == 0:
            continue
        q, k, v = seqs[i]
        a, b = cu[i], cu[i + 1]
        o_ref, l_ref = oracle.attention(q, k, v, masks[i][None])
        check_close(o_h[:, a:b][None], o_ref, f"seq {i} sparse O", out_dtype=dt)
        check_lse(l_h[:, a:b][None], l_ref, f"seq {i} sparse LSE")
        od_ref, ld_ref = oracle.attention(q, k, v, None)
        check_close(od_h[:, a:b][None], od_ref, f"seq {i} dense O", out_dtype=dt)
        # the batch-1 call on the sequence alone gives the same bits
        o1, l1 = seer.seer_block_sparse_attn_fwd(dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_u8(masks[i][None]),
                                                 out_dtype=dt, want_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(o1[0], out[:, a:b]) and torch.equal(l1[0], lse[:, a:b])


def test_varlen_long_sequence_key_chunks():
    """A sequence above 1024 blocks (key-chunked, with a workspace) packed with a short one."""
    seer = _seer()
    lens = [64 * 1100 - 30, 3000]
    seqs, qp, kp, vp, cu = _pack(lens, 64, 300)
    say(f"[varlen long] lens={lens}")
    masks = [synth.gen_block_mask(Shape(1, HQ, HKV, n, 64), 301 + i, 0.9).mask[0] for i, n in enumerate(lens)]
    flat = np.concatenate([m.reshape(-1) for m in masks])
    out, lse = seer.seer_block_sparse_attn_varlen_fwd(dev_bf16(qp), dev_bf16(kp), dev_bf16(vp), cu, dev_u8(flat),
                                                      out_dtype=torch.float32, want_lse=True)
    torch.cuda.synchronize()
    q, k, v = seqs[0]
    nb = (lens[0] + 63) // 64
    rows = [(0, h, i) for h in range(HQ) for i in (0, 511, 512, 1023, 1024, nb - 1)]
    o_ref, l_ref = oracle.attention_rows(q, k, v, masks[0][None], rows)
    o_h, l_h = host(out), host(lse)
    got = np.concatenate([o_h[h, 64 * i:64 * i + 64][: len(o_ref[n])] for n, (_, h, i) in enumerate(rows)])
    got_l = np.concatenate([l_h[h, 64 * i:64 * i + 64][: len(l_ref[n])] for n, (_, h, i) in enumerate(rows)])
    check_close(got, np.concatenate(o_ref), "long seq O (sampled)")
    check_lse(got_l, np.concatenate(l_ref), "long seq LSE (sampled)")
    q2, k2, v2 = seqs[1]
    o2, _ = oracle.attention(q2, k2, v2, masks[1][None])
    check_close(o_h[:, cu[1]:cu[2]][None], o2, "short seq O")


def test_varlen_long_sequence_xcd_path():
    """A sequence of 1300 blocks with 8 KV heads (the XCD-owned path: 128-block
    chunks, per-XCD item counters, bf16 partials) packed after a short one, so
    the long sequence's rows start at a nonzero packed offset."""
    seer = _seer()
    hq = hkv = 8
    lens = [2000, 64 * 1300 - 9]
    seqs, qp, kp, vp, cu = _pack(lens, 64, 310, hq, hkv)
    say(f"[varlen xcd] lens={lens}")
    masks = [synth.gen_block_mask(Shape(1, hq, hkv, n, 64), 311 + i, 0.9).mask[0] for i, n in enumerate(lens)]
    flat = np.concatenate([m.reshape(-1) for m in masks])
    out, lse = seer.seer_block_sparse_attn_varlen_fwd(dev_bf16(qp), dev_bf16(kp), dev_bf16(vp), cu, dev_u8(flat),
                                                      out_dtype=torch.float32, want_lse=True)
    torch.cuda.synchronize()
    o_h, l_h = host(out), host(lse)
    q, k, v = seqs[1]
    nb = (lens[1] + 63) // 64
    rows = [(0, h, i) for h in (0, 5, 7) for i in (0, 127, 128, 129, 640, 1279, 1280, nb - 1)]
    o_ref, l_ref = oracle.attention_rows(q, k, v, masks[1][None], rows)
    base = cu[1]
    got = np.concatenate([o_h[h, base + 64 * i:base + 64 * i + 64][: len(o_ref[n])] for n, (_, h, i) in enumerate(rows)])
    got_l = np.concatenate([l_h[h, base + 64 * i:base + 64 * i + 64][: len(l_ref[n])]
                            for n, (_, h, i) in enumerate(rows)])
    check_close(got, np.concatenate(o_ref), "xcd long seq O (sampled)")
    check_lse(got_l, np.concatenate(l_ref), "xcd long seq LSE (sampled)")
    q0, k0, v0 = seqs[0]
    o0, _ = oracle.attention(q0, k0, v0, masks[0][None])
    check_close(o_h[:, cu[0]:cu[1]][None], o0, "short seq O")


def test_varlen_gate_one_launch_equals_batch1():
    """The packed gate runs up to 64 consecutive sequences per launch of each
    stage (a sequence of more than 4096 blocks on its own launches): every
    sequence's scores and mask are bitwise those of its batch-1 call, with and
    without a scores output, in top-k mode with block RoPE and in threshold
    mode. 69 sequences, empty ones among them: two shared runs around the long
    one."""
    seer = _seer()
    hq, hkv, D, dg = 2, 1, 64, 64
    rng = np.random.default_rng(410)
    lens = [int(x) for x in rng.integers(1, 64 * 40, size=69)]
    lens[5] = 0
    lens[40] = 64 * 4097 + 3                      # past the register-resident row length
    lens[41] = 0
    say(f"[varlen gate one launch] {len(lens)} sequences, {sum(lens)} tokens")
    _, qp, kp, _, cu = _pack(lens, D, 420, hq, hkv)
    wq, wk = synth.gen_gate_weights(hq, D, dg, 421, var=4.0 / dg)
    q_d, k_d, wq_d, wk_d = dev_bf16(qp), dev_bf16(kp), dev_f32(wq), dev_f32(wk)
    offs, n_map = seer.varlen_map_offsets(cu, hq)
    for kw in (dict(mode="topk", topk=[5, 2], rope_theta=5e5), dict(mode="threshold", threshold=0.02)):
        m, s = seer.seer_gate_varlen_fwd(q_d, k_d, wq_d, wk_d, cu, **kw)
        m2, s2 = seer.seer_gate_varlen_fwd(q_d, k_d, wq_d, wk_d, cu, want_scores=False, **kw)
        torch.cuda.synchronize()
        assert s2 is None and m.numel() == n_map
        assert torch.equal(m, m2), f"{kw['mode']}: mask without scores differs"
        for i, n in enumerate(lens):
            if n == 0:
                continue
            nb = (n + 63) // 64
            q1 = q_d[:, cu[i]:cu[i + 1]].unsqueeze(0).contiguous()
            k1 = k_d[:, cu[i]:cu[i + 1]].unsqueeze(0).contiguous()
            mb, sb = seer.seer_gate_fwd(q1, k1, wq_d, wk_d, **kw)
            sl = slice(offs[i], offs[i] + hq * nb * nb)
            assert torch.equal(m[sl].view(1, hq, nb, nb), mb), f"{kw['mode']}: seq {i} mask"
            assert torch.equal(s[sl].view(1, hq, nb, nb), sb), f"{kw['mode']}: seq {i} scores"
        say(f"  {kw['mode']}: {int(m.sum())} active blocks, every sequence bitwise equal to its batch-1 call")


def test_varlen_gate_and_gt():
    seer = _seer()
    lens = [640, 0, 64 * 30 - 7, 65]
    D, dg = 128, 128
    seqs, qp, kp, vp, cu = _pack(lens, D, 400)
    wq, wk = synth.gen_gate_weights(HQ, D, dg, 401, var=4.0 / dg)
    offs, n_map = seer.varlen_map_offsets(cu, HQ)
    mask, scores = seer.seer_gate_varlen_fwd(dev_bf16(qp), dev_bf16(kp), dev_f32(wq), dev_f32(wk), cu,
                                             mode="topk", topk=3, rope_theta=5e5)
    _, _, gt = seer.seer_attn_maxpool_gt_varlen(dev_bf16(qp), dev_bf16(kp), dev_bf16(vp), cu, out_dtype=torch.float32)
    torch.cuda.synchronize()
    m_h, s_h, g_h = mask.cpu().numpy(), host(scores), host(gt)
    assert m_h.size == n_map
    for i, n in enumerate(lens):
        if n == 0:
            continue
        q, k, v = seqs[i]
        nb = (n + 63) // 64
        sl = slice(offs[i], offs[i] + HQ * nb * nb)
        sc_ref = oracle.gate_scores(q, k, wq, wk, rope_theta=5e5)[0]
        s_i = s_h[sl].reshape(HQ, nb, nb)
        assert np.abs(s_i - sc_ref).max() < 1e-5
        want = oracle.topk_mask(sc_ref[None], 3)[0]
        got = m_h[sl].reshape(HQ, nb, nb)
        bad = 0
        for h in range(HQ):
            for r in range(nb):
                kk = min(3, r + 1)
                assert int(got[h, r].sum()) == kk
                row = sc_ref[h, r, :r + 1]
                kth = np.sort(row)[::-1][kk - 1]
                bad += int(((got[h, r, :r + 1] != want[h, r, :r + 1]) & (np.abs(row - kth) > MASK_BAND)).sum())
        say(f"  seq {i}: gate top-3 mismatches outside the band {bad}")
        assert bad == 0
        gt_ref = oracle.maxpool_gt(q, k)[0]
        err = np.abs(g_h[sl].reshape(HQ, nb, nb) - gt_ref).max()
        say(f"  seq {i}: gt max-abs {err:.3e}")
        assert err <= 1e-6


def test_varlen_many_sequences_shared_launches():
    """70 packed sequences (more than one shared launch of 64; lengths from 0 to
    ~3k tokens in scrambled order): block-sparse, dense and the 2D map, every
    sequence bitwise equal to its batch-1 call, and a few against the oracle."""
    seer = _seer()
    rng = np.random.default_rng(320)
    lens = [int(x) for x in rng.integers(1, 3200, size=70)]
    lens[3] = 0
    lens[10] = 1
    lens[11] = 64
    lens[40] = 65
    D = 64
    seqs, qp, kp, vp, cu = _pack(lens, D, 330)
    say(f"[varlen many] {len(lens)} sequences, {cu[-1]} tokens")
    masks = [synth.gen_tiny_mask(Shape(1, HQ, HKV, max(n, 1), D), 340 + i, p_keep=0.3).mask[0] if n else
             np.zeros((HQ, 0, 0), np.uint8) for i, n in enumerate(lens)]
    flat = np.concatenate([m.reshape(-1) for m in masks])
    dq, dk, dv = dev_bf16(qp), dev_bf16(kp), dev_bf16(vp)
    out, lse = seer.seer_block_sparse_attn_varlen_fwd(dq, dk, dv, cu, dev_u8(flat), out_dtype=torch.float32,
                                                      want_lse=True)
    outd, lsed = seer.seer_block_sparse_attn_varlen_fwd(dq, dk, dv, cu, None, out_dtype=torch.bfloat16,
                                                        want_lse=True)
    og, lg, gt = seer.seer_attn_maxpool_gt_varlen(dq, dk, dv, cu, out_dtype=torch.float32, want_lse=True)
    torch.cuda.synchronize()
    offs, _ = seer.varlen_map_offsets(cu, HQ)
    for i, n in enumerate(lens):
        if n == 0:
            continue
        q, k, v = seqs[i]
        a, b = cu[i], cu[i + 1]
        nb = (n + 63) // 64
        q1, k1, v1 = dev_bf16(q), dev_bf16(k), dev_bf16(v)
        o1, l1 = seer.seer_block_sparse_attn_fwd(q1, k1, v1, dev_u8(masks[i][None]), out_dtype=torch.float32,
                                                 want_lse=True)
        od1, ld1 = seer.seer_block_sparse_attn_fwd(q1, k1, v1, None, out_dtype=torch.bfloat16, want_lse=True)
        og1, lg1, g1 = seer.seer_attn_maxpool_gt(q1, k1, v1, out_dtype=torch.float32, want_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(o1[0], out[:, a:b]) and torch.equal(l1[0], lse[:, a:b]), f"seq {i} sparse"
        assert torch.equal(od1[0], outd[:, a:b]) and torch.equal(ld1[0], lsed[:, a:b]), f"seq {i} dense"
        assert torch.equal(og1[0], og[:, a:b]) and torch.equal(lg1[0], lg[:, a:b]), f"seq {i} gt-kernel O"
        assert torch.equal(g1.reshape(-1), gt[offs[i]:offs[i] + HQ * nb * nb]), f"seq {i} map"
        if i % 17 == 0:
            o_ref, l_ref = oracle.attention(q, k, v, masks[i][None])
            check_close(host(out[:, a:b])[None], o_ref, f"seq {i} sparse O")
            check_lse(host(lse[:, a:b])[None], l_ref, f"seq {i} sparse LSE")
            g_ref = oracle.maxpool_gt(q, k)[0]
            err = np.abs(host(gt[offs[i]:offs[i] + HQ * nb * nb]).reshape(HQ, nb, nb) - g_ref).max()
            say(f"  seq {i}: gt max-abs {err:.3e}")
            assert err <= 1e-6
    say("  every sequence bitwise equal to its batch-1 call (sparse, dense, map)")
