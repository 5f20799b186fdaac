"""GPU parity on seeded random shapes: batch, query / KV heads (GQA ratios 1 to
8), ragged sequence lengths, head dim 64 / 128, mask density (empty rows and
upper-triangle noise included) and output dtype drawn from one seeded
generator, checked against the fp64 oracle element by element (block-sparse
and dense attention with LSE, the gate's scores and threshold / top-k masks)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth import Shape
from gpu_util import MASK_BAND, check_close, check_lse, dev_bf16, dev_f32, dev_u8, host, say

pytestmark = pytest.mark.gpu


def _seer():
    import learned_block_sparse_attngate_amd as seer
    seer.load_library()
    return seer


def _draw_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        hkv = int(rng.choice([1, 2, 4]))
        g = int(rng.choice([1, 2, 4, 8]))
        b = int(rng.choice([1, 2]))
        d = int(rng.choice([64, 128]))
        s = int(rng.integers(1, 2600))
        p = float(rng.choice([0.05, 0.3, 0.7, 1.0]))
        dt = torch.float32 if rng.random() < 0.5 else torch.bfloat16
        cases.append((f"r{i}_b{b}_h{hkv * g}x{hkv}_s{s}_d{d}_p{p}", Shape(b, hkv * g, hkv, s, d), 500 + i, p, dt))
    return cases


CASES = _draw_cases(10, 2024)


def _mask(shape, seed, p):
    rng = np.random.default_rng(seed)
    nb = shape.nb
    m = (rng.random((shape.batch, shape.heads_q, nb, nb)) < p).astype(np.uint8)
    m = np.tril(m)
    m[0, 0, nb // 2, :] = 0                       # an empty row: O = 0, LSE = -inf
    return synth.gen_random_upper_noise(m, seed + 1)


@pytest.mark.parametrize("name,shape,seed,p,dt", CASES, ids=[c[0] for c in CASES])
def test_random_shape_attention(name, shape, seed, p, dt):
    seer = _seer()
    say(f"[random attention {name}] shape={shape} seed={seed} out={dt}")
    q, k, v = synth.gen_qkv(shape, seed)
    m = _mask(shape, seed, p)
    dq, dk, dv = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    out, lse = seer.seer_block_sparse_attn_fwd(dq, dk, dv, dev_u8(m), out_dtype=dt, want_lse=True)
    outd, lsed = seer.seer_block_sparse_attn_fwd(dq, dk, dv, None, out_dtype=dt, want_lse=True)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(q, k, v, m)
    check_close(host(out), o_ref, f"{name} sparse O", out_dtype=dt)
    check_lse(host(lse), l_ref, f"{name} sparse LSE")
    od_ref, ld_ref = oracle.attention(q, k, v, None)
    check_close(host(outd), od_ref, f"{name} dense O", out_dtype=dt)
    check_lse(host(lsed), ld_ref, f"{name} dense LSE")


@pytest.mark.parametrize("name,shape,seed,p,dt", CASES[:6], ids=[c[0] for c in CASES[:6]])
def test_random_shape_gate(name, shape, seed, p, dt):
    seer = _seer()
    rng = np.random.default_rng(seed)
    dg = int(rng.choice([16, 48, 128]))
    per_kv = bool(rng.random() < 0.5)
    say(f"[random gate {name}] shape={shape} dg={dg} per_kv={per_kv}")
    q, k, _, _ = synth.gen_planted_qk(shape, seed)
    hw = shape.heads_kv if per_kv else shape.heads_q
    wq, wk = synth.gen_gate_weights(shape.heads_q, shape.head_dim, dg, seed + 1, heads_w_k=hw)
    sc_ref = oracle.gate_scores(q, k, wq, wk, wk_per_kv_head=per_kv)
    nb = shape.nb
    T = 1.5 / nb
    mask, scores = seer.seer_gate_fwd(dev_bf16(q), dev_bf16(k), dev_f32(wq), dev_f32(wk), mode="threshold",
                                      threshold=T, wk_per_kv_head=per_kv)
    kk = int(rng.integers(1, nb + 2))
    mask_k, _ = seer.seer_gate_fwd(dev_bf16(q), dev_bf16(k), dev_f32(wq), dev_f32(wk), mode="topk", topk=kk,
                                   wk_per_kv_head=per_kv)
    torch.cuda.synchronize()
    assert np.abs(host(scores) - sc_ref).max() < 1e-5
    got = mask.cpu().numpy()
    want = oracle.threshold_mask(sc_ref, T)
    assert not ((got != want) & (np.abs(sc_ref - T) > MASK_BAND)).any()
    got_k = mask_k.cpu().numpy()
    want_k = oracle.topk_mask(sc_ref, kk)
    for b in range(shape.batch):
        for h in range(shape.heads_q):
            for i in range(nb):
                n = min(kk, i + 1)
                assert int(got_k[b, h, i].sum()) == n
                row = sc_ref[b, h, i, :i + 1]
                kth = np.partition(row, i + 1 - n)[i + 1 - n]
                outside = np.abs(row - kth) > MASK_BAND
                assert not ((got_k[b, h, i, :i + 1] != want_k[b, h, i, :i + 1]) & outside).any()


def _draw_long_cases(n, seed):
    """Rows long enough for the persistent row queues (257-1024 blocks at
    D = 128 with >= 8 rows per resident workgroup) or the XCD-major order
    (up to 256 blocks, batch x heads a multiple of 8)."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        hkv = int(rng.choice([2, 4, 8]))
        g = int(rng.choice([1, 2, 4]))
        b = int(rng.choice([1, 2]))
        long_rows = i % 2 == 0
        s = int(rng.integers(64 * 257, 64 * 1024 + 1)) if long_rows else int(rng.integers(64 * 64, 64 * 256 + 1))
        while long_rows and b * hkv * g * ((s + 63) // 64) < 8192:
            g *= 2
        while not long_rows and (b * hkv * g) % 8 != 0:
            g *= 2
        p = float(rng.choice([0.05, 0.1, 0.3]))
        dt = torch.float32 if rng.random() < 0.5 else torch.bfloat16
        cases.append((f"L{i}_b{b}_h{hkv * g}x{hkv}_s{s}_p{p}", Shape(b, hkv * g, hkv, s, 128), 700 + i, p, dt))
    return cases


LONG_CASES = _draw_long_cases(6, 2025)


@pytest.mark.parametrize("name,shape,seed,p,dt", LONG_CASES, ids=[c[0] for c in LONG_CASES])
def test_random_long_rows_attention(name, shape, seed, p, dt):
    """Random masks on the long-row schedules; sampled query blocks of every
    head against the oracle."""
    from gpu_util import sample_rows
    seer = _seer()
    say(f"[random long rows {name}] shape={shape} seed={seed} out={dt} "
        f"workspace={seer.attn_workspace_bytes(shape.batch, shape.heads_q, shape.heads_kv, shape.seq_len, 128)}")
    q, k, v = synth.gen_qkv(shape, seed)
    m = _mask(shape, seed, p)
    out, lse = seer.seer_block_sparse_attn_fwd(dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_u8(m), out_dtype=dt,
                                               want_lse=True)
    torch.cuda.synchronize()
    rows = sample_rows(shape.batch, shape.heads_q, shape.nb, 1, seed + 2)
    got = np.concatenate([host(out[b, h, 64 * i:64 * i + 64]) for (b, h, i) in rows])
    got_l = np.concatenate([host(lse[b, h, 64 * i:64 * i + 64]) for (b, h, i) in rows])
    o_ref, l_ref = oracle.attention_rows(q, k, v, m, rows)
    check_close(got, np.concatenate(o_ref), f"{name} O (sampled)", out_dtype=dt)
    check_lse(got_l, np.concatenate(l_ref), f"{name} LSE (sampled)")
