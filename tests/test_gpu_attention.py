"""GPU parity of the block-sparse / dense attention (C ABI via the binding)
against the fp64 oracle, element by element, on seeded inputs."""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth import Shape
from gpu_util import (check_close, check_lse, dev_bf16, dev_u8, host, say, sample_rows)

pytestmark = pytest.mark.gpu


def _seer():
    import learned_block_sparse_attngate_amd as seer
    seer.load_library()
    return seer


def _run_full(shape, seed, mask, out_dtype, what):
    seer = _seer()
    say(f"[{what}] shape={shape} seed={seed} mask={'dense' if mask is None else 'sparse'} out={out_dtype}")
    q, k, v = synth.gen_qkv(shape, seed)
    out, lse = seer.seer_block_sparse_attn_fwd(dev_bf16(q), dev_bf16(k), dev_bf16(v),
                                               None if mask is None else dev_u8(mask),
                                               out_dtype=out_dtype, want_lse=True)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(q, k, v, mask)
    check_close(host(out), o_ref, f"{what} O", out_dtype=out_dtype)
    check_lse(host(lse), l_ref, f"{what} LSE")
    return out, lse


CASES = [
    # name, shape, seed, mask kind, out dtype
    ("tiny_s512_c1", synth.WORKLOADS["tiny_s512"]["shape"], synth.WORKLOADS["tiny_s512"]["seed"], "workload", torch.float32),
    ("ragged_s200_d64", Shape(1, 4, 2, 200, 64), 31, "tiny_noise", torch.float32),
    ("ragged_s1000_d128", Shape(2, 4, 1, 1000, 128), 32, "p30_empty_noise", torch.bfloat16),
    ("s1_single_token", Shape(1, 2, 2, 1, 128), 33, "tiny", torch.float32),
    ("s65_two_blocks", Shape(1, 8, 8, 65, 64), 34, "tiny", torch.float32),
    ("s4096_d128_p20", Shape(1, 4, 1, 4096, 128), 35, "p20", torch.float32),
]


def _mask_for(kind, shape, seed):
    if kind == "workload":
        return synth.workload_mask("tiny_s512").mask
    if kind == "tiny":
        return synth.gen_tiny_mask(shape, seed + 1).mask
    if kind == "tiny_noise":
        return synth.gen_random_upper_noise(synth.gen_tiny_mask(shape, seed + 1, p_keep=0.5).mask, seed + 2)
    if kind == "p30_empty_noise":
        rng = np.random.Generator(np.random.PCG64(seed))
        nb = shape.nb
        m = (rng.random((shape.batch, shape.heads_q, nb, nb)) < 0.3).astype(np.uint8)
        m = np.tril(m)
        m[0, 1, 5, :] = 0              # an empty row: O = 0, LSE = -inf
        m[1, 3, 0, :] = 0
        return synth.gen_random_upper_noise(m, seed + 3)
    if kind == "p20":
        return synth.gen_block_mask(shape, seed + 1, 0.8).mask
    raise ValueError(kind)


@pytest.mark.parametrize("name,shape,seed,kind,dt", CASES, ids=[c[0] for c in CASES])
def test_sparse_matches_oracle(name, shape, seed, kind, dt):
    _run_full(shape, seed, _mask_for(kind, shape, seed), dt, name)


@pytest.mark.parametrize("shape", [Shape(1, 4, 2, 777, 128), Shape(1, 2, 1, 300, 64)], ids=["d128_s777", "d64_s300"])
def test_dense_matches_oracle(shape):
    _run_full(shape, 40, None, torch.float32, "dense")


def test_all_ones_mask_matches_dense():
    """An all-ones mask computes every causal tile, as the dense kernel does.
    The block-sparse kernel walks a row's tiles in a rotated order, so the
    results agree to a few bf16 rounding steps of P, not bitwise."""
    seer = _seer()
    shape = Shape(1, 4, 2, 1000, 128)
    q, k, v = (dev_bf16(x) for x in synth.gen_qkv(shape, 41))
    ones = torch.ones((1, 4, shape.nb, shape.nb), dtype=torch.uint8, device="cuda")
    a, la = seer.seer_block_sparse_attn_fwd(q, k, v, ones, out_dtype=torch.float32, want_lse=True)
    b, lb = seer.seer_block_sparse_attn_fwd(q, k, v, None, out_dtype=torch.float32, want_lse=True)
    torch.cuda.synchronize()
    check_close(host(a), host(b), "all-ones vs dense O", max_abs=5e-4, mean_abs=2e-5)
    check_lse(host(la), host(lb), "all-ones vs dense LSE", tol=1e-4)


def test_deterministic_reruns():
    seer = _seer()
    shape = Shape(1, 8, 2, 2048, 128)
    q, k, v = (dev_bf16(x) for x in synth.gen_qkv(shape, 42))
    m = dev_u8(synth.gen_block_mask(shape, 43, 0.7).mask)
    a, _ = seer.seer_block_sparse_attn_fwd(q, k, v, m)
    b, _ = seer.seer_block_sparse_attn_fwd(q, k, v, m)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_llama8b_s8k_50_sampled():
    """The 8k, 50%-sparse Llama-3.1-8B-shaped layer, full GPU run, oracle on sampled query blocks."""
    seer = _seer()
    w = synth.WORKLOADS["llama8b_s8k_50"]
    shape = w["shape"]
    say(f"[llama8b_s8k_50] shape={shape} seed={w['seed']}")
    q, k, v = synth.gen_qkv(shape, w["seed"])
    minfo = synth.workload_mask("llama8b_s8k_50")
    out, lse = seer.seer_block_sparse_attn_fwd(dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_u8(minfo.mask),
                                               out_dtype=torch.bfloat16, want_lse=True)
    torch.cuda.synchronize()
    out_h, lse_h = host(out), host(lse)
    rows = sample_rows(1, shape.heads_q, shape.nb, 3, 7)
    o_ref, l_ref = oracle.attention_rows(q, k, v, minfo.mask, rows)
    got = np.concatenate([out_h[b, h, 64 * i:64 * i + 64] for (b, h, i) in rows])
    got_l = np.concatenate([lse_h[b, h, 64 * i:64 * i + 64] for (b, h, i) in rows])
    check_close(got, np.concatenate(o_ref), "8k O (sampled)", out_dtype=torch.bfloat16)
    check_lse(got_l, np.concatenate(l_ref), "8k LSE (sampled)")


def _xcd_balanced(mask):
    """Whether the per-XCD active causal tiles of the XCD-major row order (XCD
    x owns the flattened heads [x BH/8, (x+1) BH/8)) are within 1.2 x their mean."""
    B, H, nb, _ = mask.shape
    per_head = (np.tril(np.ones((nb, nb), dtype=bool)) & (mask != 0)).reshape(B * H, nb, nb).sum(axis=(1, 2))
    load = per_head.reshape(8, -1).sum(axis=1)
    return 5 * 8 * int(load.max()) <= 6 * int(load.sum())


XCD_MAJOR_CASES = [
    ("d128_s2387_h16", Shape(1, 16, 4, 64 * 37 + 19, 128), torch.bfloat16),
    ("d64_s2887_b2_h8", Shape(2, 8, 2, 64 * 45 + 7, 64), torch.float32),
]


@pytest.mark.parametrize("shape,dt", [(Shape(1, 8, 2, 16384, 128), torch.bfloat16),
                                      (Shape(1, 8, 8, 64 * 512 - 5, 64), torch.float32)],
                         ids=["d128_s16384_nb256", "d64_s32763_nb512"])
def test_sparse_xcd_major_longest_rows(shape, dt):
    """The longest rows the XCD-major order takes (256 blocks at D = 128, 512
    at D = 64) on a balanced mask, sampled rows against the oracle."""
    seed = 75 + shape.head_dim
    m = synth.gen_random_upper_noise(synth.gen_block_mask(shape, seed + 1, 0.85).mask, seed + 2)
    assert _xcd_balanced(m)
    rows = sample_rows(shape.batch, shape.heads_q, shape.nb, 3, seed + 3)
    _run_sampled(shape, seed, m, dt, rows, f"xcd-major {shape.seq_len}")


@pytest.mark.parametrize("name,shape,dt", XCD_MAJOR_CASES, ids=[c[0] for c in XCD_MAJOR_CASES])
def test_sparse_xcd_major_order(name, shape, dt):
    """Short rows with batch x heads a multiple of 8 run in the order a pre-pass
    picks from the mask: XCD-major when the per-XCD work is balanced, the
    key-chunked order otherwise (host-side counts below confirm which side of
    the threshold each mask is on). Both runs are checked against the oracle.
    A row's tiles are summed in a rotation phased by its workgroup index, so
    the heads the two masks share agree to rounding, not bitwise."""
    seer = _seer()
    seed = 70 + shape.head_dim
    nb = shape.nb
    bal = synth.gen_random_upper_noise(synth.gen_block_mask(shape, seed + 1, 0.7).mask, seed + 2)
    bal[0, 3, nb - 1, :] = 0                      # an empty row
    imb = bal.copy()
    per = shape.batch * shape.heads_q // 8        # flattened heads of XCD 0 in that order: dense
    flat = imb.reshape(-1, nb, nb)
    flat[:per] = np.tril(np.ones((nb, nb), dtype=np.uint8))
    assert _xcd_balanced(bal) and not _xcd_balanced(imb)
    q, k, v = synth.gen_qkv(shape, seed)
    qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    outs = []
    for what, m in (("balanced", bal), ("imbalanced", imb)):
        say(f"[{name} {what}] shape={shape} seed={seed} out={dt}")
        out, lse = seer.seer_block_sparse_attn_fwd(qd, kd, vd, dev_u8(m), out_dtype=dt, want_lse=True)
        torch.cuda.synchronize()
        o_ref, l_ref = oracle.attention(q, k, v, m)
        check_close(host(out), o_ref, f"{name} {what} O", out_dtype=dt)
        check_lse(host(lse), l_ref, f"{name} {what} LSE")
        outs.append(host(out).reshape(-1, shape.seq_len, shape.head_dim))
    check_close(outs[0][per:], outs[1][per:], f"{name} shared heads, both orders", max_abs=1e-2, mean_abs=1e-4,
                out_dtype=dt)


ROWS_CASES = [
    # one-item rows of more than 256 blocks at D = 128 with at least 8 rows per
    # resident workgroup: the persistent launch with per-XCD queues and stealing
    ("d128_s19217_h32_bf16", Shape(1, 32, 8, 64 * 300 + 17, 128), torch.bfloat16),
    ("d128_s33000_b2_h16_f32", Shape(2, 16, 4, 64 * 515 + 40, 128), torch.float32),
    # the longest one-item rows (1024 blocks), one head per queue
    ("d128_s65536_h8_bf16", Shape(1, 8, 2, 65536, 128), torch.bfloat16),
    # 12 heads: queues of one or two heads
    ("d128_s44800_h12_bf16", Shape(1, 12, 3, 64 * 700, 128), torch.bfloat16),
]


@pytest.mark.parametrize("name,shape,dt", ROWS_CASES, ids=[c[0] for c in ROWS_CASES])
def test_sparse_persistent_rows(name, shape, dt):
    """Per-head sparsity in [0.8, 0.97] and the heads of the first queue fully
    dense, so the other workgroups run dry early and take rows from that queue;
    an empty row, a row active only on its diagonal and one without its
    diagonal, a ragged last block. Sampled rows, every head, against the oracle."""
    seed = 90 + shape.batch
    nb = shape.nb
    bh = shape.batch * shape.heads_q
    rng = np.random.Generator(np.random.PCG64(seed))
    s_heads = synth.per_head_sparsity(bh, 0.8, 0.97, 0.9, rng).reshape(shape.batch, shape.heads_q)
    m = synth.gen_block_mask(shape, seed + 1, s_heads).mask.copy()
    per = bh // 8                                  # flattened heads of queue 0
    flat = m.reshape(-1, nb, nb)
    flat[:per] = np.tril(np.ones((nb, nb), dtype=np.uint8))
    b1, h1 = divmod(per, shape.heads_q)            # the first head of queue 1
    m[b1, h1, nb - 1, :] = 0                       # no active key: O = 0, LSE = -inf
    m[b1, h1 + 1, 200, :] = 0
    m[b1, h1 + 1, 200, 200] = 1                    # only the diagonal
    m[b1, h1 + 2, nb - 2, nb - 2] = 0              # diagonal off
    m = synth.gen_random_upper_noise(m, seed + 2)
    rows = sample_rows(shape.batch, shape.heads_q, nb, 2, seed + 3)
    rows += [(b1, h1, nb - 1), (b1, h1 + 1, 200), (b1, h1 + 2, nb - 2)]
    _run_sampled(shape, seed, m, dt, sorted(set(rows)), name)


def _chunk_boundary_rows(B, H, nb, seed, chunk=512):
    """Sampled rows plus every query block next to a key-chunk boundary."""
    extra = [x for c in range(chunk, nb, chunk) for x in (c - 1, c, c + 1) if x < nb]
    return sample_rows(B, H, nb, 3, seed, extra=extra)


def _run_sampled(shape, seed, mask, out_dtype, rows, what):
    seer = _seer()
    say(f"[{what}] shape={shape} seed={seed} out={out_dtype} rows={len(rows)}")
    q, k, v = synth.gen_qkv(shape, seed)
    out, lse = seer.seer_block_sparse_attn_fwd(dev_bf16(q), dev_bf16(k), dev_bf16(v),
                                               None if mask is None else dev_u8(mask),
                                               out_dtype=out_dtype, want_lse=True)
    torch.cuda.synchronize()
    got = np.concatenate([host(out[b, h, 64 * i:64 * i + 64]) for (b, h, i) in rows])
    got_l = np.concatenate([host(lse[b, h, 64 * i:64 * i + 64]) for (b, h, i) in rows])
    del out, lse
    o_ref, l_ref = oracle.attention_rows(q, k, v, mask, rows)
    check_close(got, np.concatenate(o_ref), f"{what} O (sampled)", out_dtype=out_dtype)
    check_lse(got_l, np.concatenate(l_ref), f"{what} LSE (sampled)")


@pytest.mark.parametrize("shape,dt", [(Shape(1, 4, 2, 64 * 1100 - 17, 64), torch.float32),
                                      (Shape(2, 4, 1, 64 * 1040 + 5, 128), torch.bfloat16)],
                         ids=["d64_s70383_f32", "d128_s66565_bf16"])
def test_sparse_multichunk_rows(shape, dt):
    """Rows whose causal key range spans several key chunks (partials + merge),
    with a ragged last block, an empty row, a row active only in its first
    chunk and a row active only on its diagonal."""
    seed = 50 + shape.head_dim
    nb = shape.nb
    m = synth.gen_block_mask(shape, seed + 1, 0.85).mask.copy()
    m[0, 1, nb - 1, :] = 0                       # no active key at all: O = 0, LSE = -inf
    m[0, 2, nb - 2, :] = 0
    m[0, 2, nb - 2, :5] = 1                      # only the first chunk contributes
    m[0, 3, 600, :] = 0
    m[0, 3, 600, 600] = 1                        # only the diagonal (in the second chunk)
    m = synth.gen_random_upper_noise(m, seed + 2)
    rows = _chunk_boundary_rows(shape.batch, shape.heads_q, nb, seed + 3)
    rows += [(0, 1, nb - 1), (0, 2, nb - 2), (0, 3, 600)]
    _run_sampled(shape, seed, m, dt, sorted(set(rows)), "multichunk")


def test_sparse_multichunk_all_ones_matches_dense():
    """An all-ones mask over several key chunks agrees with the dense kernel.
    Not bitwise: each chunk rounds its probabilities to bf16 relative to its own
    running maximum before the P.V product, so the two differ by a few bf16
    rounding steps of P (2^-8 relative), far inside the oracle tolerance."""
    seer = _seer()
    shape = Shape(1, 2, 1, 64 * 1030, 128)
    q, k, v = (dev_bf16(x) for x in synth.gen_qkv(shape, 44))
    ones = torch.ones((1, 2, shape.nb, shape.nb), dtype=torch.uint8, device="cuda")
    a, la = seer.seer_block_sparse_attn_fwd(q, k, v, ones, out_dtype=torch.float32, want_lse=True)
    b, lb = seer.seer_block_sparse_attn_fwd(q, k, v, None, out_dtype=torch.float32, want_lse=True)
    torch.cuda.synchronize()
    check_close(host(a), host(b), "all-ones vs dense O", max_abs=5e-4, mean_abs=2e-5)
    check_lse(host(la), host(lb), "all-ones vs dense LSE", tol=1e-4)


XCD_CASES = [
    # rows of >= 960 blocks and >= 64 (batch, KV group, 128-block chunk) jobs:
    # the XCD-owned persistent path with bf16 partials
    ("d64_s83183_g2_f32", Shape(1, 16, 8, 64 * 1300 - 17, 64), torch.float32),
    ("d128_s82565_g1_bf16", Shape(1, 8, 8, 64 * 1290 + 5, 128), torch.bfloat16),
    # the shortest rows of the path (960 blocks, a last chunk of 64 blocks)
    ("d128_s61400_g1_bf16", Shape(1, 8, 8, 64 * 960 - 40, 128), torch.bfloat16),
    # two sequences, GQA groups of 2: jobs of both batches dealt over the XCDs
    ("d128_s64000_b2_g2_f32", Shape(2, 8, 4, 64 * 1000, 128), torch.float32),
    # a last chunk of one row (1025 blocks), head_dim 64
    ("d64_s65537_g1_f32", Shape(1, 8, 8, 64 * 1024 + 1, 64), torch.float32),
    # GQA groups of 8 (the diagonal launch's query-block-major order over 8 heads)
    ("d64_s64000_g8_bf16", Shape(1, 64, 8, 64 * 1000, 64), torch.bfloat16),
    # 88 jobs (2 x 4 KV groups x 11 chunks): the last 16 of the dealing only partly filled
    ("d64_s89550_b2_g2_f32", Shape(2, 8, 4, 64 * 1400 - 50, 64), torch.float32),
]


@pytest.mark.parametrize("name,shape,dt", XCD_CASES, ids=[c[0] for c in XCD_CASES])
def test_sparse_xcd_rows(name, shape, dt):
    """Rows cut into 128-block key chunks owned by XCDs (persistent workgroups,
    bf16 partials merged by the rows' diagonal chunks): chunk-boundary rows, a ragged last block, an
    empty row, rows active only in their first chunk, only on the diagonal,
    only in the first and last chunk (empty chunks between), with a full chunk,
    and without the diagonal."""
    seed = 60 + shape.head_dim
    nb = shape.nb
    m = synth.gen_block_mask(shape, seed + 1, 0.85).mask.copy()
    m[0, 1, nb - 1, :] = 0                       # no active key at all: O = 0, LSE = -inf
    m[0, 2, nb - 2, :] = 0
    m[0, 2, nb - 2, :5] = 1                      # only the first chunk contributes
    m[0, 3, 600, :] = 0
    m[0, 3, 600, 600] = 1                        # only the diagonal (in the fifth chunk)
    m[0, 4, nb - 3, :] = 0
    m[0, 4, nb - 3, [0, 3, nb - 5, nb - 3]] = 1  # first and last chunk only
    m[0, 5, 700, 256:384] = 1                    # one whole chunk active
    m[0, 6, 900, 900] = 0                        # diagonal off
    m = synth.gen_random_upper_noise(m, seed + 2)
    rows = sample_rows(shape.batch, shape.heads_q, nb, 2, seed + 3)
    rows += [(b, h, x) for b in {0, shape.batch - 1} for h in (0, shape.heads_q - 1)
             for c in range(128, nb, 128) for x in (c - 1, c, c + 1) if x < nb]
    rows += [(0, 1, nb - 1), (0, 2, nb - 2), (0, 3, 600), (0, 4, nb - 3), (0, 5, 700), (0, 6, 900)]
    _run_sampled(shape, seed, m, dt, sorted(set(rows)), name)


def test_sparse_xcd_all_ones_matches_dense():
    """An all-ones mask through the XCD-owned path agrees with the dense kernel
    to the rounding of its bf16 partial outputs (2^-9 relative per chunk)."""
    seer = _seer()
    shape = Shape(1, 8, 8, 64 * 1290, 128)
    q, k, v = (dev_bf16(x) for x in synth.gen_qkv(shape, 45))
    ones = torch.ones((1, 8, shape.nb, shape.nb), dtype=torch.uint8, device="cuda")
    a, la = seer.seer_block_sparse_attn_fwd(q, k, v, ones, out_dtype=torch.float32, want_lse=True)
    b, lb = seer.seer_block_sparse_attn_fwd(q, k, v, None, out_dtype=torch.float32, want_lse=True)
    torch.cuda.synchronize()
    check_close(host(a), host(b), "xcd all-ones vs dense O", max_abs=1e-3, mean_abs=5e-5)
    check_lse(host(la), host(lb), "xcd all-ones vs dense LSE", tol=1e-4)


@pytest.mark.parametrize("name", ["llama8b_s32k_90", "llama8b_s128k_90"])
def test_workload_sampled(name):
    """The Llama-3.1-8B-shaped layers at full length with their seeded masks, in
    the launch configuration the benchmark times; oracle on sampled query blocks
    (including the blocks next to every key-chunk boundary of one head)."""
    w = synth.WORKLOADS[name]
    shape = w["shape"]
    minfo = synth.workload_mask(name)
    rows = sample_rows(shape.batch, shape.heads_q, shape.nb, 1, 9)
    extra = [x for c in range(128, shape.nb, 128) for x in (c - 1, c)]
    rows = sorted(set(rows) | {(0, 5, x) for x in extra})
    _run_sampled(shape, w["seed"], minfo.mask, torch.bfloat16, rows, name)


def _growing_scores(shape, seed, hot_blocks, boost_log2):
    """Q/K/V from the seed with a shared direction u per KV group added to the
    queries (amplitude a) and to the keys of `hot_blocks` (amplitude b), a b
    chosen so those keys score about `boost_log2` log2 units above the others.
    A row that meets a hot block after its first tile then raises its running
    maximum far past the lazy rescale's slack, and the chunks of a long row
    carry very different log-sum-exps into their merge."""
    q, k, v = synth.gen_qkv(shape, seed)
    qf, kf = synth.f32_from_bf16_bits(q).copy(), synth.f32_from_bf16_bits(k).copy()
    d = shape.head_dim
    g = shape.heads_q // shape.heads_kv
    rng = np.random.default_rng(seed + 1)
    a = 4.0
    b = boost_log2 / (a * np.log2(np.e) / np.sqrt(d))
    for kv in range(shape.heads_kv):
        u = rng.standard_normal(d).astype(np.float32)
        u /= np.linalg.norm(u)
        qf[:, kv * g:(kv + 1) * g] += a * u
        for blk in hot_blocks:
            kf[:, kv, 64 * blk:64 * blk + 64] += b * u
    return synth.bf16_bits_from_f32(qf), synth.bf16_bits_from_f32(kf), v


def test_sparse_running_max_grows_past_slack():
    """Later tiles of a row raise the running maximum by ~24 log2 units (three
    times the slack), through the row kernel: the lazy update's rescale branch
    against the oracle, every row."""
    seer = _seer()
    shape = Shape(1, 4, 2, 64 * 40 - 7, 64)
    q, k, v = _growing_scores(shape, 90, (2, 9, 17, 30), 24.0)
    mask = np.ones((1, 4, shape.nb, shape.nb), dtype=np.uint8)
    mask[0, 1, :, 9] = 0                          # one head without the second hot block
    say(f"[growing max] shape={shape}")
    out, lse = seer.seer_block_sparse_attn_fwd(dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_u8(mask),
                                               out_dtype=torch.float32, want_lse=True)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(q, k, v, mask)
    check_close(host(out), o_ref, "growing max O", out_dtype=torch.float32)
    check_lse(host(lse), l_ref, "growing max LSE")


def test_sparse_xcd_running_max_grows_past_slack():
    """The same through the XCD-owned path (960 blocks, 8 KV groups): hot
    blocks in the first, a middle and the last chunks, so the first launch's
    partials and the diagonal chunks' merge see log-sum-exps ~24 log2 units
    apart (the one-pass merge's rescale). Sampled rows of every head."""
    seer = _seer()
    shape = Shape(1, 8, 8, 64 * 960, 128)
    q, k, v = _growing_scores(shape, 91, (2, 300, 700, 940), 24.0)
    nb = shape.nb
    mask = synth.gen_block_mask(shape, 92, 0.8).mask.copy()
    mask[:, :, :, [2, 300, 700, 940]] = 1
    rows = sample_rows(1, 8, nb, 2, 93) + [(0, h, x) for h in (0, 7) for x in (1, 2, 127, 128, 301, 701, 939, 959)]
    rows = sorted(set(rows))
    say(f"[growing max xcd] shape={shape} rows={len(rows)}")
    out, lse = seer.seer_block_sparse_attn_fwd(dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_u8(mask),
                                               out_dtype=torch.float32, want_lse=True)
    torch.cuda.synchronize()
    got = np.concatenate([host(out[b, h, 64 * i:64 * i + 64]) for (b, h, i) in rows])
    got_l = np.concatenate([host(lse[b, h, 64 * i:64 * i + 64]) for (b, h, i) in rows])
    o_ref, l_ref = oracle.attention_rows(q, k, v, mask, rows)
    check_close(got, np.concatenate(o_ref), "growing max xcd O (sampled)", out_dtype=torch.float32)
    check_lse(got_l, np.concatenate(l_ref), "growing max xcd LSE (sampled)")


@pytest.mark.parametrize("name,shape", [("persistent_rows_s19200", Shape(1, 32, 8, 64 * 300, 128)),
                                        ("xcd_two_launches_s61440", Shape(1, 8, 8, 64 * 960, 128))])
def test_deterministic_reruns_dynamic_schedules(name, shape):
    """The persistent launches hand out rows and items through atomic counters,
    so which workgroup runs which item changes from call to call; every item's
    arithmetic and every merge order are fixed, so O and LSE are bitwise equal
    across calls."""
    seer = _seer()
    q, k, v = (dev_bf16(x) for x in synth.gen_qkv(shape, 47))
    m = dev_u8(synth.gen_block_mask(shape, 48, 0.9).mask)
    say(f"[determinism {name}] shape={shape}")
    runs = [seer.seer_block_sparse_attn_fwd(q, k, v, m, want_lse=True) for _ in range(3)]
    torch.cuda.synchronize()
    for o, l in runs[1:]:
        assert torch.equal(o.view(torch.int16), runs[0][0].view(torch.int16))
        assert torch.equal(l, runs[0][1])
