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
    check_close(host(out), o_ref, f"{what} O")
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
    check_close(host(a), host(b), "all-ones vs dense O", max_abs=2e-3, mean_abs=2e-5)
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
    check_close(got, np.concatenate(o_ref), "8k O (sampled)")
    check_lse(got_l, np.concatenate(l_ref), "8k LSE (sampled)")


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
    check_close(got, np.concatenate(o_ref), f"{what} O (sampled)")
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
    check_close(host(a), host(b), "all-ones vs dense O", max_abs=2e-3, mean_abs=2e-5)
    check_lse(host(la), host(lb), "all-ones vs dense LSE", tol=1e-4)


XCD_CASES = [
    # rows of >= 1280 blocks and >= 64 (batch, KV group, 128-block chunk) jobs:
    # the XCD-owned persistent path with bf16 partials
    ("d64_s83183_g2_f32", Shape(1, 16, 8, 64 * 1300 - 17, 64), torch.float32),
    ("d128_s82565_g1_bf16", Shape(1, 8, 8, 64 * 1290 + 5, 128), torch.bfloat16),
]


@pytest.mark.parametrize("name,shape,dt", XCD_CASES, ids=[c[0] for c in XCD_CASES])
def test_sparse_xcd_rows(name, shape, dt):
    """Rows cut into 128-block key chunks owned by XCDs (persistent workgroups,
    bf16 partials, merge kernel): chunk-boundary rows, a ragged last block, an
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
    rows += [(0, h, x) for h in (0, shape.heads_q - 1) for c in range(128, nb, 128) for x in (c - 1, c, c + 1)]
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
    check_close(host(a), host(b), "xcd all-ones vs dense O", max_abs=2e-3, mean_abs=1e-4)
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
