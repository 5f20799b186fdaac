"""Pins for the fp64 oracle: checks against facts that do not come from the oracle.

Each pin takes the oracle module `O` as its argument, so the same checks run
against the real oracle (tests/test_oracle_pins.py) and against copies of it
with a planted mistake (tests/test_oracle_mutations.py), which must fail at
least one pin. Sources of truth used here:
  * library special cases: torch's scaled_dot_product_attention (fp64, CPU,
    causal, GQA), torch's max_pool2d / avg_pool1d / max_pool1d, np.add.reduceat;
  * closed forms: Q = 0 gives the mean of V over the visible keys and
    LSE = log(#keys); constant V gives O = V; W_q = 0 gives gate scores
    1/(i+1); a one-hot V returns the attention probabilities themselves;
  * brute force in pure Python (math.exp loops) on tiny inputs;
  * a hand-computed gate example under tests/golden/;
  * the bfloat16 format's definition (sign, 8-bit exponent, 7-bit fraction)
    and torch's bfloat16 dtype, for the widening of raw bf16 bit patterns;
  * invariants the pages state: softmax rows sum to 1 (explainer section 3.4,
    "After softmax, each row sums to 1.0"); the max-pooled value of a block is
    small only if every entry in it is small (section 3.4, "Ground truth
    generation"); a larger threshold activates fewer blocks (section 3.4,
    "Method 2: Thresholding").
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F

from synth import Shape, gen_qkv, gen_tiny_mask, gen_random_upper_noise, f32_from_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TOL = 1e-12


def _f64(bits):
    return f32_from_bf16_bits(bits).astype(np.float64)


def _qkv(shape, seed):
    q, k, v = gen_qkv(shape, seed)
    return _f64(q), _f64(k), _f64(v)


def _sdpa(q, k, v, causal=True, gqa=True):
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v))
    return torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, is_causal=causal, enable_gqa=gqa).numpy()


# ----------------------------------------------------------------------------
# attention
# ----------------------------------------------------------------------------
def pin_dense_matches_torch_sdpa(O):
    """All-ones mask and mask=None both equal torch's causal GQA SDPA (ragged S)."""
    shape = Shape(1, 4, 2, 200, 16)
    q, k, v = _qkv(shape, 11)
    ref = _sdpa(q, k, v)
    o_none, _ = O.attention(q, k, v, None)
    ones = np.ones((1, 4, shape.nb, shape.nb), dtype=np.uint8)
    o_ones, _ = O.attention(q, k, v, ones)
    assert np.abs(o_none - ref).max() < TOL
    assert np.abs(o_ones - ref).max() < TOL


def pin_probabilities_via_one_hot_v(O):
    """V = identity returns P itself: rows sum to 1, zero on masked/future keys."""
    S = 160
    shape = Shape(1, 1, 1, S, 8)
    q, k, _ = _qkv(shape, 12)
    v = np.eye(S)[None, None]
    minfo = gen_tiny_mask(shape, 5, p_keep=0.4)
    m = minfo.mask
    P, _ = O.attention(q, k, v, m)
    P = P[0, 0]
    assert P.min() >= 0.0
    assert np.abs(P.sum(axis=1) - 1.0).max() < TOL
    for t in range(S):
        for u in range(S):
            allowed = u <= t and m[0, 0, t // 64, u // 64] != 0
            if not allowed:
                assert P[t, u] == 0.0


def pin_constant_v_and_empty_rows(O):
    """Constant V gives O = V on non-empty rows; an empty row gives O = 0, LSE = -inf."""
    shape = Shape(1, 2, 1, 256, 8)
    q, k, _ = _qkv(shape, 13)
    c = np.linspace(-1.0, 2.0, 8)
    v = np.broadcast_to(c, (1, 1, 256, 8)).copy()
    m = np.tril(np.ones((1, 2, 4, 4), dtype=np.uint8))
    m[0, 1, 2, :] = 0          # query block 2 of head 1 has no key block at all
    o, lse = O.attention(q, k, v, m)
    empty = np.zeros((1, 2, 256), dtype=bool)
    empty[0, 1, 128:192] = True
    assert np.abs(o[~empty] - c).max() < 1e-12
    assert np.all(o[empty] == 0.0)
    assert np.all(np.isneginf(lse[empty]))
    assert np.all(np.isfinite(lse[~empty]))


def pin_q_zero_closed_form(O):
    """Q = 0: O_t = mean of V over visible active keys, LSE_t = log(#keys)."""
    shape = Shape(1, 2, 1, 200, 8)
    _, k, v = _qkv(shape, 14)
    q = np.zeros((1, 2, 200, 8))
    m = gen_tiny_mask(shape, 6, p_keep=0.5).mask
    o, lse = O.attention(q, k, v, m)
    for h in range(2):
        for t in range(200):
            keys = [u for u in range(t + 1) if m[0, h, t // 64, u // 64]]
            assert abs(lse[0, h, t] - math.log(len(keys))) < 1e-12
            assert np.abs(o[0, h, t] - v[0, 0, keys].mean(axis=0)).max() < 1e-12


def pin_single_block_row(O):
    """A row with one active block j < i is plain (non-causal) attention on block j."""
    shape = Shape(1, 1, 1, 256, 16)
    q, k, v = _qkv(shape, 15)
    m = np.zeros((1, 1, 4, 4), dtype=np.uint8)
    m[0, 0, 3, 1] = 1
    m[0, 0, 2, 2] = 1
    o, _ = O.attention(q, k, v, m)
    ref = _sdpa(q[:, :, 192:256], k[:, :, 64:128], v[:, :, 64:128], causal=False)
    assert np.abs(o[:, :, 192:256] - ref).max() < TOL
    ref2 = _sdpa(q[:, :, 128:192], k[:, :, 128:192], v[:, :, 128:192], causal=True)
    assert np.abs(o[:, :, 128:192] - ref2).max() < TOL


def pin_gqa_equals_mha(O):
    """GQA (4 query heads on 2 KV heads) equals MHA with K/V repeated per group."""
    shape = Shape(1, 4, 2, 192, 8)
    q, k, v = _qkv(shape, 16)
    m = gen_tiny_mask(shape, 7).mask
    o1, l1 = O.attention(q, k, v, m)
    o2, l2 = O.attention(q, np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1), m)
    assert np.abs(o1 - o2).max() < TOL and np.abs(l1 - l2).max() < TOL


def pin_bruteforce_python_loops(O):
    """Pure-Python loops (math.exp) on a tiny ragged GQA case with upper-triangle noise."""
    shape = Shape(1, 2, 1, 130, 4)
    q, k, v = _qkv(shape, 17)
    m = gen_random_upper_noise(gen_tiny_mask(shape, 8, p_keep=0.5).mask, 9)
    o, lse = O.attention(q, k, v, m)
    D = 4
    for h in range(2):
        for t in range(0, 130, 7):
            ks = [u for u in range(t + 1) if m[0, h, t // 64, u // 64] != 0]
            s = [sum(q[0, h, t, d] * k[0, 0, u, d] for d in range(D)) / math.sqrt(D) for u in ks]
            mx = max(s)
            e = [math.exp(x - mx) for x in s]
            den = sum(e)
            for d in range(D):
                ref = sum(e[n] * v[0, 0, ks[n], d] for n in range(len(ks))) / den
                assert abs(o[0, h, t, d] - ref) < 1e-12
            assert abs(lse[0, h, t] - (mx + math.log(den))) < 1e-12


# ----------------------------------------------------------------------------
# 2D-maxpooled ground truth
# ----------------------------------------------------------------------------
def pin_gt_matches_torch_maxpool(O):
    """gt equals torch max_pool2d (64x64, stride 64) of P taken from torch SDPA with V = I."""
    for S in (192, 200):
        shape = Shape(1, 4, 2, S, 16)                            # GQA: 4 query heads on 2 KV heads
        q, k, _ = _qkv(shape, 18 + S)
        eye = np.broadcast_to(np.eye(S), (1, 2, S, S)).copy()
        P = torch.from_numpy(_sdpa(q, k, eye))                  # [1, 4, S, S]
        ref = F.max_pool2d(P, 64, 64, ceil_mode=True).numpy()
        gt = O.maxpool_gt(q, k)
        assert np.abs(gt - ref).max() < TOL


def pin_gt_four_loop_bruteforce(O):
    """Explicit 4-loop 2D maxpool of a pure-Python softmax map (tiny, ragged)."""
    S, D = 130, 4
    shape = Shape(1, 1, 1, S, D)
    q, k, _ = _qkv(shape, 19)
    P = [[0.0] * S for _ in range(S)]
    for t in range(S):
        s = [sum(q[0, 0, t, d] * k[0, 0, u, d] for d in range(D)) / math.sqrt(D) for u in range(t + 1)]
        mx = max(s)
        e = [math.exp(x - mx) for x in s]
        den = sum(e)
        for u in range(t + 1):
            P[t][u] = e[u] / den
    nb = 3
    gt = O.maxpool_gt(q, k)[0, 0]
    for i in range(nb):
        for j in range(nb):
            best = 0.0
            for t in range(i * 64, min(i * 64 + 64, S)):
                for u in range(j * 64, min(j * 64 + 64, S)):
                    best = max(best, P[t][u])
            assert abs(gt[i, j] - best) < 1e-12


def pin_gt_properties(O):
    """gt[0,0] = 1 (token 0 sees only itself); 0 <= gt <= 1; 0 above the
    diagonal; row max >= 1/(64(i+1))."""
    shape = Shape(1, 2, 1, 320, 16)
    q, k, _ = _qkv(shape, 20)
    gt = O.maxpool_gt(q, k)
    nb = 5
    assert np.all(gt[..., 0, 0] == 1.0)
    assert gt.min() >= 0.0 and gt.max() <= 1.0
    assert np.all(gt[..., np.triu_indices(nb, 1)[0], np.triu_indices(nb, 1)[1]] == 0.0)
    for i in range(nb):
        assert np.all(gt[..., i, :].max(axis=-1) >= 1.0 / (64 * (i + 1)) - 1e-15)


def pin_gt_rows_match_full(O):
    """Sampled rows equal the same rows of the full map."""
    shape = Shape(1, 2, 1, 256, 8)
    q, k, _ = _qkv(shape, 21)
    full = O.maxpool_gt(q, k)
    rows = [(0, 1, 3), (0, 0, 0), (0, 1, 2)]
    for (b, h, i), r in zip(rows, O.maxpool_gt_rows(q, k, rows)):
        assert np.array_equal(r, full[b, h, i])


# ----------------------------------------------------------------------------
# AttnGate
# ----------------------------------------------------------------------------
def _hand_inputs():
    with open(os.path.join(GOLDEN, "gate_hand_example.json")) as f:
        g = json.load(f)
    S, D = g["seq_len"], g["head_dim"]
    q = np.zeros((1, 1, S, D))
    k = np.zeros((1, 1, S, D))
    for blk, spec in enumerate(g["q_blocks"]):
        for t in range(64):
            q[0, 0, blk * 64 + t] = spec["rows_even"] if t % 2 == 0 else spec["rows_odd"]
    for blk, spec in enumerate(g["k_blocks"]):
        for t in range(64):
            k[0, 0, blk * 64 + t] = spec["rows_even"] if t % 2 == 0 else spec["rows_odd"]
    wq = np.array(g["w_q"])[None]
    wk = np.array(g["w_k"])[None]
    return g, q, k, wq, wk


def pin_gate_hand_example(O):
    """The hand-computed gate example in tests/golden/gate_hand_example.json."""
    g, q, k, wq, wk = _hand_inputs()
    assert np.abs(O.pool_q(q)[0, 0] - np.array(g["expected_pooled_q"])).max() < 1e-15
    assert np.abs(O.pool_k(k)[0, 0] - np.array(g["expected_pooled_k"])).max() < 1e-15
    sc = O.gate_scores(q, k, wq, wk)[0, 0]
    logits = g["expected_logits_unscaled"]
    for i, row in enumerate(logits):
        zs = [x / math.sqrt(2.0) for x in row if x is not None]
        e = [math.exp(z - max(zs)) for z in zs]
        for j in range(3):
            want = e[j] / sum(e) if j <= i else 0.0
            assert abs(sc[i, j] - want) < 1e-14
            assert abs(sc[i, j] - g["expected_scores_4dp"][i][j]) < 5e-5


def pin_gate_rows_sum_to_one(O):
    shape = Shape(1, 4, 2, 640, 32)
    q, k, _ = _qkv(shape, 22)
    rng = np.random.default_rng(0)
    wq = rng.standard_normal((4, 32, 16)) / 4.0
    wk = rng.standard_normal((4, 96, 16)) / 4.0
    sc = O.gate_scores(q, k, wq, wk)
    nb = 10
    assert np.abs(sc.sum(axis=-1) - 1.0).max() < 1e-13
    iu = np.triu_indices(nb, 1)
    assert np.all(sc[..., iu[0], iu[1]] == 0.0)
    assert sc.min() >= 0.0


def pin_gate_wq_zero_closed_form(O):
    """W_q = 0 makes every causal logit 0, so score[i, j] = 1/(i+1) for j <= i."""
    shape = Shape(1, 2, 1, 64 * 50 - 10, 8)
    q, k, _ = _qkv(shape, 23)
    rng = np.random.default_rng(1)
    wq = np.zeros((2, 8, 8))
    wk = rng.standard_normal((2, 24, 8))
    sc = O.gate_scores(q, k, wq, wk)
    nb = 50
    want = np.tril(np.ones((nb, nb))) / np.arange(1, nb + 1)[:, None]
    assert np.abs(sc - want).max() < 1e-15


def pin_pool_matches_torch(O):
    """Pooling equals torch avg/max pooling (and -max(-x) for min); ragged via reduceat."""
    shape = Shape(2, 3, 3, 256, 8)
    q, k, _ = _qkv(shape, 24)
    tq = torch.from_numpy(q).reshape(6, 256, 8).transpose(1, 2)
    tk = torch.from_numpy(k).reshape(6, 256, 8).transpose(1, 2)
    avg_q = F.avg_pool1d(tq, 64, 64).transpose(1, 2).reshape(2, 3, 4, 8).numpy()
    mx = F.max_pool1d(tk, 64, 64).transpose(1, 2)
    mn = -F.max_pool1d(-tk, 64, 64).transpose(1, 2)
    av = F.avg_pool1d(tk, 64, 64).transpose(1, 2)
    kp = torch.cat([mx, mn, av], dim=-1).reshape(2, 3, 4, 24).numpy()
    assert np.abs(O.pool_q(q) - avg_q).max() < 1e-15
    assert np.abs(O.pool_k(k) - kp).max() < 1e-15
    # ragged: 200 tokens -> blocks of 64, 64, 64, 8
    qr = q[0, 0, :200]
    starts = np.array([0, 64, 128, 192])
    want = np.add.reduceat(qr, starts, axis=0) / np.array([64, 64, 64, 8])[:, None]
    assert np.abs(O.pool_q(qr) - want).max() < 1e-15
    kr = k[0, 0, :200]
    kmax = np.maximum.reduceat(kr, starts, axis=0)
    kmin = np.minimum.reduceat(kr, starts, axis=0)
    assert np.abs(O.pool_k(kr)[:, :8] - kmax).max() == 0.0
    assert np.abs(O.pool_k(kr)[:, 8:16] - kmin).max() == 0.0


def pin_pool_k_constant_blocks(O):
    """K constant inside each block: max = min = avg = that row."""
    rng = np.random.default_rng(2)
    rows = rng.standard_normal((3, 8))
    k = np.repeat(rows, 64, axis=0)
    kp = O.pool_k(k)
    assert np.array_equal(kp[:, :16], np.concatenate([rows, rows], axis=1))   # max, min exact
    assert np.abs(kp[:, 16:] - rows).max() < 1e-14                            # avg up to rounding


def pin_gate_gqa_equals_mha(O):
    """GQA gate equals MHA gate with K repeated; per-KV-head W_k equals W_k repeated."""
    shape = Shape(1, 4, 2, 320, 16)
    q, k, _ = _qkv(shape, 25)
    rng = np.random.default_rng(3)
    wq = rng.standard_normal((4, 16, 8))
    wk_kv = rng.standard_normal((2, 48, 8))
    a = O.gate_scores(q, k, wq, wk_kv, wk_per_kv_head=True)
    b = O.gate_scores(q, np.repeat(k, 2, axis=1), wq, np.repeat(wk_kv, 2, axis=0))
    c = O.gate_scores(q, k, wq, np.repeat(wk_kv, 2, axis=0))
    assert np.abs(a - b).max() < 1e-13
    assert np.abs(a - c).max() < 1e-13


# ----------------------------------------------------------------------------
# masks
# ----------------------------------------------------------------------------
def _flat_scores(O, nb, heads=2):
    S = 64 * nb
    shape = Shape(1, heads, 1, S, 4)
    q, k, _ = _qkv(shape, 26)
    wq = np.zeros((heads, 4, 4))
    wk = np.ones((heads, 12, 4))
    return O.gate_scores(q, k, wq, wk)


def pin_threshold_strict(O):
    """With equal logits score[i, j] = 1/(i+1); T = 0.25 keeps rows 0..2 only
    (row 3 has score exactly 0.25, which a strict '>' drops)."""
    sc = _flat_scores(O, 8)
    assert np.all(sc[..., 3, :4] == 0.25)
    m = O.threshold_mask(sc, 0.25)
    want = np.zeros((8, 8), dtype=np.uint8)
    want[:3] = np.tril(np.ones((3, 8), dtype=np.uint8))
    assert np.array_equal(m[0, 0], want) and np.array_equal(m[0, 1], want)


def pin_threshold_nesting(O):
    """Larger T activates a subset of blocks; realized sparsity is monotone in T."""
    rng = np.random.default_rng(4)
    z = rng.standard_normal((1, 2, 40, 40)) * 2.0
    z = np.where(np.tril(np.ones((40, 40), dtype=bool)), z, -np.inf)
    e = np.exp(z - z.max(axis=-1, keepdims=True))
    sc = e / e.sum(axis=-1, keepdims=True)
    ts = [0.0, 1e-3, 5e-3, 1e-2, 3e-2, 0.1, 0.5]
    masks = [O.threshold_mask(sc, t) for t in ts]
    for a, b in zip(masks, masks[1:]):
        assert np.all(b <= a)
    kept = [int(m.sum()) for m in masks]
    assert kept == sorted(kept, reverse=True)
    assert kept[0] == 2 * 40 * 41 // 2          # T = 0 keeps every causal block
    assert np.all(np.triu(masks[0][0, 0], 1) == 0)


def pin_topk_counts(O):
    rng = np.random.default_rng(5)
    sc = np.tril(rng.random((1, 3, 30, 30)))
    for k in (1, 4, 29, 30, 100):
        m = O.topk_mask(sc, k)
        cnt = m.sum(axis=-1)
        assert np.all(cnt == np.minimum(k, np.arange(1, 31)))
        assert np.all(np.triu(m[0, 0], 1) == 0)
    full = O.topk_mask(sc, 30)
    assert np.array_equal(full[0, 0], np.tril(np.ones((30, 30), dtype=np.uint8)))


def pin_topk_ties_low_index(O):
    """Equal scores: top-k keeps the k lowest key-block indices."""
    sc = _flat_scores(O, 10)
    m = O.topk_mask(sc, 3)
    for i in range(10):
        want = np.zeros(10, dtype=np.uint8)
        want[:min(3, i + 1)] = 1
        assert np.array_equal(m[0, 0, i], want)


def pin_topk_bruteforce(O):
    """Per-head k against Python's sorted() over (-score, j) on random scores with ties."""
    rng = np.random.default_rng(6)
    sc = np.round(rng.random((1, 2, 25, 25)), 1)        # coarse values -> many ties
    sc = np.tril(sc)
    ks = [3, 7]
    m = O.topk_mask(sc, ks)
    for h in range(2):
        for i in range(25):
            order = sorted(range(i + 1), key=lambda j: (-sc[0, h, i, j], j))
            keep = set(order[:ks[h]])
            for j in range(25):
                assert m[0, h, i, j] == (1 if j in keep else 0)


# ----------------------------------------------------------------------------
# block-level RoPE of the gate
# ----------------------------------------------------------------------------
def pin_rope_hand_complex(O):
    """theta = 6400, block 64 gives base 100, so the two pair frequencies of a
    Dg = 4 vector are 100^0 = 1 and 100^(-1/2) = 0.1 (worked by hand). Pair d
    is the complex number x[d] + i x[d + 2]; a rotation multiplies it by
    exp(i * position * frequency)."""
    import cmath
    x = np.array([[1.0, 2.0, 3.0, 4.0]] * 4)
    got = O.block_rope(x, 6400.0, 64)
    freqs = [1.0, 0.1]
    for pos in range(4):
        for d in range(2):
            z = complex(x[pos, d], x[pos, d + 2]) * cmath.exp(1j * pos * freqs[d])
            assert abs(got[pos, d] - z.real) < 1e-14 and abs(got[pos, d + 2] - z.imag) < 1e-14


def pin_rope_relative_and_orthogonal(O):
    """Rotated dot products depend only on the position difference; rotations
    keep norms; the negated positions undo the rotation."""
    rng = np.random.default_rng(5)
    qv = rng.standard_normal((1, 16))
    kv = rng.standard_normal((1, 16))
    for (i, j, shift) in [(3, 1, 5), (7, 7, 11), (2, 9, 40)]:
        a = O.block_rope(qv, 5e5, 64, positions=[i])[0] @ O.block_rope(kv, 5e5, 64, positions=[j])[0]
        b = O.block_rope(qv, 5e5, 64, positions=[i + shift])[0] @ O.block_rope(kv, 5e5, 64, positions=[j + shift])[0]
        assert abs(a - b) < 1e-12
    x = rng.standard_normal((6, 16))
    r = O.block_rope(x, 1e4, 64)
    assert np.abs(np.linalg.norm(r, axis=1) - np.linalg.norm(x, axis=1)).max() < 1e-12
    back = O.block_rope(r, 1e4, 64, positions=-np.arange(6))
    assert np.abs(back - x).max() < 1e-12
    assert np.abs(r[0] - x[0]).max() == 0.0              # position 0: no rotation


def pin_gate_rope_complex_bruteforce(O):
    """Gate scores with block RoPE equal a brute force written with complex
    numbers: logit(i, j) = Re(sum_d zq_d conj(zk_d) e^(i (i - j) f_d)) / sqrt(D),
    zq = Q'_i pairs, zk = K'_j pairs, f_d = (theta/64)^(-2d/Dg); pooling by torch."""
    import cmath
    shape = Shape(1, 2, 1, 64 * 6 - 9, 8)
    q, k, _ = _qkv(shape, 26)
    rng = np.random.default_rng(6)
    wq = rng.standard_normal((2, 8, 8)) / 2.0
    wk = rng.standard_normal((2, 24, 8)) / 2.0
    theta = 5e5
    sc = O.gate_scores(q, k, wq, wk, rope_theta=theta)
    nb, dg = 6, 8
    f = [(theta / 64.0) ** (-2.0 * d / dg) for d in range(dg // 2)]
    pad = 64 * nb - shape.seq_len
    for h in range(2):
        tq = torch.from_numpy(q[0, h])
        tk = torch.from_numpy(k[0, 0])
        # ragged last block: mean / max / min over the tokens it has
        qp = np.stack([tq[64 * i:64 * i + 64].mean(0).numpy() for i in range(nb)])
        kp = np.stack([np.concatenate([tk[64 * i:64 * i + 64].max(0).values.numpy(),
                                       tk[64 * i:64 * i + 64].min(0).values.numpy(),
                                       tk[64 * i:64 * i + 64].mean(0).numpy()]) for i in range(nb)])
        assert pad > 0
        qg = qp @ wq[h]
        kg = kp @ wk[h]
        for i in range(nb):
            logits = []
            for j in range(i + 1):
                acc = 0.0
                for d in range(dg // 2):
                    zq = complex(qg[i, d], qg[i, d + dg // 2])
                    zk = complex(kg[j, d], kg[j, d + dg // 2])
                    acc += (zq * zk.conjugate() * cmath.exp(1j * (i - j) * f[d])).real
                logits.append(acc / math.sqrt(8))
            mx = max(logits)
            e = [math.exp(z - mx) for z in logits]
            for j in range(nb):
                want = e[j] / sum(e) if j <= i else 0.0
                assert abs(sc[0, h, i, j] - want) < 1e-13


# ----------------------------------------------------------------------------
# distillation step (KL of the row-normalized ground truth and the gate score)
# ----------------------------------------------------------------------------
def _distill_case(seed, per_kv):
    shape = Shape(1, 4, 2, 64 * 5 - 7, 8)
    q, k, _ = _qkv(shape, seed)
    rng = np.random.default_rng(seed)
    wq = rng.standard_normal((4, 8, 4)) / 2.0
    wk = rng.standard_normal((2 if per_kv else 4, 24, 4)) / 2.0
    nb = 5
    gt = np.tril(rng.random((1, 4, nb, nb)) + 0.01)
    gt[0, 1, 3, :2] = 0.0                       # zero entries contribute nothing
    return q, k, wq, wk, gt


def pin_distill_finite_differences(O):
    """Analytic gradients equal central differences of the loss (fp64, with and
    without block RoPE, W_k per query head and per KV head)."""
    for seed, per_kv, theta in [(31, False, None), (32, True, 5e5), (33, False, 1e4)]:
        q, k, wq, wk, gt = _distill_case(seed, per_kv)
        loss, gq, gk = O.gate_distill(q, k, wq, wk, gt, wk_per_kv_head=per_kv, rope_theta=theta)
        rng = np.random.default_rng(seed + 100)
        eps = 1e-6
        for w, g, which in [(wq, gq, "q"), (wk, gk, "k")]:
            for _ in range(6):
                idx = tuple(int(rng.integers(n)) for n in w.shape)
                wp, wm = w.copy(), w.copy()
                wp[idx] += eps
                wm[idx] -= eps
                args_p = (wp, wk) if which == "q" else (wq, wp)
                args_m = (wm, wk) if which == "q" else (wq, wm)
                lp = O.gate_distill(q, k, *args_p, gt, wk_per_kv_head=per_kv, rope_theta=theta)[0]
                lm = O.gate_distill(q, k, *args_m, gt, wk_per_kv_head=per_kv, rope_theta=theta)[0]
                fd = (lp - lm) / (2 * eps)
                assert abs(fd - g[idx]) <= 1e-7 + 1e-5 * abs(fd), (which, idx, fd, g[idx])


def pin_distill_loss_definition(O):
    """The loss is the mean over query-block rows of sum_j p log(p / score),
    with p the gt row divided by its sum (pure-Python brute force on the
    oracle's own, separately pinned, gate scores); it is 0 with zero gradients
    when gt is the gate's own score, and it ignores a positive scale per row."""
    q, k, wq, wk, gt = _distill_case(34, False)
    loss, _, _ = O.gate_distill(q, k, wq, wk, gt, rope_theta=5e5)
    sc = O.gate_scores(q, k, wq, wk, rope_theta=5e5)
    total, rows = 0.0, 0
    for h in range(4):
        for i in range(5):
            row = [gt[0, h, i, j] for j in range(i + 1)]
            tot = sum(row)
            for j in range(i + 1):
                pj = row[j] / tot
                if pj > 0:
                    total += pj * math.log(pj / sc[0, h, i, j])
            rows += 1
    assert abs(loss - total / rows) < 1e-13
    assert loss > 0
    scaled = gt * np.random.default_rng(7).uniform(0.5, 3.0, size=(1, 4, 5, 1))
    assert abs(O.gate_distill(q, k, wq, wk, scaled, rope_theta=5e5)[0] - loss) < 1e-13
    self_loss, gq, gk = O.gate_distill(q, k, wq, wk, sc, rope_theta=5e5)
    assert abs(self_loss) < 1e-14 and np.abs(gq).max() < 1e-14 and np.abs(gk).max() < 1e-14
    # a row with no ground-truth mass has no target: it adds nothing to the loss
    # (which stays a mean over all rows) and nothing to the gradient
    gz = gt.copy()
    gz[0, 2, 3, :] = 0.0
    lz, gqz, _ = O.gate_distill(q, k, wq, wk, gz, rope_theta=5e5)
    row = [gt[0, 2, 3, j] / sum(gt[0, 2, 3, :4]) for j in range(4)]
    drop = sum(pj * math.log(pj / sc[0, 2, 3, j]) for j, pj in enumerate(row) if pj > 0)
    assert abs(lz - (loss - drop / rows)) < 1e-13
    lo, gqo, gko = O.gate_distill(q, k, wq, wk, np.zeros_like(gt), rope_theta=5e5)
    assert lo == 0.0 and np.abs(gqo).max() == 0.0 and np.abs(gko).max() == 0.0


# ----------------------------------------------------------------------------
# decode-stage gating
# ----------------------------------------------------------------------------
def pin_decode_attention_matches_sdpa_and_prefill(O):
    """Dense decode attention equals torch SDPA (fp64, one query against every
    key, GQA); with a block mask it equals the last row of the separately
    pinned prefill attention given that mask row (the newest token of a
    prefill sees exactly the cached keys)."""
    shape = Shape(2, 4, 2, 64 * 5 - 11, 16)
    q, k, v = _qkv(shape, 81)
    qd = q[:, :, -1]
    o, lse = O.decode_attention(qd, k, v, None)
    ref = _sdpa(qd[:, :, None], k, v, causal=False)[:, :, 0]
    assert np.abs(o - ref).max() < 1e-12
    s_ = np.einsum("bhd,bhsd->bhs", qd, np.repeat(k, 2, axis=1)) / 4.0
    assert np.abs(lse - np.log(np.exp(s_).sum(-1))).max() < 1e-12
    rng = np.random.default_rng(3)
    nb = shape.nb
    m2 = (rng.random((2, 4, nb, nb)) < 0.5).astype(np.uint8)
    m2[0, 1, nb - 1, :] = 0                        # empty row
    od, ld = O.decode_attention(qd, k, v, m2[:, :, nb - 1])
    rows = [(b, h, nb - 1) for b in range(2) for h in range(4)]
    o_rows, l_rows = O.attention_rows(q, k, v, m2, rows)
    for n, (b, h, _) in enumerate(rows):
        assert np.abs(od[b, h] - o_rows[n][-1]).max() < 1e-12
        assert (ld[b, h] == l_rows[n][-1]) or abs(ld[b, h] - l_rows[n][-1]) < 1e-12
    assert ld[0, 1] == -np.inf and np.all(od[0, 1] == 0.0)


def pin_decode_gt_bruteforce_and_2d(O):
    """1D max-pooled map: pure-Python brute force, and equal to the last row of
    the separately pinned 2D map when the last block holds only the newest token."""
    shape = Shape(1, 2, 1, 64 * 3 + 1, 8)
    q, k, _ = _qkv(shape, 82)
    got = O.decode_gt(q[:, :, -1], k)
    for h in range(2):
        s_ = [sum(q[0, h, -1, d] * k[0, 0, u, d] for d in range(8)) / math.sqrt(8) for u in range(shape.seq_len)]
        mx = max(s_)
        e = [math.exp(x - mx) for x in s_]
        tot = sum(e)
        for j in range(4):
            want = max(e[u] / tot for u in range(64 * j, min(64 * j + 64, shape.seq_len)))
            assert abs(got[0, h, j] - want) < 1e-14
    gt2 = O.maxpool_gt(q, k)
    assert np.abs(got - gt2[:, :, -1, :]).max() < 1e-14


def pin_decode_gate(O):
    """Compressed cache = torch max/min/avg pooling then W_k (per query head and
    per KV head); W_k = 0 gives uniform scores 1/nb; scores are a softmax of
    q . K'_j / sqrt(D) over every block (brute force)."""
    shape = Shape(1, 4, 2, 64 * 6 - 20, 8)
    q, k, _ = _qkv(shape, 83)
    rng = np.random.default_rng(8)
    nb = shape.nb
    for per_kv in (False, True):
        hw = 2 if per_kv else 4
        wk = rng.standard_normal((hw, 24, 8)) / 3.0
        kc = O.decode_kcomp(k, wk, 4, wk_per_kv_head=per_kv)
        for w in range(hw):
            g = w if per_kv else w // 2
            tk = torch.from_numpy(k[0, g])
            kp = np.stack([np.concatenate([tk[64 * j:64 * j + 64].max(0).values.numpy(),
                                           tk[64 * j:64 * j + 64].min(0).values.numpy(),
                                           tk[64 * j:64 * j + 64].mean(0).numpy()]) for j in range(nb)])
            assert np.abs(kc[0, w] - kp @ wk[w]).max() < 1e-12
        sc = O.decode_gate_scores(q[:, :, -1], kc, wk_per_kv_head=per_kv)
        for h in range(4):
            w = h // 2 if per_kv else h
            z = [sum(q[0, h, -1, d] * kc[0, w, j, d] for d in range(8)) / math.sqrt(8) for j in range(nb)]
            mx = max(z)
            e = [math.exp(x - mx) for x in z]
            for j in range(nb):
                assert abs(sc[0, h, j] - e[j] / sum(e)) < 1e-14
    kc0 = O.decode_kcomp(k, np.zeros((4, 24, 8)), 4)
    assert np.abs(O.decode_gate_scores(q[:, :, -1], kc0) - 1.0 / nb).max() < 1e-15


def pin_decode_masks(O):
    s_ = np.array([[[0.1, 0.3, 0.3, 0.05, 0.25]]])
    assert O.decode_threshold_mask(s_, 0.25).tolist() == [[[0, 1, 1, 0, 0]]]
    assert O.decode_topk_mask(s_, 2).tolist() == [[[0, 1, 1, 0, 0]]]
    assert O.decode_topk_mask(s_, 3).tolist() == [[[0, 1, 1, 0, 1]]]
    flat = np.full((1, 2, 6), 1.0 / 6)
    assert O.decode_topk_mask(flat, [2, 9]).tolist() == [[[1, 1, 0, 0, 0, 0], [1] * 6]]
    rng = np.random.default_rng(9)
    sc = rng.random((2, 3, 40))
    m = O.decode_topk_mask(sc, 7)
    for b in range(2):
        for h in range(3):
            keep = set(sorted(range(40), key=lambda j: (-sc[b, h, j], j))[:7])
            assert [int(x) for x in m[b, h]] == [1 if j in keep else 0 for j in range(40)]


# ----------------------------------------------------------------------------
# bfloat16 inputs: the oracle widens raw bf16 bit patterns (uint16), which is
# how every seeded generator hands Q, K and V to both sides
# ----------------------------------------------------------------------------
def _bf16_definition(bits: int) -> float:
    """Value of one bfloat16 pattern from the format's definition: 1 sign bit,
    8 exponent bits (bias 127), 7 fraction bits; exponent 0 is subnormal."""
    sign = -1.0 if bits >> 15 else 1.0
    e, m = (bits >> 7) & 0xFF, bits & 0x7F
    assert e != 0xFF, "inf/NaN patterns are not inputs"
    mag = math.ldexp(m, -133) if e == 0 else math.ldexp(128 + m, e - 134)
    return math.copysign(mag, sign)


def _torch_widen(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 through torch's own bfloat16 dtype."""
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def pin_bf16_bits_widening(O):
    """as_f64 on uint16 patterns gives the exact bfloat16 values: hand-checked
    patterns, every finite pattern against the format's definition and
    against torch's bfloat16, signed zeros kept."""
    table = {0x3F80: 1.0, 0xBF80: -1.0, 0xC020: -2.5, 0x4049: 3.140625, 0x3F81: 1.0 + 2.0 ** -7,
             0x0001: 2.0 ** -133, 0x0080: 2.0 ** -126, 0x7F7F: (2.0 - 2.0 ** -7) * 2.0 ** 127,
             0x0000: 0.0, 0x8000: -0.0}
    keys = np.array(sorted(table), dtype=np.uint16)
    got = O.as_f64(keys)
    assert got.dtype == np.float64
    for b, g in zip(keys.tolist(), got.tolist()):
        assert g == table[b] and math.copysign(1.0, g) == math.copysign(1.0, table[b]), (hex(b), g)
    allbits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = ((allbits >> 7) & 0xFF) != 0xFF
    pats = allbits[finite]
    got = O.as_f64(pats)
    want = np.array([_bf16_definition(int(b)) for b in pats.tolist()])
    assert np.array_equal(got, want) and np.array_equal(np.signbit(got), np.signbit(want))
    assert np.array_equal(got, _torch_widen(pats))
    # shape is kept
    assert O.as_f64(pats[:24].reshape(2, 3, 4)).shape == (2, 3, 4)


def pin_bf16_inputs_match_widened_floats(O):
    """Every entry point gives bit-identical results on bf16 bit patterns and
    on the same values widened to float64 by torch."""
    shape = Shape(1, 4, 2, 150, 16)
    qb, kb, vb = gen_qkv(shape, 21)
    qf, kf, vf = _torch_widen(qb), _torch_widen(kb), _torch_widen(vb)
    m = gen_tiny_mask(shape, 22, p_keep=0.6).mask
    ob, lb = O.attention(qb, kb, vb, m)
    of, lf = O.attention(qf, kf, vf, m)
    assert np.array_equal(ob, of) and np.array_equal(lb, lf)
    assert np.array_equal(O.maxpool_gt(qb, kb), O.maxpool_gt(qf, kf))
    assert np.array_equal(O.pool_q(qb), O.pool_q(qf)) and np.array_equal(O.pool_k(kb), O.pool_k(kf))
    rng = np.random.default_rng(23)
    wq = rng.standard_normal((4, 16, 16)).astype(np.float32)
    wk = rng.standard_normal((4, 48, 16)).astype(np.float32)
    assert np.array_equal(O.gate_scores(qb, kb, wq, wk), O.gate_scores(qf, kf, wq, wk))
    assert np.array_equal(O.gate_scores(qb, kb, wq, wk, rope_theta=1e4),
                          O.gate_scores(qf, kf, wq, wk, rope_theta=1e4))
    gt = O.maxpool_gt(qf, kf)
    lb_, gqb, gkb = O.gate_distill(qb, kb, wq, wk, gt)
    lf_, gqf, gkf = O.gate_distill(qf, kf, wq, wk, gt)
    assert lb_ == lf_ and np.array_equal(gqb, gqf) and np.array_equal(gkb, gkf)
    qd_b = qb[:, :, -1]
    qd_f = qf[:, :, -1]
    wd = rng.standard_normal((4, 48, 16)).astype(np.float32)
    kcb, kcf = O.decode_kcomp(kb, wd, 4), O.decode_kcomp(kf, wd, 4)
    assert np.array_equal(kcb, kcf)
    assert np.array_equal(O.decode_gate_scores(qd_b, kcb), O.decode_gate_scores(qd_f, kcf))
    dm = (rng.random((1, 4, shape.nb)) < 0.5).astype(np.uint8)
    for a, b in zip(O.decode_attention(qd_b, kb, vb, dm), O.decode_attention(qd_f, kf, vf, dm)):
        assert np.array_equal(a, b)
    assert np.array_equal(O.decode_gt(qd_b, kb), O.decode_gt(qd_f, kf))


ATTENTION_PINS = [pin_dense_matches_torch_sdpa, pin_probabilities_via_one_hot_v,
                  pin_constant_v_and_empty_rows, pin_q_zero_closed_form, pin_single_block_row,
                  pin_gqa_equals_mha, pin_bruteforce_python_loops]
GT_PINS = [pin_gt_matches_torch_maxpool, pin_gt_four_loop_bruteforce, pin_gt_properties,
           pin_gt_rows_match_full]
GATE_PINS = [pin_gate_hand_example, pin_gate_rows_sum_to_one, pin_gate_wq_zero_closed_form,
             pin_pool_matches_torch, pin_pool_k_constant_blocks, pin_gate_gqa_equals_mha]
MASK_PINS = [pin_threshold_strict, pin_threshold_nesting, pin_topk_counts, pin_topk_ties_low_index,
             pin_topk_bruteforce]
ROPE_PINS = [pin_rope_hand_complex, pin_rope_relative_and_orthogonal, pin_gate_rope_complex_bruteforce]
DISTILL_PINS = [pin_distill_finite_differences, pin_distill_loss_definition]
DECODE_PINS = [pin_decode_attention_matches_sdpa_and_prefill, pin_decode_gt_bruteforce_and_2d, pin_decode_gate,
               pin_decode_masks]
INPUT_PINS = [pin_bf16_bits_widening, pin_bf16_inputs_match_widened_floats]
ALL_PINS = INPUT_PINS + ATTENTION_PINS + GT_PINS + GATE_PINS + MASK_PINS + ROPE_PINS + DISTILL_PINS + DECODE_PINS
