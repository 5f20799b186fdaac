"""Property checks of the fp64 oracle on randomized shapes (hypothesis).

The fixed-seed pins in tests/oracle_pins.py fix the oracle against library
routines, closed forms and brute force at a few shapes; these draw the shapes
(ragged lengths, GQA groups, masks, thresholds, k) at random and check the
same independent facts: block-masked attention equals torch's fp64 SDPA with
the token-level mask written out, gate rows are softmax rows over the causal
blocks, the threshold and top-k masks are what their definitions say
(checked by sorting), the maxpooled map equals torch's max_pool2d of the
SDPA probabilities, and the block RoPE is a rotation that the negated
positions undo.
"""
import numpy as np
import torch
import torch.nn.functional as F
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle.seer_oracle as O
from synth import Shape, f32_from_bf16_bits, gen_qkv

SETTINGS = settings(max_examples=60, deadline=None, suppress_health_check=[HealthCheck.too_slow])


def _qkv(shape, seed):
    q, k, v = gen_qkv(shape, seed)
    return tuple(f32_from_bf16_bits(x).astype(np.float64) for x in (q, k, v))


shapes = st.builds(
    lambda b, hkv, g, s, d: Shape(b, hkv * g, hkv, s, d),
    st.integers(1, 2), st.integers(1, 2), st.sampled_from([1, 2, 4]), st.integers(1, 300),
    st.sampled_from([4, 8, 16]))


@SETTINGS
@given(shape=shapes, seed=st.integers(0, 2**31 - 1), p_keep=st.floats(0.0, 1.0))
def test_masked_attention_matches_sdpa(shape, seed, p_keep):
    """O and LSE of a random block mask (diagonal blocks on, so no row is empty)
    equal torch SDPA / logsumexp with the expanded token-level causal mask."""
    q, k, v = _qkv(shape, seed % 100000)
    nb, S = shape.nb, shape.seq_len
    rng = np.random.default_rng(seed)
    m = (rng.random((shape.batch, shape.heads_q, nb, nb)) < p_keep).astype(np.uint8)
    m[..., np.arange(nb), np.arange(nb)] = 1
    o, lse = O.attention(q, k, v, m)
    tok = np.arange(S) // 64
    allowed = m[:, :, tok[:, None], tok[None, :]].astype(bool) & np.tril(np.ones((S, S), dtype=bool))
    G = shape.heads_q // shape.heads_kv
    kk = np.repeat(k, G, axis=1)
    vv = np.repeat(v, G, axis=1)
    tq, tk, tv, tm = (torch.from_numpy(np.ascontiguousarray(x)) for x in (q, kk, vv, allowed))
    ref = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=tm).numpy()
    scores = (tq @ tk.transpose(-1, -2)) / np.sqrt(shape.head_dim)
    ref_lse = torch.logsumexp(scores.masked_fill(~tm, float("-inf")), dim=-1).numpy()
    assert np.abs(o - ref).max() < 1e-12
    assert np.abs(lse - ref_lse).max() < 1e-12


gate_shapes = st.builds(
    lambda b, hkv, g, nbk, tail, d: Shape(b, hkv * g, hkv, 64 * nbk - tail, d),
    st.integers(1, 2), st.integers(1, 2), st.sampled_from([1, 2]), st.integers(1, 12), st.integers(0, 63),
    st.sampled_from([8, 16]))


@SETTINGS
@given(shape=gate_shapes, seed=st.integers(0, 2**31 - 1), per_kv=st.booleans(), dg=st.sampled_from([4, 8]),
       t_lo=st.floats(0.0, 0.5), t_gap=st.floats(0.0, 0.5), k=st.integers(1, 14))
def test_gate_rows_and_masks(shape, seed, per_kv, dg, t_lo, t_gap, k):
    q, k_, _ = _qkv(shape, seed % 100000)
    rng = np.random.default_rng(seed)
    D, Hq = shape.head_dim, shape.heads_q
    hw = shape.heads_kv if per_kv else Hq
    wq = rng.standard_normal((Hq, D, dg)) / np.sqrt(D)
    wk = rng.standard_normal((hw, 3 * D, dg)) / np.sqrt(3 * D)
    sc = O.gate_scores(q, k_, wq, wk, wk_per_kv_head=per_kv)
    nb = shape.nb
    causal = np.tril(np.ones((nb, nb), dtype=bool))
    # softmax rows over the causal blocks
    assert np.abs(sc.sum(-1) - 1.0).max() < 1e-12
    assert np.all(sc[..., ~causal] == 0.0) and sc.min() >= 0.0
    # threshold: exactly the causal entries above T, nested in T
    t1, t2 = t_lo, t_lo + t_gap
    m1, m2 = O.threshold_mask(sc, t1), O.threshold_mask(sc, t2)
    assert np.array_equal(m1.astype(bool), (sc > t1) & causal)
    assert np.all(m2 <= m1)
    # top-k: the first min(k, i+1) entries of the row sorted by (-score, index)
    tk = O.topk_mask(sc, k)
    for b in range(shape.batch):
        for h in range(Hq):
            for i in range(nb):
                row = sc[b, h, i, :i + 1]
                order = np.lexsort((np.arange(i + 1), -row))
                want = np.zeros(nb, dtype=np.uint8)
                want[order[:min(k, i + 1)]] = 1
                assert np.array_equal(tk[b, h, i], want)


@SETTINGS
@given(S=st.integers(1, 200), g=st.sampled_from([1, 2]), seed=st.integers(0, 2**31 - 1))
def test_maxpool_gt_matches_torch(S, g, seed):
    shape = Shape(1, 2 * g, 2, S, 8)
    q, k, _ = _qkv(shape, seed % 100000)
    eye = np.broadcast_to(np.eye(S), (1, 2, S, S)).copy()
    tq, tk, te = (torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, eye))
    P = F.scaled_dot_product_attention(tq, tk, te, is_causal=True, enable_gqa=True)
    ref = F.max_pool2d(P, 64, 64, ceil_mode=True).numpy()
    assert np.abs(O.maxpool_gt(q, k) - ref).max() < 1e-12


@SETTINGS
@given(n=st.integers(1, 40), half=st.integers(1, 8), theta=st.floats(10.0, 1e6), seed=st.integers(0, 2**31 - 1))
def test_block_rope_is_an_invertible_rotation(n, half, theta, seed):
    x = np.random.default_rng(seed).standard_normal((3, n, 2 * half))
    y = O.block_rope(x, theta)
    # each pair (d, d + Dg/2) keeps its length; position 0 is not rotated
    assert np.allclose(x[..., :half] ** 2 + x[..., half:] ** 2, y[..., :half] ** 2 + y[..., half:] ** 2,
                       rtol=1e-12, atol=1e-12)
    assert np.array_equal(y[:, 0], x[:, 0])
    back = O.block_rope(y, theta, positions=-np.arange(n))
    assert np.abs(back - x).max() < 1e-12
