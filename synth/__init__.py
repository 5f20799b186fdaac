"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module only draws random numbers and packs them; it holds none of the
method's arithmetic (no pooling, projection, softmax, masking or attention).
Both the fp64 oracle and the HIP library are fed from here, so neither has to
import the other.

Workloads follow the shapes of the Llama-3.1-8B attention layer that the
SeerAttention pages evaluate on (32 query heads, 8 KV heads, head dim 128,
block 64), with N(0, 1) activations rounded to bfloat16.

Every generator takes an integer seed and uses NumPy's PCG64 with a fixed
draw order, so a record of (generator, seed, sizes) reproduces its inputs.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

BLOCK = 64


# --------------------------------------------------------------------------
# bfloat16 packing (round-to-nearest-even from fp32), kept as raw uint16 bits
# --------------------------------------------------------------------------
def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """fp32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    flat_in, flat_out = x.reshape(-1), out.reshape(-1)
    step = 1 << 24                        # bounded temporaries for large tensors
    for a in range(0, flat_in.size, step):
        u = flat_in[a:a + step].view(np.uint32)
        # finite inputs only: the carry never leaves 32 bits below the NaN range
        flat_out[a:a + step] = ((u + np.uint32(0x7FFF) + ((u >> 16) & np.uint32(1))) >> 16).astype(np.uint16)
    return out


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> exactly equal fp32 values."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bfloat16 and return them as fp32."""
    return f32_from_bf16_bits(bf16_bits_from_f32(x))


@dataclass
class Shape:
    batch: int
    heads_q: int
    heads_kv: int
    seq_len: int
    head_dim: int
    block: int = BLOCK

    @property
    def nb(self) -> int:
        return -(-self.seq_len // self.block)

    @property
    def group(self) -> int:
        return self.heads_q // self.heads_kv


def gen_qkv(shape: Shape, seed: int, want_v: bool = True):
    """Q [B,Hq,S,D], K [B,Hkv,S,D], V [B,Hkv,S,D] ~ N(0,1), rounded to bf16.

    Returned as uint16 bf16 bit patterns (row-major BHSD). Draw order: Q, K, V.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    b, hq, hk, s, d = shape.batch, shape.heads_q, shape.heads_kv, shape.seq_len, shape.head_dim
    q = bf16_bits_from_f32(rng.standard_normal((b, hq, s, d), dtype=np.float32))
    k = bf16_bits_from_f32(rng.standard_normal((b, hk, s, d), dtype=np.float32))
    v = bf16_bits_from_f32(rng.standard_normal((b, hk, s, d), dtype=np.float32)) if want_v else None
    return q, k, v


# --------------------------------------------------------------------------
# Block masks for the attention-only workloads
# --------------------------------------------------------------------------
@dataclass
class MaskInfo:
    mask: np.ndarray                       # uint8 [B, Hq, nb, nb], lower triangle meaningful
    target_sparsity: np.ndarray            # per (b, h) target causal-block sparsity
    realized_sparsity: np.ndarray          # per (b, h) realized causal-block sparsity
    stripes: list = field(default_factory=list)

    @property
    def mean_sparsity(self) -> float:
        return float(self.realized_sparsity.mean())


def causal_block_count(nb: int) -> int:
    return nb * (nb + 1) // 2


def _realized(mask: np.ndarray) -> np.ndarray:
    nb = mask.shape[-1]
    tri = np.tril(np.ones((nb, nb), dtype=bool))
    kept = (mask.astype(bool) & tri).sum(axis=(-1, -2))
    return 1.0 - kept / causal_block_count(nb)


def per_head_sparsity(n_heads: int, lo: float, hi: float, mean: float,
                      rng: np.random.Generator, tol: float = 1e-4) -> np.ndarray:
    """Per-head sparsities drawn from U[lo, hi], shifted so their mean is `mean`.

    U[lo, hi] alone has mean (lo+hi)/2, which need not equal the wanted mean,
    so the draws are shifted by (mean - sample mean) and clipped to [lo, hi];
    the shift is repeated until the sample mean is within `tol`.
    """
    s = rng.uniform(lo, hi, size=n_heads)
    for _ in range(1000):
        s = np.clip(s + (mean - s.mean()), lo, hi)
        if abs(s.mean() - mean) < tol:
            break
    return s


def gen_block_mask(shape: Shape, seed: int, sparsity, n_stripes: int = 4,
                   keep_diag: bool = True, keep_sink: bool = True) -> MaskInfo:
    """Seeded causal block mask with forced diagonal + sink and vertical stripes.

    Per (batch, query head):
      * the diagonal block (i, i) and the sink block (i, 0) are kept for all i;
      * `n_stripes` distinct key-block columns c in [1, nb-1] are kept for all i >= c;
      * every other causal block is kept i.i.d. with the probability that makes
        the expected kept count equal round((1 - s_h) * nb(nb+1)/2).
    `sparsity` is a scalar or an array of per-head targets s_h.
    The realized sparsity is measured afterwards and returned.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    B, H, nb = shape.batch, shape.heads_q, shape.nb
    s_target = np.broadcast_to(np.asarray(sparsity, dtype=np.float64), (B, H)).copy()
    tri = np.tril(np.ones((nb, nb), dtype=bool))
    mask = np.zeros((B, H, nb, nb), dtype=np.uint8)
    stripes = []
    total = causal_block_count(nb)
    for b in range(B):
        for h in range(H):
            forced = np.zeros((nb, nb), dtype=bool)
            if keep_diag:
                forced[np.arange(nb), np.arange(nb)] = True
            if keep_sink:
                forced[:, 0] = True
            cols = []
            if n_stripes > 0 and nb > 1:
                cols = rng.choice(np.arange(1, nb), size=min(n_stripes, nb - 1), replace=False)
                for c in cols:
                    forced[c:, c] = True
            forced &= tri
            stripes.append(sorted(int(c) for c in cols))
            n_forced = int(forced.sum())
            remaining = total - n_forced
            want = round((1.0 - s_target[b, h]) * total)
            p = 0.0 if remaining <= 0 else min(1.0, max(0.0, (want - n_forced) / remaining))
            fill = rng.random((nb, nb)) < p
            mask[b, h] = (forced | (fill & tri)).astype(np.uint8)
    return MaskInfo(mask=mask, target_sparsity=s_target, realized_sparsity=_realized(mask),
                    stripes=stripes)


def gen_tiny_mask(shape: Shape, seed: int, p_keep: float = 0.5) -> MaskInfo:
    """Lower-triangular block mask: diagonal and block 0 kept, others kept with p."""
    rng = np.random.Generator(np.random.PCG64(seed))
    B, H, nb = shape.batch, shape.heads_q, shape.nb
    tri = np.tril(np.ones((nb, nb), dtype=bool))
    mask = (rng.random((B, H, nb, nb)) < p_keep) & tri
    mask[..., np.arange(nb), np.arange(nb)] = True
    mask[..., :, 0] = True
    mask = mask.astype(np.uint8)
    return MaskInfo(mask=mask, target_sparsity=np.full((B, H), float("nan")),
                    realized_sparsity=_realized(mask))


def gen_random_upper_noise(mask: np.ndarray, seed: int) -> np.ndarray:
    """Copy of `mask` with random non-zero bytes above the diagonal.

    The library and the oracle must both ignore the upper triangle; this makes
    tests able to check that.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    nb = mask.shape[-1]
    upper = np.triu(np.ones((nb, nb), dtype=bool), k=1)
    noise = rng.integers(1, 256, size=mask.shape, dtype=np.uint8)
    out = mask.copy()
    out[..., upper] = noise[..., upper]
    return out


# --------------------------------------------------------------------------
# Gate inputs: planted structure + random-init gate weights
# --------------------------------------------------------------------------
@dataclass
class PlantedInfo:
    hot_blocks: np.ndarray   # [B, Hkv, n_hot] key-block indices
    directions: np.ndarray   # [B, Hkv, D] unit vectors


def gen_planted_qk(shape: Shape, seed: int, n_hot: int = 3, shift: float = 1.5):
    """Q, K ~ N(0,1) with planted hot key blocks, rounded to bf16 (uint16 bits).

    For every (batch, KV head) a unit direction u is drawn; the K rows of
    `n_hot` distinct random key blocks get +shift*u, and every Q row of the
    query heads in that KV group gets +shift*u, so those blocks draw extra
    attention from every query. Draw order: Q, K, V, then per (b, g): u, hot blocks.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    B, Hq, Hk, S, D = shape.batch, shape.heads_q, shape.heads_kv, shape.seq_len, shape.head_dim
    G = Hq // Hk
    q = rng.standard_normal((B, Hq, S, D), dtype=np.float32)
    k = rng.standard_normal((B, Hk, S, D), dtype=np.float32)
    v = rng.standard_normal((B, Hk, S, D), dtype=np.float32)
    nb = shape.nb
    hot = np.zeros((B, Hk, n_hot), dtype=np.int64)
    dirs = np.zeros((B, Hk, D), dtype=np.float32)
    for b in range(B):
        for g in range(Hk):
            u = rng.standard_normal(D)
            u = (u / np.linalg.norm(u)).astype(np.float32)
            blocks = np.sort(rng.choice(nb, size=min(n_hot, nb), replace=False))
            hot[b, g, :len(blocks)] = blocks
            dirs[b, g] = u
            for blk in blocks:
                k[b, g, blk * shape.block:(blk + 1) * shape.block] += shift * u
            q[b, g * G:(g + 1) * G] += shift * u
    return (bf16_bits_from_f32(q), bf16_bits_from_f32(k), bf16_bits_from_f32(v),
            PlantedInfo(hot_blocks=hot, directions=dirs))


def gen_gate_weights(heads_q: int, head_dim: int, gate_dim: int, seed: int,
                     heads_w_k: int | None = None, var: float | None = None):
    """Random-init gate weights ~ N(0, var) in fp32 (default var = 1/gate_dim).

    W_q [Hq, D, Dg] and W_k [Hwk, 3D, Dg] with Hwk = Hq (one W_k per query head)
    unless `heads_w_k` is given (e.g. Hkv for one W_k per KV head).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    var = 1.0 / gate_dim if var is None else var
    std = math.sqrt(var)
    hwk = heads_q if heads_w_k is None else heads_w_k
    wq = (rng.standard_normal((heads_q, head_dim, gate_dim), dtype=np.float32) * np.float32(std))
    wk = (rng.standard_normal((hwk, 3 * head_dim, gate_dim), dtype=np.float32) * np.float32(std))
    return wq.astype(np.float32), wk.astype(np.float32)


# --------------------------------------------------------------------------
# Named workloads with recorded seeds
# --------------------------------------------------------------------------
SEED_BASE = 1000

WORKLOADS = {
    # tiny causal block-sparse attention: 2 query heads on 1 KV head, D 64, S 512
    "tiny_s512": dict(shape=Shape(1, 2, 1, 512, 64), sparsity="tiny", out="f32", seed=SEED_BASE + 1),
    # Llama-3.1-8B-shaped layer at 8k, 50% causal-block sparsity
    "llama8b_s8k_50": dict(shape=Shape(1, 32, 8, 8192, 128), sparsity=0.5, out="bf16", seed=SEED_BASE + 2),
    # 32k, per-head sparsity in [0.8, 0.97], mean 0.9
    "llama8b_s32k_90": dict(shape=Shape(1, 32, 8, 32768, 128), sparsity=(0.8, 0.97, 0.9), out="bf16",
                            seed=SEED_BASE + 3),
    # 128k, same generator (headline)
    "llama8b_s128k_90": dict(shape=Shape(1, 32, 8, 131072, 128), sparsity=(0.8, 0.97, 0.9), out="bf16",
                             seed=SEED_BASE + 4),
    # gate + ground-truth path at 32k with planted hot blocks, T = 5e-4
    "gate_gt_s32k": dict(shape=Shape(1, 32, 8, 32768, 128), sparsity="gate", out="bf16", seed=SEED_BASE + 5,
                         gate_dim=128, threshold=5e-4),
}


def workload_mask(name: str, shape: Shape | None = None) -> MaskInfo:
    """The block mask of a named attention workload (optionally at another shape)."""
    w = WORKLOADS[name]
    shape = shape or w["shape"]
    sp = w["sparsity"]
    mseed = w["seed"] * 7 + 3
    if sp == "tiny":
        return gen_tiny_mask(shape, mseed)
    if isinstance(sp, tuple):
        lo, hi, mean = sp
        rng = np.random.Generator(np.random.PCG64(w["seed"] * 11 + 5))
        s = per_head_sparsity(shape.batch * shape.heads_q, lo, hi, mean, rng).reshape(shape.batch, shape.heads_q)
        return gen_block_mask(shape, mseed, s)
    return gen_block_mask(shape, mseed, float(sp))
