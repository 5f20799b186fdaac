"""Plain fp64 CPU oracle for SeerAttention's gate, block mask, block-sparse
attention and 2D-maxpooled ground truth.

TEST INFRASTRUCTURE ONLY. Nothing on the library path may import, call or
execute this module; only the tests, the smoke check and the bench's CPU
baseline leg use it. It shares no code with the HIP library: it is written
from the definitions on the pages, in NumPy float64, with no blocking, fusion
or reordering beyond what those definitions state.

Pages cited (titles as they appear on the pages):
  [E] "SeerAttention: Learning Intrinsic Sparse Attention in Your LLMs" -- the
      paper-graph-ui explainer of arXiv 2410.13276.
  [R] "SeerAttention: Self-distilled Attention Gating for Efficient Long-context
      Prefilling" -- the OpenReview discussion (paperhub).

Readings taken where the pages are silent (each is listed with its reason in
the design notes):
  * the gate softmax is causal over key blocks j <= i (prefill of a causal LM);
  * gate scale 1/sqrt(d) with d the per-head dimension; no bias in W_q, W_k;
  * K pools are concatenated in the order [max | min | avg];
  * a ragged last block (seq_len not a multiple of the block) pools over the
    tokens it has;
  * threshold is strict (score > T); top-k keeps the k largest of the causal
    entries of a row, ties to the lower key-block index, all of them if the
    row has <= k causal entries;
  * upper-triangle mask entries are ignored, any non-zero byte means "compute";
  * a query whose active key set is empty gets O = 0 and LSE = -inf;
  * the ground truth is the raw max-pooled attention map (no renormalization);
  * block RoPE: theta' = theta / block with theta the model's RoPE base, at
    block positions, dims d and d + Dg/2 paired;
  * distillation: gt rows are normalized to sum 1 before the divergence, and
    the loss is the mean of the row divergences over all query-block rows; a
    row whose gt sums to 0 has no target and contributes nothing;
  * decode gating: see the readings above decode_kcomp.

Inputs may be bfloat16 bit patterns (uint16 arrays, as produced by the
seeded generators) or float arrays; they are widened exactly to float64.

Every function is pinned by tests under tests/ against closed forms, library
special cases and brute force (see the header of tests/test_oracle_pins.py).
"""
from __future__ import annotations

import numpy as np

BLOCK = 64


# --------------------------------------------------------------------------
# helpers
# --------------------------------------------------------------------------
def as_f64(x) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) or float arrays to float64 exactly."""
    a = np.asarray(x)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def n_blocks(seq_len: int, block: int = BLOCK) -> int:
    return -(-seq_len // block)


def _block_range(i: int, seq_len: int, block: int):
    return i * block, min((i + 1) * block, seq_len)


# --------------------------------------------------------------------------
# AttnGate: pooling ([E] section 3.4, "Input and pooling" and "Pooling Method
# Selection": AvgPool on Q; Max, Min and Avg pooling on K concatenated along
# the hidden dimension; kernel = stride = block size B = 64)
# --------------------------------------------------------------------------
def pool_q(q, block: int = BLOCK) -> np.ndarray:
    """Average of the Q rows of each block: [..., S, D] -> [..., nb, D]."""
    q = as_f64(q)
    S = q.shape[-2]
    nb = n_blocks(S, block)
    out = np.empty(q.shape[:-2] + (nb, q.shape[-1]), dtype=np.float64)
    for i in range(nb):
        a, b = _block_range(i, S, block)
        out[..., i, :] = q[..., a:b, :].mean(axis=-2)
    return out


def pool_k(k, block: int = BLOCK) -> np.ndarray:
    """[max | min | avg] of the K rows of each block: [..., S, D] -> [..., nb, 3D]."""
    k = as_f64(k)
    S, D = k.shape[-2], k.shape[-1]
    nb = n_blocks(S, block)
    out = np.empty(k.shape[:-2] + (nb, 3 * D), dtype=np.float64)
    for i in range(nb):
        a, b = _block_range(i, S, block)
        blk = k[..., a:b, :]
        out[..., i, 0:D] = blk.max(axis=-2)
        out[..., i, D:2 * D] = blk.min(axis=-2)
        out[..., i, 2 * D:3 * D] = blk.mean(axis=-2)
    return out


# --------------------------------------------------------------------------
# Block-level RoPE of the gate ([E] section 3.4, "Block-Level RoPE: Enabling
# Length Generalization": the gate takes Q and K before the model's rotary
# embedding and, after its own projections, applies a separate rotary
# embedding whose base theta' is the model's base theta divided by the block
# size, at block positions). The pages' formula is read literally: theta is
# the base, so the angle of pair d at block position i is
# i * (theta / block) ** (-2 d / Dg). Dims d and d + Dg/2 form a pair (the
# rotate-half layout of the Llama models the pages evaluate).
# --------------------------------------------------------------------------
def block_rope(x, theta: float, block: int = BLOCK, positions=None) -> np.ndarray:
    """Rotate gate vectors x [..., n, Dg] (Dg even) by their block positions.

    positions defaults to 0 .. n-1 (the block index of each row); passing the
    negated positions applies the inverse rotation.
    """
    x = as_f64(x)
    n, dg = x.shape[-2], x.shape[-1]
    half = dg // 2
    pos = np.arange(n, dtype=np.float64) if positions is None else np.asarray(positions, dtype=np.float64)
    inv_freq = (theta / block) ** (-2.0 * np.arange(half, dtype=np.float64) / dg)
    ang = pos[:, None] * inv_freq[None, :]                   # [n, Dg/2]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


# --------------------------------------------------------------------------
# AttnGate: projections and the block-level score ([E] section 3.4,
# "Linear transformation" and "Scoring via multiplication", the score
# equation: softmax((W_q P_q(Q)) (W_k P_k(K))^T / sqrt(d)), row-wise)
# --------------------------------------------------------------------------
def gate_scores(q, k, w_q, w_k, block: int = BLOCK, wk_per_kv_head: bool = False,
                rope_theta=None) -> np.ndarray:
    """Gate score [B, Hq, nb, nb]; row i is a softmax over key blocks j <= i, 0 above.

    q: [B, Hq, S, D]; k: [B, Hkv, S, D]; w_q: [Hq, D, Dg];
    w_k: [Hq, 3D, Dg] (one per query head) or [Hkv, 3D, Dg] (wk_per_kv_head).
    The pooled query of head h meets the pooled key of its KV head g = h // G.
    rope_theta: if given, the projected Q' and K' are rotated by block_rope
    (the gate then expects pre-RoPE Q and K).
    """
    w_q = as_f64(w_q)
    w_k = as_f64(w_k)
    B, Hq, S, D = np.shape(q)
    Hkv = np.shape(k)[1]
    G = Hq // Hkv
    nb = n_blocks(S, block)
    scale = 1.0 / np.sqrt(D)
    causal = np.tril(np.ones((nb, nb), dtype=bool))
    out = np.zeros((B, Hq, nb, nb), dtype=np.float64)
    for b in range(B):
        kp_cache = {}
        for h in range(Hq):
            g = h // G
            if g not in kp_cache:
                kp_cache[g] = pool_k(np.asarray(k)[b, g], block)
            qp = pool_q(np.asarray(q)[b, h], block)          # [nb, D]
            kp = kp_cache[g]                                  # [nb, 3D]
            qg = qp @ w_q[h]                                  # [nb, Dg]
            kg = kp @ (w_k[g] if wk_per_kv_head else w_k[h])  # [nb, Dg]
            if rope_theta is not None:
                qg = block_rope(qg, rope_theta, block)
                kg = block_rope(kg, rope_theta, block)
            z = (qg @ kg.T) * scale
            z = np.where(causal, z, -np.inf)
            z = z - z.max(axis=1, keepdims=True)
            e = np.exp(z)
            out[b, h] = e / e.sum(axis=1, keepdims=True)
    return out


# --------------------------------------------------------------------------
# Self-distillation step of the gate ([E] section 3.4, "Training Procedure":
# loss = D_KL(gt || score) with gt the 2D-maxpooled attention map and score
# the gate's output, both read as distributions over the key blocks of a query
# block). Readings: each causal row of gt is divided by its sum to give the
# target distribution p (the map itself is not normalized); terms with
# p_ij = 0 contribute 0; the loss is the mean of the row divergences over all
# B * Hq * nb query-block rows. The gradient is the derivative of that loss
# with respect to W_q and W_k.
# --------------------------------------------------------------------------
def gate_distill(q, k, w_q, w_k, gt, block: int = BLOCK, wk_per_kv_head: bool = False, rope_theta=None):
    """Loss and weight gradients of one distillation step.

    Same inputs as gate_scores plus gt [B, Hq, nb, nb] (raw max-pooled map).
    Returns (loss, grad_wq [Hq, D, Dg], grad_wk shaped like w_k), float64.
    """
    w_q = as_f64(w_q)
    w_k = as_f64(w_k)
    gt = np.asarray(gt, dtype=np.float64)
    B, Hq, S, D = np.shape(q)
    Hkv = np.shape(k)[1]
    G = Hq // Hkv
    nb = n_blocks(S, block)
    scale = 1.0 / np.sqrt(D)
    causal = np.tril(np.ones((nb, nb), dtype=bool))
    n_rows = B * Hq * nb
    neg_pos = -np.arange(nb, dtype=np.float64)
    loss = 0.0
    grad_wq = np.zeros_like(w_q)
    grad_wk = np.zeros_like(w_k)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            wk_idx = g if wk_per_kv_head else h
            qp = pool_q(np.asarray(q)[b, h], block)          # [nb, D]
            kp = pool_k(np.asarray(k)[b, g], block)          # [nb, 3D]
            qg = qp @ w_q[h]
            kg = kp @ w_k[wk_idx]
            if rope_theta is not None:
                qg = block_rope(qg, rope_theta, block)
                kg = block_rope(kg, rope_theta, block)
            z = np.where(causal, (qg @ kg.T) * scale, -np.inf)
            zmax = z.max(axis=1, keepdims=True)
            log_score = z - (zmax + np.log(np.exp(z - zmax).sum(axis=1, keepdims=True)))
            score = np.exp(log_score)                        # 0 above the diagonal
            target = np.where(causal, gt[b, h], 0.0)
            tsum = target.sum(axis=1, keepdims=True)
            valid = tsum > 0                                  # rows without target mass contribute nothing
            p = np.where(valid, target / np.where(valid, tsum, 1.0), 0.0)
            pos = p > 0
            loss += float(np.sum(p[pos] * (np.log(p[pos]) - log_score[pos])))
            # d loss / d z = (score - p) / n_rows on causal entries of valid rows (softmax + KL)
            dz = np.where(causal & valid, score - p, 0.0) / n_rows
            dqg = (dz @ kg) * scale
            dkg = (dz.T @ qg) * scale
            if rope_theta is not None:                        # rotations are orthogonal: back-rotate
                dqg = block_rope(dqg, rope_theta, block, positions=neg_pos)
                dkg = block_rope(dkg, rope_theta, block, positions=neg_pos)
            grad_wq[h] += qp.T @ dqg
            grad_wk[wk_idx] += kp.T @ dkg
    return loss / n_rows, grad_wq, grad_wk


# --------------------------------------------------------------------------
# Decode-stage gating ([R], the responses on decoding: for decode the gate
# drops the query branch's pooling and linear map, so the query of each new
# token meets a small compressed K cache -- pooled keys taken after the
# model's RoPE -- and the gate is distilled against the attention map
# max-pooled along the sequence only; the selected blocks' K and V are the
# only ones read).
# Readings: the decode query is the model's (post-RoPE) query of the newest
# token and it sees every cached key; the compressed cache holds the keys
# [max | min | avg]-pooled per block, as for the prefill gate, projected by
# W_k to the head dimension D (W_k is 3D x D, one per query head or one per
# KV head), so score_j = softmax over all blocks j of q . K'_j / sqrt(D); no
# extra block-level RoPE; masks keep the blocks with score > T, or the k
# largest scores (ties to the lower block index, all blocks if nb <= k).
# --------------------------------------------------------------------------
def decode_kcomp(k, w_k, heads_q: int, block: int = BLOCK, wk_per_kv_head: bool = False) -> np.ndarray:
    """Compressed K cache K' [B, Hwk, nb, D] = pool_k(K) @ W_k.

    k: [B, Hkv, S, D]; w_k: [Hwk, 3D, D] with Hwk = Hkv (wk_per_kv_head) or
    heads_q (query head h uses the pooled keys of its KV head h // G).
    """
    w_k = as_f64(w_k)
    B, Hkv = np.shape(k)[:2]
    G = heads_q // Hkv
    hwk = Hkv if wk_per_kv_head else heads_q
    out = []
    for b in range(B):
        rows = []
        for w in range(hwk):
            g = w if wk_per_kv_head else w // G
            rows.append(pool_k(np.asarray(k)[b, g], block) @ w_k[w])
        out.append(np.stack(rows))
    return np.stack(out)


def decode_gate_scores(q, kcomp, wk_per_kv_head: bool = False) -> np.ndarray:
    """Decode gate score [B, Hq, nb]: softmax over all key blocks j of q . K'_j / sqrt(D).

    q: [B, Hq, D], one query per head; kcomp: [B, Hwk, nb, D] from decode_kcomp.
    """
    q = as_f64(q)
    kcomp = np.asarray(kcomp, dtype=np.float64)
    B, Hq, D = q.shape
    hwk = kcomp.shape[1]
    G = Hq // hwk if wk_per_kv_head else 1
    out = np.zeros((B, Hq, kcomp.shape[2]))
    for b in range(B):
        for h in range(Hq):
            z = kcomp[b, h // G if wk_per_kv_head else h] @ q[b, h] / np.sqrt(D)
            e = np.exp(z - z.max())
            out[b, h] = e / e.sum()
    return out


def decode_threshold_mask(scores, threshold: float) -> np.ndarray:
    """uint8 [B, Hq, nb]: 1 where score > threshold (strict)."""
    return (np.asarray(scores, dtype=np.float64) > threshold).astype(np.uint8)


def decode_topk_mask(scores, k) -> np.ndarray:
    """uint8 [B, Hq, nb] keeping the k largest scores of each (b, h) row, ties to the lower j."""
    s = np.asarray(scores, dtype=np.float64)
    B, H, nb = s.shape
    ks = np.broadcast_to(np.asarray(k, dtype=np.int64), (H,))
    out = np.zeros(s.shape, dtype=np.uint8)
    for b in range(B):
        for h in range(H):
            order = np.argsort(-s[b, h], kind="stable")
            out[b, h, order[:min(int(ks[h]), nb)]] = 1
    return out


def decode_attention(q, k, v, block_mask=None, block: int = BLOCK):
    """One query per head against every cached key, restricted to active blocks.

    q: [B, Hq, D]; k, v: [B, Hkv, S, D]; block_mask: [B, Hq, nb] (non-zero =
    read the block) or None (all blocks). Returns (O [B, Hq, Dv], LSE [B, Hq]),
    O = 0 and LSE = -inf when no block is active.
    """
    q = as_f64(q)
    B, Hq, D = q.shape
    Hkv, S = np.shape(k)[1], np.shape(k)[2]
    G = Hq // Hkv
    nb = n_blocks(S, block)
    o = np.zeros((B, Hq, np.shape(v)[-1]))
    lse = np.full((B, Hq), -np.inf)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            blocks = range(nb) if block_mask is None else [j for j in range(nb) if block_mask[b, h, j] != 0]
            keys = [u for j in blocks for u in range(*_block_range(j, S, block))]
            if not keys:
                continue
            kk = as_f64(np.asarray(k)[b, g, keys])
            vv = as_f64(np.asarray(v)[b, g, keys])
            s_ = kk @ q[b, h] / np.sqrt(D)
            mx = s_.max()
            e = np.exp(s_ - mx)
            o[b, h] = e @ vv / e.sum()
            lse[b, h] = mx + np.log(e.sum())
    return o, lse


def decode_gt(q, k, block: int = BLOCK) -> np.ndarray:
    """1D max-pooled attention map [B, Hq, nb]: for each block j, the largest
    attention probability of the decode query on a key of that block (full
    attention over every cached key)."""
    q = as_f64(q)
    B, Hq, D = q.shape
    Hkv, S = np.shape(k)[1], np.shape(k)[2]
    G = Hq // Hkv
    nb = n_blocks(S, block)
    out = np.zeros((B, Hq, nb))
    for b in range(B):
        for h in range(Hq):
            s_ = as_f64(np.asarray(k)[b, h // G]) @ q[b, h] / np.sqrt(D)
            p = np.exp(s_ - s_.max())
            p /= p.sum()
            for j in range(nb):
                a, e = _block_range(j, S, block)
                out[b, h, j] = p[a:e].max()
    return out


# --------------------------------------------------------------------------
# Binary block mask ([E] section 3.4, "Inference Procedure", Method 1 TopK and
# Method 2 thresholding; [R] response 3.3 on mask generation: mask = o > T,
# torch.topk per row)
# --------------------------------------------------------------------------
def threshold_mask(scores, threshold: float) -> np.ndarray:
    """uint8 mask: 1 where score > threshold (strict) on causal entries j <= i."""
    s = np.asarray(scores, dtype=np.float64)
    nb = s.shape[-1]
    causal = np.tril(np.ones((nb, nb), dtype=bool))
    return ((s > threshold) & causal).astype(np.uint8)


def topk_mask(scores, k) -> np.ndarray:
    """uint8 mask keeping, per row i, the k largest causal scores (j <= i).

    `k` is an int (uniform) or a sequence of per-query-head values.
    Ties go to the lower j; a row with i+1 <= k keeps all its causal entries.
    """
    s = np.asarray(scores, dtype=np.float64)
    B, H, nb, _ = s.shape
    ks = np.broadcast_to(np.asarray(k, dtype=np.int64), (H,))
    out = np.zeros(s.shape, dtype=np.uint8)
    for b in range(B):
        for h in range(H):
            kk = int(ks[h])
            for i in range(nb):
                row = s[b, h, i, :i + 1]
                order = np.argsort(-row, kind="stable")   # descending, ties keep lower j first
                out[b, h, i, order[:min(kk, i + 1)]] = 1
    return out


# --------------------------------------------------------------------------
# Block-sparse attention ([E] section 3.4, "Block-sparse FlashAttention
# kernel": a tile with b_ij = 0 is skipped entirely, a tile with b_ij = 1 is
# ordinary attention; equivalently, masked blocks take -inf before the
# softmax). Causal prefill: key u is visible to query t only if u <= t.
# --------------------------------------------------------------------------
def attention_rows(q, k, v, block_mask, rows, block: int = BLOCK):
    """Attention output for selected (b, h, query block) rows.

    q: [B, Hq, S, D]; k, v: [B, Hkv, S, D]; block_mask: [B, Hq, nb, nb]
    (non-zero = compute) or None for dense causal attention.
    rows: iterable of (b, h, i). Returns (O list of [rows_in_block, D],
    LSE list of [rows_in_block]) in float64, LSE in natural log.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(D)
    outs, lses = [], []
    for (b, h, i) in rows:
        g = h // G
        t0, t1 = _block_range(i, S, block)
        qi = as_f64(q[b, h, t0:t1])                                   # [n, D]
        if block_mask is None:
            active = np.arange(i + 1)
        else:
            row = np.asarray(block_mask[b, h, i])
            active = np.array([j for j in range(i + 1) if row[j] != 0], dtype=np.int64)
        o = np.zeros((t1 - t0, v.shape[-1]), dtype=np.float64)
        lse = np.full((t1 - t0,), -np.inf, dtype=np.float64)
        if active.size:
            keys = np.concatenate([np.arange(*_block_range(int(j), S, block)) for j in active])
            kk = as_f64(k[b, g, keys])                                # [m, D]
            vv = as_f64(v[b, g, keys])
            s = (qi @ kk.T) * scale                                   # [n, m]
            tq = np.arange(t0, t1)[:, None]
            s = np.where(keys[None, :] <= tq, s, -np.inf)
            mx = s.max(axis=1, keepdims=True)
            has = np.isfinite(mx[:, 0])
            mx = np.where(np.isfinite(mx), mx, 0.0)
            e = np.exp(s - mx)
            den = e.sum(axis=1, keepdims=True)
            p = np.divide(e, den, out=np.zeros_like(e), where=den > 0)
            o = p @ vv
            lse = np.where(has, mx[:, 0] + np.log(np.where(has, den[:, 0], 1.0)), -np.inf)
        outs.append(o)
        lses.append(lse)
    return outs, lses


def attention(q, k, v, block_mask=None, block: int = BLOCK):
    """Full attention output O [B, Hq, S, Dv] and LSE [B, Hq, S] (float64)."""
    q = np.asarray(q)
    B, Hq, S, D = q.shape
    nb = n_blocks(S, block)
    rows = [(b, h, i) for b in range(B) for h in range(Hq) for i in range(nb)]
    outs, lses = attention_rows(q, k, v, block_mask, rows, block)
    O = np.zeros((B, Hq, S, np.shape(v)[-1]))
    L = np.zeros((B, Hq, S))
    for (b, h, i), o, l in zip(rows, outs, lses):
        t0, t1 = _block_range(i, S, block)
        O[b, h, t0:t1] = o
        L[b, h, t0:t1] = l
    return O, L


# --------------------------------------------------------------------------
# 2D-maxpooled ground truth ([E] section 3.4, "Training Procedure", the gt
# equation: gt = MaxPool2D(softmax(Q K^T / sqrt(d))) with a B x B kernel and
# stride B; only when every score in a block is small is its pooled value small)
# --------------------------------------------------------------------------
def maxpool_gt_rows(q, k, rows, block: int = BLOCK):
    """Rows of the max-pooled causal attention map.

    For each (b, h, i) returns a float64 vector of length nb:
    gt[j] = max over queries t in block i and keys u in block j with u <= t of
    softmax_u(q_t . k_u / sqrt(D)) (full causal softmax, no block mask);
    gt[j] = 0 for j > i.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    nb = n_blocks(S, block)
    scale = 1.0 / np.sqrt(D)
    out = []
    for (b, h, i) in rows:
        g = h // G
        t0, t1 = _block_range(i, S, block)
        qi = as_f64(q[b, h, t0:t1])
        kk = as_f64(k[b, g, :t1])
        s = (qi @ kk.T) * scale                                       # [n, t1]
        tq = np.arange(t0, t1)[:, None]
        s = np.where(np.arange(t1)[None, :] <= tq, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        e = np.exp(s)
        p = e / e.sum(axis=1, keepdims=True)
        row = np.zeros(nb, dtype=np.float64)
        for j in range(i + 1):
            a, bb = _block_range(j, S, block)
            row[j] = p[:, a:bb].max()
        out.append(row)
    return out


def maxpool_gt(q, k, block: int = BLOCK) -> np.ndarray:
    """Full ground-truth map [B, Hq, nb, nb] (float64)."""
    q = np.asarray(q)
    B, Hq, S, D = q.shape
    nb = n_blocks(S, block)
    rows = [(b, h, i) for b in range(B) for h in range(Hq) for i in range(nb)]
    gt = np.zeros((B, Hq, nb, nb))
    for (b, h, i), r in zip(rows, maxpool_gt_rows(q, k, rows, block)):
        gt[b, h, i] = r
    return gt
