"""GPU parity of the ground-truth kernel and of the AttnGate (scores, masks)
against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth import Shape
from gpu_util import MASK_BAND, check_close, check_lse, dev_bf16, dev_f32, host, say

pytestmark = pytest.mark.gpu


def _seer():
    import learned_block_sparse_attngate_amd as seer
    seer.load_library()
    return seer


# ---------------------------------------------------------------------------
# ground truth
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("shape,dt", [(Shape(1, 2, 1, 200, 64), torch.float32),
                                      (Shape(1, 4, 2, 1000, 128), torch.bfloat16),
                                      (Shape(2, 2, 2, 64, 128), torch.float32)],
                         ids=["s200_d64", "s1000_d128", "s64_b2"])
def test_gt_matches_oracle(shape, dt):
    seer = _seer()
    say(f"[gt] shape={shape}")
    q, k, v = synth.gen_qkv(shape, 50)
    out, lse, gt = seer.seer_attn_maxpool_gt(dev_bf16(q), dev_bf16(k), dev_bf16(v), out_dtype=dt, want_lse=True)
    torch.cuda.synchronize()
    gt_ref = oracle.maxpool_gt(q, k)
    o_ref, l_ref = oracle.attention(q, k, v, None)
    g = host(gt)
    # fp32 row statistics: the runs show max-abs ~1e-7 and relative ~1e-6
    check_close(g, gt_ref, "gt", max_abs=1e-6, mean_abs=1e-7)
    rel = np.abs(g - gt_ref)[gt_ref > 1e-6] / gt_ref[gt_ref > 1e-6]
    say(f"  gt max relative error on entries > 1e-6: {rel.max():.3e}")
    assert rel.max() < 1e-4
    assert np.all(g[..., np.triu_indices(shape.nb, 1)[0], np.triu_indices(shape.nb, 1)[1]] == 0.0)
    check_close(host(out), o_ref, "gt-kernel O", out_dtype=dt)
    check_lse(host(lse), l_ref, "gt-kernel LSE")


def test_gt_output_equals_dense_bitwise():
    seer = _seer()
    shape = Shape(1, 4, 2, 700, 128)
    q, k, v = (dev_bf16(x) for x in synth.gen_qkv(shape, 51))
    a, la, _ = seer.seer_attn_maxpool_gt(q, k, v, out_dtype=torch.float32, want_lse=True)
    b, lb = seer.seer_block_sparse_attn_fwd(q, k, v, None, out_dtype=torch.float32, want_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(la, lb)


# ---------------------------------------------------------------------------
# gate
# ---------------------------------------------------------------------------
def _gate_inputs(shape, seed, dg, per_kv=False):
    q, k, v, _ = synth.gen_planted_qk(shape, seed)
    hw = shape.heads_kv if per_kv else shape.heads_q
    wq, wk = synth.gen_gate_weights(shape.heads_q, shape.head_dim, dg, seed + 1, heads_w_k=hw)
    return q, k, wq, wk


def _check_threshold_mask(got_mask, scores_ref, T, what):
    want = oracle.threshold_mask(scores_ref, T)
    band = np.abs(scores_ref - T) <= MASK_BAND
    diff = (got_mask != want) & ~band
    say(f"  {what}: {int(want.sum())} active blocks, {int(band.sum())} in the band, {int(diff.sum())} mismatches")
    assert not diff.any(), f"{what}: mask differs from the oracle outside the {MASK_BAND} band"


GATE_CASES = [
    ("s2500_d128_dg128", Shape(1, 4, 2, 64 * 40 - 60, 128), 128, False),
    ("s4096_d64_dg64_kvw", Shape(2, 4, 1, 4096, 64), 64, True),
    ("s640_d128_dg48", Shape(1, 2, 2, 640, 128), 48, False),
]


@pytest.mark.parametrize("name,shape,dg,per_kv", GATE_CASES, ids=[c[0] for c in GATE_CASES])
def test_gate_threshold_matches_oracle(name, shape, dg, per_kv):
    seer = _seer()
    say(f"[gate threshold {name}] shape={shape} dg={dg} per_kv={per_kv}")
    q, k, wq, wk = _gate_inputs(shape, 60, dg, per_kv)
    sc_ref = oracle.gate_scores(q, k, wq, wk, wk_per_kv_head=per_kv)
    nb = shape.nb
    for T in (5e-4, 0.6 / nb, 1.2 / nb, 0.05):
        mask, scores = seer.seer_gate_fwd(dev_bf16(q), dev_bf16(k), dev_f32(wq), dev_f32(wk), mode="threshold",
                                          threshold=T, wk_per_kv_head=per_kv)
        torch.cuda.synchronize()
        s = host(scores)
        err = np.abs(s - sc_ref)
        say(f"  T={T:.3e} scores max-abs {err.max():.3e}, max rel {(err / np.maximum(sc_ref, 1e-30)).max():.3e}")
        assert err.max() < 1e-5
        _check_threshold_mask(mask.cpu().numpy(), sc_ref, T, f"T={T:.3e}")


@pytest.mark.parametrize("topk", [1, 5, [2, 7, 3, 40]], ids=["k1", "k5", "per_head"])
def test_gate_topk_matches_oracle(topk):
    seer = _seer()
    shape = Shape(1, 4, 2, 64 * 37, 128)
    q, k, wq, wk = _gate_inputs(shape, 61, 128)
    sc_ref = oracle.gate_scores(q, k, wq, wk)
    mask, scores = seer.seer_gate_fwd(dev_bf16(q), dev_bf16(k), dev_f32(wq), dev_f32(wk), mode="topk", topk=topk)
    torch.cuda.synchronize()
    _check_topk_mask(mask.cpu().numpy(), sc_ref, topk)


def _check_topk_mask(got, sc_ref, topk):
    """Every row keeps exactly min(k, i+1) causal blocks, and agrees with the
    oracle's top-k except for scores within the band of the row's k-th one."""
    B, H, nb, _ = sc_ref.shape
    ks = np.broadcast_to(np.asarray(topk), (H,))
    want = oracle.topk_mask(sc_ref, topk)
    bad = 0
    for b in range(B):
        for h in range(H):
            for i in range(nb):
                kk = min(int(ks[h]), i + 1)
                assert int(got[b, h, i].sum()) == kk, f"row {b},{h},{i}"
                assert not got[b, h, i, i + 1:].any()
                row = sc_ref[b, h, i, :i + 1]
                kth = np.partition(row, i + 1 - kk)[i + 1 - kk]
                outside = np.abs(row - kth) > MASK_BAND
                bad += int(((got[b, h, i, :i + 1] != want[b, h, i, :i + 1]) & outside).sum())
    say(f"  top-k {topk}: {bad} mismatches outside the band")
    assert bad == 0


# Rows longer than one wavefront's 256-element pass, aligned and not, up to the
# register-resident limit (4096 blocks) and one past it (a workgroup per row).
LONG_GATE_CASES = [
    ("nb300", 300, [7, 150]),
    ("nb701", 701, [33, 700]),
    ("nb1500", 1500, [106, 1]),
    ("nb2100", 2100, [210, 5]),
    ("nb4100", 4100, [410, 64]),
]


@pytest.mark.parametrize("name,nb,topk", LONG_GATE_CASES, ids=[c[0] for c in LONG_GATE_CASES])
def test_gate_long_rows_match_oracle(name, nb, topk):
    seer = _seer()
    shape = Shape(1, 2, 1, 64 * nb - 5, 64)
    say(f"[gate long rows {name}] shape={shape} topk={topk}")
    q, k, wq, wk = _gate_inputs(shape, 66, 64)
    sc_ref = oracle.gate_scores(q, k, wq, wk)
    mask, scores = seer.seer_gate_fwd(dev_bf16(q), dev_bf16(k), dev_f32(wq), dev_f32(wk), mode="topk", topk=topk)
    torch.cuda.synchronize()
    err = np.abs(host(scores) - sc_ref)
    say(f"  scores max-abs {err.max():.3e}")
    assert err.max() < 1e-5
    _check_topk_mask(mask.cpu().numpy(), sc_ref, topk)
    T = 1.5 / nb
    mask_t, _ = seer.seer_gate_fwd(dev_bf16(q), dev_bf16(k), dev_f32(wq), dev_f32(wk), mode="threshold", threshold=T)
    torch.cuda.synchronize()
    _check_threshold_mask(mask_t.cpu().numpy(), sc_ref, T, f"T={T:.3e}")


@pytest.mark.parametrize("mode", ["topk", "threshold"])
@pytest.mark.parametrize("nb", [300, 2100, 4100], ids=["nb300", "nb2100", "nb4100"])
def test_gate_mask_only_equals_mask_with_scores(nb, mode):
    """Without a scores output the probabilities are not written back; the
    mask must be the same bits (a wavefront per row up to 4096 blocks, a
    workgroup per row past that)."""
    seer = _seer()
    shape = Shape(1, 2, 1, 64 * nb - 5, 64)
    say(f"[gate mask only {mode}] shape={shape}")
    q, k, wq, wk = (dev_bf16(x) if i < 2 else dev_f32(x) for i, x in enumerate(_gate_inputs(shape, 71, 64)))
    kw = dict(mode="topk", topk=[nb // 10, 3]) if mode == "topk" else dict(mode="threshold", threshold=1.5 / nb)
    m0, s0 = seer.seer_gate_fwd(q, k, wq, wk, **kw)
    m1, s1 = seer.seer_gate_fwd(q, k, wq, wk, want_scores=False, **kw)
    torch.cuda.synchronize()
    assert s1 is None and s0 is not None
    say(f"  {int(m0.sum())} active blocks")
    assert torch.equal(m0, m1)


@pytest.mark.parametrize("nb", [517, 1101], ids=["nb517", "nb1101"])
def test_gate_flat_long_rows_keep_lowest_indices(nb):
    """W_q = 0: every causal score of row i is 1/(i+1), so top-k keeps blocks
    0 .. k-1 (ties to the lower index, across the row's 256-element passes)."""
    seer = _seer()
    shape = Shape(1, 1, 1, 64 * nb, 64)
    q, k, _ = synth.gen_qkv(shape, 67, want_v=False)
    wq = np.zeros((1, 64, 64), np.float32)
    wk = synth.gen_gate_weights(1, 64, 64, 68)[1]
    kk = 300
    mask, scores = seer.seer_gate_fwd(dev_bf16(q), dev_bf16(k), dev_f32(wq), dev_f32(wk), mode="topk", topk=kk)
    torch.cuda.synchronize()
    m = mask.cpu().numpy()[0, 0]
    s = host(scores)[0, 0]
    for i in (0, 255, 256, 299, 300, 511, nb - 1):
        assert np.all(s[i, :i + 1] == np.float32(1.0) / np.float32(i + 1)) and not s[i, i + 1:].any()
        want = np.zeros(nb, np.uint8)
        want[:min(kk, i + 1)] = 1
        assert np.array_equal(m[i], want), f"row {i}"
    assert np.array_equal(m.sum(1), np.minimum(kk, np.arange(1, nb + 1)))


def test_gate_flat_scores_ties_and_strictness():
    """W_q = 0 gives score 1/(i+1) exactly; T = 0.25 drops row 3 (strict >), top-k keeps the lowest j."""
    seer = _seer()
    shape = Shape(1, 2, 1, 64 * 12, 128)
    q, k, _ = synth.gen_qkv(shape, 62, want_v=False)
    wq = np.zeros((2, 128, 128), np.float32)
    wk = synth.gen_gate_weights(2, 128, 128, 63)[1]
    mask, scores = seer.seer_gate_fwd(dev_bf16(q), dev_bf16(k), dev_f32(wq), dev_f32(wk), threshold=0.25)
    torch.cuda.synchronize()
    s = host(scores)
    assert np.all(s[0, :, 3, :4] == 0.25)
    m = mask.cpu().numpy()
    assert m[0, :, :3].sum() == 2 * 6 and m[0, :, 3:].sum() == 0
    mask2, _ = seer.seer_gate_fwd(dev_bf16(q), dev_bf16(k), dev_f32(wq), dev_f32(wk), mode="topk", topk=3)
    torch.cuda.synchronize()
    m2 = mask2.cpu().numpy()
    for i in range(12):
        want = np.zeros(12, np.uint8)
        want[:min(3, i + 1)] = 1
        assert np.array_equal(m2[0, 0, i], want)


def _offset_view(shape, dtype, elems):
    """A contiguous tensor whose data starts `elems` elements into its buffer."""
    n = int(np.prod(shape))
    return torch.zeros(n + elems, dtype=dtype, device="cuda")[elems:].view(shape)


@pytest.mark.parametrize("mode", ["topk", "threshold"])
def test_gate_misaligned_maps_equal_aligned(mode):
    """Scores 4 bytes and mask 1 byte past 16-byte alignment (allowed by the
    ABI; varlen maps start at such offsets) give the same bits as aligned
    maps, at a row length that is a multiple of 4 (the 16-byte path)."""
    seer = _seer()
    shape = Shape(1, 2, 1, 64 * 300, 64)
    q, k, wq, wk = (dev_bf16(x) if i < 2 else dev_f32(x) for i, x in enumerate(_gate_inputs(shape, 69, 64)))
    nb = shape.nb
    kw = dict(mode="topk", topk=[17, 90]) if mode == "topk" else dict(mode="threshold", threshold=1.5 / nb)
    m0, s0 = seer.seer_gate_fwd(q, k, wq, wk, **kw)
    sc1 = _offset_view((1, 2, nb, nb), torch.float32, 1)
    mk1 = _offset_view((1, 2, nb, nb), torch.uint8, 1)
    assert sc1.data_ptr() % 16 == 4 and mk1.data_ptr() % 4 == 1
    m1, s1 = seer.seer_gate_fwd(q, k, wq, wk, scores=sc1, block_mask=mk1, **kw)
    torch.cuda.synchronize()
    assert torch.equal(s0, s1) and torch.equal(m0, m1)


def test_distill_misaligned_gt_equals_aligned():
    """A ground-truth map 4 bytes past 16-byte alignment gives the same loss
    and gradients as an aligned one (rows a multiple of 4 blocks long)."""
    seer = _seer()
    shape = Shape(1, 2, 1, 64 * 300, 64)
    q, k, wq, wk = (dev_bf16(x) if i < 2 else dev_f32(x) for i, x in enumerate(_gate_inputs(shape, 70, 64)))
    nb = shape.nb
    gt_np = np.tril(np.random.default_rng(71).random((1, 2, nb, nb))).astype(np.float32)
    gt0 = dev_f32(gt_np)
    gt1 = _offset_view((1, 2, nb, nb), torch.float32, 1)
    gt1.copy_(gt0)
    assert gt1.data_ptr() % 16 == 4
    a = seer.seer_gate_distill_bwd(q, k, wq, wk, gt0, rope_theta=5e5)
    b = seer.seer_gate_distill_bwd(q, k, wq, wk, gt1, rope_theta=5e5)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_gate_to_sparse_attention_end_to_end():
    """Gate mask -> block-sparse attention, checked against the oracle's own gate + attention."""
    seer = _seer()
    shape = Shape(1, 4, 2, 64 * 24, 128)
    q, k, wq, wk = _gate_inputs(shape, 64, 128)
    _, _, v = synth.gen_qkv(shape, 65)
    T = 1.0 / shape.nb
    mask, _ = seer.seer_gate_fwd(dev_bf16(q), dev_bf16(k), dev_f32(wq), dev_f32(wk), threshold=T)
    out, _ = seer.seer_block_sparse_attn_fwd(dev_bf16(q), dev_bf16(k), dev_bf16(v), mask, out_dtype=torch.float32)
    torch.cuda.synchronize()
    sc_ref = oracle.gate_scores(q, k, wq, wk)
    m_gpu = mask.cpu().numpy()
    _check_threshold_mask(m_gpu, sc_ref, T, "e2e mask")
    o_ref, _ = oracle.attention(q, k, v, m_gpu)
    check_close(host(out), o_ref, "e2e O")
