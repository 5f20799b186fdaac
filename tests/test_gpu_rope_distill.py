"""GPU parity of the gate's block-level RoPE and of the self-distillation step
(KL loss and W_q / W_k gradients) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth import Shape
from gpu_util import MASK_BAND, dev_bf16, dev_f32, host, say

pytestmark = pytest.mark.gpu


def _seer():
    import learned_block_sparse_attngate_amd as seer
    seer.load_library()
    return seer


def _gate_inputs(shape, seed, dg, per_kv=False, var=None):
    q, k, _, _ = synth.gen_planted_qk(shape, seed)
    hw = shape.heads_kv if per_kv else shape.heads_q
    wq, wk = synth.gen_gate_weights(shape.heads_q, shape.head_dim, dg, seed + 1, heads_w_k=hw, var=var)
    return q, k, wq, wk


ROPE_CASES = [
    # name, shape, gate dim, W_k per KV head, RoPE base
    ("s2500_d128_theta5e5", Shape(1, 4, 2, 64 * 40 - 60, 128), 128, False, 5e5),
    ("s4096_d64_kvw_theta1e4", Shape(2, 4, 1, 4096, 64), 64, True, 1e4),
    ("s131072_d128_theta5e5", Shape(1, 2, 1, 131072, 128), 128, False, 5e5),   # 2048 block positions
]


@pytest.mark.parametrize("name,shape,dg,per_kv,theta", ROPE_CASES, ids=[c[0] for c in ROPE_CASES])
def test_gate_rope_matches_oracle(name, shape, dg, per_kv, theta):
    seer = _seer()
    say(f"[gate rope {name}] shape={shape} dg={dg} per_kv={per_kv} theta={theta}")
    q, k, wq, wk = _gate_inputs(shape, 70, dg, per_kv, var=4.0 / dg)
    sc_ref = oracle.gate_scores(q, k, wq, wk, wk_per_kv_head=per_kv, rope_theta=theta)
    sc_plain = oracle.gate_scores(q, k, wq, wk, wk_per_kv_head=per_kv)
    assert np.abs(sc_ref - sc_plain).max() > 1e-4          # the rotation matters for these inputs
    nb = shape.nb
    for T in (0.6 / nb, 1.5 / nb):
        mask, scores = seer.seer_gate_fwd(dev_bf16(q), dev_bf16(k), dev_f32(wq), dev_f32(wk), mode="threshold",
                                          threshold=T, wk_per_kv_head=per_kv, rope_theta=theta)
        torch.cuda.synchronize()
        s = host(scores)
        err = np.abs(s - sc_ref)
        say(f"  T={T:.3e} scores max-abs {err.max():.3e}")
        assert err.max() < 1e-5
        want = oracle.threshold_mask(sc_ref, T)
        band = np.abs(sc_ref - T) <= MASK_BAND
        diff = (mask.cpu().numpy() != want) & ~band
        say(f"  {int(want.sum())} active blocks, {int(band.sum())} in the band, {int(diff.sum())} mismatches")
        assert not diff.any()


def test_gate_rope_topk_matches_oracle():
    seer = _seer()
    shape = Shape(1, 4, 2, 64 * 37, 128)
    q, k, wq, wk = _gate_inputs(shape, 71, 128, var=4.0 / 128)
    sc_ref = oracle.gate_scores(q, k, wq, wk, rope_theta=5e5)
    mask, _ = seer.seer_gate_fwd(dev_bf16(q), dev_bf16(k), dev_f32(wq), dev_f32(wk), mode="topk", topk=5,
                                 rope_theta=5e5)
    torch.cuda.synchronize()
    got = mask.cpu().numpy()
    want = oracle.topk_mask(sc_ref, 5)
    bad = 0
    for h in range(4):
        for i in range(shape.nb):
            kk = min(5, i + 1)
            assert int(got[0, h, i].sum()) == kk
            row = sc_ref[0, h, i, :i + 1]
            kth = np.sort(row)[::-1][kk - 1]
            outside = np.abs(row - kth) > MASK_BAND
            bad += int(((got[0, h, i, :i + 1] != want[0, h, i, :i + 1]) & outside).sum())
    say(f"  rope top-5: {bad} mismatches outside the band")
    assert bad == 0


def _check_distill(got, want, what):
    loss, gq, gk = (host(t) for t in got)
    l_ref, gq_ref, gk_ref = want
    say(f"  {what}: loss {float(loss[0]):.8f} vs {l_ref:.8f}")
    assert abs(float(loss[0]) - l_ref) <= 1e-4 * abs(l_ref) + 1e-7
    for g, r, nm in ((gq, gq_ref, "grad_wq"), (gk, gk_ref, "grad_wk")):
        err = np.abs(g - r).max()
        scale = np.abs(r).max()
        say(f"  {what} {nm}: max-abs {err:.3e} (max |grad| {scale:.3e})")
        assert np.all(np.isfinite(g))
        assert err <= 2e-4 * scale + 1e-12


DISTILL_CASES = [
    # name, shape, gate dim, W_k per KV head, RoPE base
    ("s1267_d128_rope", Shape(1, 4, 2, 64 * 20 - 13, 128), 128, False, 5e5),
    ("s576_d64_b2_kvw", Shape(2, 4, 1, 64 * 9, 64), 64, True, 0.0),
    ("s2560_d128_dg48_rope_kvw", Shape(1, 4, 2, 64 * 40, 128), 48, True, 1e4),
]


@pytest.mark.parametrize("name,shape,dg,per_kv,theta", DISTILL_CASES, ids=[c[0] for c in DISTILL_CASES])
def test_distill_matches_oracle(name, shape, dg, per_kv, theta):
    """Loss and gradients for a ground-truth map from the oracle, given as fp32
    to both sides; one ground-truth row is zeroed (it must add nothing)."""
    seer = _seer()
    say(f"[distill {name}] shape={shape} dg={dg} per_kv={per_kv} theta={theta}")
    q, k, wq, wk = _gate_inputs(shape, 72, dg, per_kv, var=4.0 / dg)
    gt = oracle.maxpool_gt(q, k).astype(np.float32)
    gt[0, 1, shape.nb // 2, :] = 0.0
    want = oracle.gate_distill(q, k, wq, wk, gt, wk_per_kv_head=per_kv, rope_theta=theta or None)
    got = seer.seer_gate_distill_bwd(dev_bf16(q), dev_bf16(k), dev_f32(wq), dev_f32(wk), dev_f32(gt),
                                     wk_per_kv_head=per_kv, rope_theta=theta)
    torch.cuda.synchronize()
    _check_distill(got, want, name)


# Rows longer than one wavefront's 256-element pass (aligned and not) and past
# the register-resident limit of 4096 blocks (a workgroup per row), with a
# seeded lower-triangular target map in place of the (costly) oracle ground
# truth, one row of it zeroed.
LONG_DISTILL_CASES = [
    ("nb600", 600, 5e5),
    ("nb1501", 1501, 0.0),
    ("nb4100", 4100, 5e5),
]


@pytest.mark.parametrize("name,nb,theta", LONG_DISTILL_CASES, ids=[c[0] for c in LONG_DISTILL_CASES])
def test_distill_long_rows_match_oracle(name, nb, theta):
    seer = _seer()
    shape = Shape(1, 2, 1, 64 * nb - 7, 64)
    say(f"[distill long rows {name}] shape={shape} theta={theta}")
    q, k, wq, wk = _gate_inputs(shape, 76, 64, var=4.0 / 64)
    gt = np.tril(np.random.default_rng(77).random((1, 2, nb, nb))).astype(np.float32)
    gt[0, 0, nb // 3, :] = 0.0
    want = oracle.gate_distill(q, k, wq, wk, gt, rope_theta=theta or None)
    got = seer.seer_gate_distill_bwd(dev_bf16(q), dev_bf16(k), dev_f32(wq), dev_f32(wk), dev_f32(gt),
                                     rope_theta=theta)
    torch.cuda.synchronize()
    _check_distill(got, want, name)


def test_distill_end_to_end_and_descent():
    """GPU ground truth -> GPU distillation step against the oracle's ground
    truth -> oracle step; then one gradient step lowers the GPU loss."""
    seer = _seer()
    shape = Shape(1, 4, 2, 64 * 24, 128)
    q, k, wq, wk = _gate_inputs(shape, 73, 128, var=4.0 / 128)
    _, _, v = synth.gen_qkv(shape, 74)
    dq, dk, dv = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    _, _, gt = seer.seer_attn_maxpool_gt(dq, dk, dv, out_dtype=torch.float32)
    d_wq, d_wk = dev_f32(wq), dev_f32(wk)
    got = seer.seer_gate_distill_bwd(dq, dk, d_wq, d_wk, gt, rope_theta=5e5)
    torch.cuda.synchronize()
    want = oracle.gate_distill(q, k, wq, wk, oracle.maxpool_gt(q, k), rope_theta=5e5)
    _check_distill(got, want, "gpu gt -> distill")
    loss0 = float(got[0].item())
    lr = 0.05 / max(float(got[1].abs().max()), float(got[2].abs().max()))
    loss1 = float(seer.seer_gate_distill_bwd(dq, dk, d_wq - lr * got[1], d_wk - lr * got[2], gt,
                                             rope_theta=5e5)[0].item())
    say(f"  loss {loss0:.6f} -> {loss1:.6f} after one step")
    assert loss1 < loss0


def test_distill_deterministic():
    seer = _seer()
    shape = Shape(1, 8, 2, 64 * 64, 128)
    q, k, wq, wk = _gate_inputs(shape, 75, 128)
    gt = np.tril(np.random.default_rng(5).random((1, 8, 64, 64))).astype(np.float32)
    args = (dev_bf16(q), dev_bf16(k), dev_f32(wq), dev_f32(wk), dev_f32(gt))
    a = seer.seer_gate_distill_bwd(*args, rope_theta=5e5)
    b = seer.seer_gate_distill_bwd(*args, rope_theta=5e5)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
