"""GPU parity of the decode stage (compressed K cache, decode gate and masks,
block-sparse decode attention, 1D max-pooled map) against the fp64 oracle."""
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


def _inputs(shape, seed, per_kv=False, var=None):
    q, k, v = synth.gen_qkv(shape, seed)
    qd = np.ascontiguousarray(q[:, :, -1])           # the newest token's query
    hw = shape.heads_kv if per_kv else shape.heads_q
    _, wk = synth.gen_gate_weights(shape.heads_q, shape.head_dim, shape.head_dim, seed + 1, heads_w_k=hw, var=var)
    return qd, k, v, wk


@pytest.mark.parametrize("shape,per_kv", [(Shape(1, 4, 2, 64 * 30 - 17, 128), False),
                                          (Shape(2, 8, 2, 64 * 9 + 1, 64), True)],
                         ids=["d128_ragged", "d64_b2_kvw"])
def test_compress_k_full_and_incremental(shape, per_kv):
    seer = _seer()
    say(f"[decode kcomp] shape={shape} per_kv={per_kv}")
    _, k, _, wk = _inputs(shape, 90, per_kv)
    want = oracle.decode_kcomp(k, wk, shape.heads_q, wk_per_kv_head=per_kv)
    dk, dwk = dev_bf16(k), dev_f32(wk)
    cap = shape.nb + 5
    kc = seer.seer_decode_compress_k(dk, dwk, shape.heads_q, wk_per_kv_head=per_kv, capacity_blocks=cap)
    torch.cuda.synchronize()
    got = host(kc)[:, :, :shape.nb]
    err = np.abs(got - want).max()
    say(f"  full: max-abs {err:.3e} (max |K'| {np.abs(want).max():.3e})")
    assert err <= 1e-5 * max(1.0, np.abs(want).max())
    # a shorter cache first, then the tokens appended: recompute from the first changed block
    s1 = shape.seq_len - 70
    kc2 = seer.seer_decode_compress_k(dk[:, :, :s1].contiguous(), dwk, shape.heads_q, wk_per_kv_head=per_kv,
                                      capacity_blocks=cap)
    kc2 = seer.seer_decode_compress_k(dk, dwk, shape.heads_q, wk_per_kv_head=per_kv, kcomp=kc2,
                                      block_begin=(s1 - 1) // 64)
    torch.cuda.synchronize()
    assert torch.equal(kc2[:, :, :shape.nb], kc[:, :, :shape.nb])


@pytest.mark.parametrize("per_kv,shape", [(False, Shape(2, 8, 2, 64 * 300 - 33, 128)),
                                           (True, Shape(2, 8, 2, 64 * 300 - 33, 128)),
                                           (False, Shape(1, 4, 1, 64 * 2101 - 5, 64)),
                                           (True, Shape(1, 4, 2, 64 * 4100, 64)),
                                           (False, Shape(1, 4, 1, 64 * 9000 + 7, 64))],
                         ids=["wk_per_q", "wk_per_kv", "nb2101", "nb4100_kvw", "nb9001"])
def test_decode_gate_matches_oracle(per_kv, shape):
    seer = _seer()
    say(f"[decode gate] shape={shape} per_kv={per_kv}")
    qd, k, _, wk = _inputs(shape, 91, per_kv, var=4.0 / 128)
    kc_ref = oracle.decode_kcomp(k, wk, shape.heads_q, wk_per_kv_head=per_kv)
    sc_ref = oracle.decode_gate_scores(qd, kc_ref, wk_per_kv_head=per_kv)
    kc = seer.seer_decode_compress_k(dev_bf16(k), dev_f32(wk), shape.heads_q, wk_per_kv_head=per_kv)
    nb = shape.nb
    for mode, arg in (("threshold", 1.5 / nb), ("threshold", 0.5 / nb), ("topk", 20),
                      ("topk", [3, 40] * (shape.heads_q // 2))):
        kw = dict(threshold=arg) if mode == "threshold" else dict(topk=arg)
        mask, scores = seer.seer_decode_gate_fwd(dev_bf16(qd), kc, shape.seq_len, shape.heads_kv,
                                                 wk_per_kv_head=per_kv, mode=mode, **kw)
        torch.cuda.synchronize()
        s = host(scores)
        assert np.abs(s - sc_ref).max() < 1e-5
        got = mask.cpu().numpy()
        if mode == "threshold":
            want = oracle.decode_threshold_mask(sc_ref, arg)
            band = np.abs(sc_ref - arg) <= MASK_BAND
        else:
            want = oracle.decode_topk_mask(sc_ref, arg)
            ks = np.broadcast_to(np.asarray(arg), (shape.heads_q,))
            kth = np.stack([np.sort(sc_ref[:, h], axis=-1)[:, ::-1][:, min(int(ks[h]), nb) - 1]
                            for h in range(shape.heads_q)], axis=1)
            band = np.abs(sc_ref - kth[..., None]) <= MASK_BAND
            counts = got.sum(-1)
            assert np.array_equal(counts, np.minimum(ks, nb)[None, :].repeat(shape.batch, 0))
        bad = int(((got != want) & ~band).sum())
        say(f"  {mode} {arg if mode == 'topk' else f'{arg:.3e}'}: {int(want.sum())} active, {bad} mismatches")
        assert bad == 0



@pytest.mark.parametrize("mode", ["topk", "threshold"])
def test_decode_gate_misaligned_maps_equal_aligned(mode):
    """Scores 4 bytes and mask 1 byte past 16-byte alignment (the ABI asks
    only for 4- and 1-byte alignment) give the same bits as aligned maps, at a
    row length that is a multiple of 4 (the 16-byte path when aligned)."""
    seer = _seer()
    shape = Shape(2, 8, 2, 64 * 1200, 64)
    say(f"[decode gate misaligned] shape={shape} mode={mode}")
    qd, k, _, wk = _inputs(shape, 93, False, var=4.0 / 128)
    kc = seer.seer_decode_compress_k(dev_bf16(k), dev_f32(wk), shape.heads_q)
    nb = shape.nb
    kw = dict(mode="topk", topk=[5, 120] * (shape.heads_q // 2)) if mode == "topk" else dict(mode="threshold", threshold=1.5 / nb)
    q = dev_bf16(qd)
    m0, s0 = seer.seer_decode_gate_fwd(q, kc, shape.seq_len, shape.heads_kv, **kw)
    n = shape.batch * shape.heads_q * nb
    sc1 = torch.zeros(n + 1, dtype=torch.float32, device="cuda")[1:].view(shape.batch, shape.heads_q, nb)
    mk1 = torch.zeros(n + 1, dtype=torch.uint8, device="cuda")[1:].view(shape.batch, shape.heads_q, nb)
    assert sc1.data_ptr() % 16 == 4 and mk1.data_ptr() % 4 == 1
    m1, s1 = seer.seer_decode_gate_fwd(q, kc, shape.seq_len, shape.heads_kv, scores=sc1, block_mask=mk1, **kw)
    torch.cuda.synchronize()
    assert torch.equal(s0, s1) and torch.equal(m0, m1)
    if mode == "topk":
        assert torch.equal(m0.sum(-1).cpu(), torch.tensor([5, 120] * (shape.heads_q // 2)).repeat(shape.batch, 1))

DECODE_CASES = [
    # name, shape, mask density (None: dense), out dtype
    ("llama8b_s131072_p10", Shape(1, 32, 8, 131072, 128), 0.1, torch.bfloat16),
    ("g8_s5000_p30", Shape(1, 16, 2, 5000, 128), 0.3, torch.float32),
    ("mha_s77_d128", Shape(1, 4, 4, 77, 128), 0.6, torch.float32),
    ("b2_d64_s1000_p20", Shape(2, 8, 2, 1000, 64), 0.2, torch.float32),
    ("s1_single_token", Shape(1, 4, 2, 1, 64), 1.0, torch.float32),
]


@pytest.mark.parametrize("name,shape,dens,dt", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
def test_decode_attention_matches_oracle(name, shape, dens, dt):
    seer = _seer()
    say(f"[decode attn {name}] shape={shape} density={dens}")
    qd, k, v, _ = _inputs(shape, 92)
    nb = shape.nb
    rng = np.random.default_rng(93)
    mask = (rng.random((shape.batch, shape.heads_q, nb)) < dens).astype(np.uint8)
    if shape.heads_q > 1:
        mask[0, 1, :] = 0                             # a head with no block: O = 0, LSE = -inf
    o_ref, l_ref = oracle.decode_attention(qd, k, v, mask)
    out, lse, _ = seer.seer_decode_attn_fwd(dev_bf16(qd), dev_bf16(k), dev_bf16(v), dev_u8(mask), out_dtype=dt,
                                            want_lse=True)
    torch.cuda.synchronize()
    check_close(host(out), o_ref, f"{name} O", out_dtype=dt)
    check_lse(host(lse), l_ref, f"{name} LSE")


@pytest.mark.parametrize("shape", [Shape(1, 8, 2, 64 * 40 - 5, 128), Shape(2, 4, 1, 64 * 7 + 1, 64)],
                         ids=["d128", "d64_b2"])
def test_decode_dense_and_gt_matches_oracle(shape):
    seer = _seer()
    say(f"[decode dense+gt] shape={shape}")
    qd, k, v, _ = _inputs(shape, 94)
    o_ref, l_ref = oracle.decode_attention(qd, k, v, None)
    gt_ref = oracle.decode_gt(qd, k)
    out, lse, gt = seer.seer_decode_attn_fwd(dev_bf16(qd), dev_bf16(k), dev_bf16(v), None, out_dtype=torch.float32,
                                             want_lse=True, want_gt=True)
    ones = torch.ones((shape.batch, shape.heads_q, shape.nb), dtype=torch.uint8, device="cuda")
    out1, _, _ = seer.seer_decode_attn_fwd(dev_bf16(qd), dev_bf16(k), dev_bf16(v), ones, out_dtype=torch.float32)
    torch.cuda.synchronize()
    check_close(host(out), o_ref, "dense O")
    check_lse(host(lse), l_ref, "dense LSE")
    err = np.abs(host(gt) - gt_ref)
    big = gt_ref > 1e-6
    rel = err[big] / gt_ref[big]
    say(f"  gt max-abs {err.max():.3e}, max rel on entries > 1e-6 {rel.max():.3e}")
    assert err.max() <= 1e-6            # the runs show ~1e-8
    assert rel.max() <= 1e-4
    assert torch.equal(out, out1)                      # an all-ones mask is the dense path


def test_decode_step_end_to_end():
    """Compressed cache -> top-k gate -> sparse decode attention, against the
    oracle's gate and attention on the GPU's mask (the oracle mask agrees
    outside the tie band, checked in the gate test)."""
    seer = _seer()
    shape = Shape(1, 32, 8, 64 * 512, 128)
    qd, k, v, wk = _inputs(shape, 95, var=4.0 / 128)
    dq, dk, dv = dev_bf16(qd), dev_bf16(k), dev_bf16(v)
    kc = seer.seer_decode_compress_k(dk, dev_f32(wk), shape.heads_q)
    mask, _ = seer.seer_decode_gate_fwd(dq, kc, shape.seq_len, shape.heads_kv, mode="topk", topk=52,
                                        want_scores=False)
    out, lse, _ = seer.seer_decode_attn_fwd(dq, dk, dv, mask, out_dtype=torch.float32, want_lse=True)
    torch.cuda.synchronize()
    m = mask.cpu().numpy()
    assert np.all(m.sum(-1) == 52)
    o_ref, l_ref = oracle.decode_attention(qd, k, v, m)
    check_close(host(out), o_ref, "e2e O")
    check_lse(host(lse), l_ref, "e2e LSE")


def test_decode_deterministic():
    seer = _seer()
    shape = Shape(1, 32, 8, 64 * 256, 128)
    qd, k, v, _ = _inputs(shape, 96)
    mask = dev_u8((np.random.default_rng(1).random((1, 32, shape.nb)) < 0.2).astype(np.uint8))
    args = (dev_bf16(qd), dev_bf16(k), dev_bf16(v), mask)
    a, la, _ = seer.seer_decode_attn_fwd(*args, want_lse=True)
    b, lb, _ = seer.seer_decode_attn_fwd(*args, want_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(la, lb)
