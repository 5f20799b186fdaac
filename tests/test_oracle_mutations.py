"""Planted mistakes in copies of the oracle must each fail at least one pin.

Each mutation is a textual edit of oracle/seer_oracle.py (a dropped term, a
wrong sign or index, a transposed operand, an off-by-one); the edited source
is executed as a throwaway module on the CPU and the pins of
tests/oracle_pins.py are run against it. The real oracle is never modified.
This shows the pins are strong enough to catch plausible slips in every
function of the oracle.
"""
import os
import types

import pytest

from oracle_pins import ALL_PINS

SRC_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "oracle", "seer_oracle.py")

# (name, old text, new text, which occurrence of old text to replace)
MUTATIONS = [
    ("as_f64_bits_shift", "(a.astype(np.uint32) << 16)", "(a.astype(np.uint32) << 15)", 0),
    ("as_f64_bits_not_reinterpreted", "<< 16).view(np.float32)", "<< 16).astype(np.float32)", 0),
    ("as_f64_bits_read_as_integers", "if a.dtype == np.uint16:", "if a.dtype == np.int8:", 0),
    ("pool_k_max_to_min", "out[..., i, 0:D] = blk.max(axis=-2)", "out[..., i, 0:D] = blk.min(axis=-2)", 0),
    ("pool_k_order_swapped",
     "out[..., i, D:2 * D] = blk.min(axis=-2)\n        out[..., i, 2 * D:3 * D] = blk.mean(axis=-2)",
     "out[..., i, D:2 * D] = blk.mean(axis=-2)\n        out[..., i, 2 * D:3 * D] = blk.min(axis=-2)", 0),
    ("pool_q_sum_not_mean", "out[..., i, :] = q[..., a:b, :].mean(axis=-2)",
     "out[..., i, :] = q[..., a:b, :].sum(axis=-2)", 0),
    ("pool_ragged_block_dropped", "return i * block, min((i + 1) * block, seq_len)",
     "return i * block, (i + 1) * block - (1 if (i + 1) * block > seq_len else 0)", 0),
    ("gate_scale_dropped", "scale = 1.0 / np.sqrt(D)", "scale = 1.0", 0),
    ("gate_not_causal", "z = np.where(causal, z, -np.inf)", "z = z", 0),
    ("gate_gqa_head_map", "g = h // G\n            if g not in", "g = h % Hkv\n            if g not in", 0),
    ("gate_wk_index_swapped", "kg = kp @ (w_k[g] if wk_per_kv_head else w_k[h])",
     "kg = kp @ (w_k[h] if wk_per_kv_head else w_k[g])", 0),
    ("gate_transposed_scores", "z = (qg @ kg.T) * scale", "z = (kg @ qg.T) * scale", 0),
    ("gate_softmax_over_columns", "e / e.sum(axis=1, keepdims=True)", "e / e.sum(axis=0, keepdims=True)", 0),
    ("threshold_not_strict", "((s > threshold) & causal)", "((s >= threshold) & causal)", 0),
    ("threshold_not_causal", "((s > threshold) & causal)", "((s > threshold) | ~causal)", 0),
    ("topk_off_by_one", "order[:min(kk, i + 1)]", "order[:min(kk, i)]", 0),
    ("topk_ascending", "np.argsort(-row, kind=\"stable\")", "np.argsort(row, kind=\"stable\")", 0),
    ("topk_ties_high_index", "np.argsort(-row, kind=\"stable\")",
     "(len(row) - 1 - np.argsort(-row[::-1], kind=\"stable\"))", 0),
    ("attn_causal_strict", "s = np.where(keys[None, :] <= tq, s, -np.inf)",
     "s = np.where(keys[None, :] < tq, s, -np.inf)", 0),
    ("attn_scale_dropped", "scale = 1.0 / np.sqrt(D)", "scale = 1.0", 1),
    ("attn_v_is_k", "vv = as_f64(v[b, g, keys])", "vv = as_f64(k[b, g, keys])", 0),
    ("attn_mask_transposed", "row = np.asarray(block_mask[b, h, i])", "row = np.asarray(block_mask[b, h, :, i])", 0),
    ("attn_gqa_head_map", "g = h // G\n        t0, t1", "g = h % Hkv\n        t0, t1", 0),
    ("attn_empty_row_lse_zero", "lse = np.full((t1 - t0,), -np.inf", "lse = np.full((t1 - t0,), 0.0", 0),
    ("attn_lse_missing_max", "lse = np.where(has, mx[:, 0] + np.log(", "lse = np.where(has, 0.0 + np.log(", 0),
    ("gt_mean_not_max", "row[j] = p[:, a:bb].max()", "row[j] = p[:, a:bb].mean()", 0),
    ("gt_not_causal", "s = np.where(np.arange(t1)[None, :] <= tq, s, -np.inf)", "s = s", 0),
    ("gt_scale_dropped", "scale = 1.0 / np.sqrt(D)", "scale = 1.0", 2),
    ("gt_gqa_head_map", "g = h // G\n        t0, t1", "g = h % Hkv\n        t0, t1", 1),
    ("gt_upper_not_zero", "for j in range(i + 1):\n            a, bb", "for j in range(nb):\n            a, bb", 0),
    ("rope_sign_flipped", "x2 * c + x1 * s", "x2 * c - x1 * s", 0),
    ("rope_interleaved_pairs", "x1, x2 = x[..., :half], x[..., half:]", "x1, x2 = x[..., 0::2], x[..., 1::2]", 0),
    ("rope_base_not_divided", "inv_freq = (theta / block) **", "inv_freq = theta **", 0),
    ("rope_frequency_exponent", "** (-2.0 * np.arange(half, dtype=np.float64) / dg)",
     "** (-1.0 * np.arange(half, dtype=np.float64) / dg)", 0),
    ("gate_rope_key_not_rotated", "                kg = block_rope(kg, rope_theta, block)\n            z = (qg",
     "                kg = kg\n            z = (qg", 0),
    ("distill_gt_not_normalized", "p = np.where(valid, target / np.where(valid, tsum, 1.0), 0.0)",
     "p = np.where(valid, target, 0.0)", 0),
    ("distill_gradient_sign", "dz = np.where(causal & valid, score - p, 0.0) / n_rows",
     "dz = np.where(causal & valid, p - score, 0.0) / n_rows", 0),
    ("distill_empty_row_gradient", "dz = np.where(causal & valid, score - p, 0.0) / n_rows",
     "dz = np.where(causal, score - p, 0.0) / n_rows", 0),
    ("distill_grad_scale_dropped", "dqg = (dz @ kg) * scale", "dqg = (dz @ kg)", 0),
    ("distill_key_grad_untransposed", "dkg = (dz.T @ qg) * scale", "dkg = (dz @ qg) * scale", 0),
    ("distill_no_back_rotation", "dqg = block_rope(dqg, rope_theta, block, positions=neg_pos)",
     "dqg = block_rope(dqg, rope_theta, block)", 0),
    ("distill_sum_not_mean", "return loss / n_rows, grad_wq, grad_wk", "return loss, grad_wq, grad_wk", 0),
    ("decode_kcomp_wrong_group", "g = w if wk_per_kv_head else w // G", "g = w if wk_per_kv_head else w % Hkv", 0),
    ("decode_gate_scale_dropped", "@ q[b, h] / np.sqrt(D)\n            e = np.exp(z - z.max())",
     "@ q[b, h]\n            e = np.exp(z - z.max())", 0),
    ("decode_threshold_not_strict", "return (np.asarray(scores, dtype=np.float64) > threshold)",
     "return (np.asarray(scores, dtype=np.float64) >= threshold)", 0),
    ("decode_topk_ascending", "order = np.argsort(-s[b, h], kind=\"stable\")",
     "order = np.argsort(s[b, h], kind=\"stable\")", 0),
    ("decode_attn_mask_ignored", "blocks = range(nb) if block_mask is None else",
     "blocks = range(nb) if True else", 0),
    ("decode_attn_lse_no_max", "lse[b, h] = mx + np.log(e.sum())", "lse[b, h] = np.log(e.sum())", 0),
    ("decode_gt_unnormalized", "p /= p.sum()\n", "p /= 1.0\n", 0),
    ("decode_gt_mean_not_max", "out[b, h, j] = p[a:e].max()", "out[b, h, j] = p[a:e].mean()", 0),
    ("distill_kl_reversed", "loss += float(np.sum(p[pos] * (np.log(p[pos]) - log_score[pos])))",
     "loss += float(np.sum(score[pos] * (log_score[pos] - np.log(p[pos]))))", 0),
]


def _mutant(old, new, occurrence):
    with open(SRC_PATH) as f:
        src = f.read()
    pos = -1
    for _ in range(occurrence + 1):
        pos = src.find(old, pos + 1)
        assert pos >= 0, f"mutation anchor not found: {old!r} (occurrence {occurrence})"
    src = src[:pos] + new + src[pos + len(old):]
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src, "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new,occ", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(name, old, new, occ):
    mod = _mutant(old, new, occ)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(mod)
        except Exception:                      # assertion or crash both count as caught
            caught.append(pin.__name__)
            break
    assert caught, f"no pin caught mutation {name}"
