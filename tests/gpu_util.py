"""Helpers for the GPU tests: seeded inputs to device tensors, tolerances."""
from __future__ import annotations

import sys

import numpy as np
import torch

# bf16 inputs, fp32 accumulation: the bound the method's comparison uses
O_MAX_ABS = 1e-2
O_MEAN_ABS = 1e-3
MASK_BAND = 1e-6     # scores this close to the decision boundary may flip


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev_u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def bf16_half_ulp(x: np.ndarray) -> np.ndarray:
    """Half the spacing of bfloat16 values at |x| (8 significant bits): the
    most that rounding an exact result to a bf16 output can move it."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return np.ldexp(1.0, (e - 8).astype(np.int64))


def check_close(got: np.ndarray, want: np.ndarray, what: str, max_abs=O_MAX_ABS, mean_abs=O_MEAN_ABS,
                out_dtype=None):
    """Element-wise comparison with the bound for bf16 inputs and fp32
    accumulation. A bf16 output is the fp32 result rounded once more, so each
    of its elements is also allowed half a bf16 ulp of the reference value."""
    assert got.shape == want.shape, (what, got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    err = np.abs(got - want)
    mx, mean = float(err.max()) if err.size else 0.0, float(err.mean()) if err.size else 0.0
    if out_dtype == torch.bfloat16 and err.size:
        beyond = float((err - bf16_half_ulp(np.maximum(np.abs(want), np.abs(got)))).max())
        say(f"  {what}: max-abs {mx:.3e} mean-abs {mean:.3e} over {err.size} values (bf16 output; "
            f"max-abs beyond its rounding {beyond:.3e})")
        assert beyond <= max_abs, f"{what}: max-abs beyond the bf16 output rounding {beyond} > {max_abs}"
    else:
        say(f"  {what}: max-abs {mx:.3e} mean-abs {mean:.3e} over {err.size} values")
        assert mx <= max_abs, f"{what}: max-abs {mx} > {max_abs}"
    assert mean <= mean_abs, f"{what}: mean-abs {mean} > {mean_abs}"


def check_lse(got: np.ndarray, want: np.ndarray, what: str, tol=2e-3):
    fin = np.isfinite(want)
    assert np.array_equal(np.isfinite(got), fin), f"{what}: -inf pattern differs"
    assert np.all(got[~fin] == -np.inf)
    if fin.any():
        err = np.abs(got[fin] - want[fin])
        say(f"  {what}: max-abs {err.max():.3e}")
        assert err.max() <= tol


def sample_rows(B, H, nb, n_per_head, seed, extra=()):
    """Seeded sample of query blocks per head, always including 0, 1, nb/2, nb-1."""
    rng = np.random.Generator(np.random.PCG64(seed))
    rows = []
    for b in range(B):
        for h in range(H):
            base = {0, min(1, nb - 1), nb // 2, nb - 1} | set(extra)
            pick = set(int(x) for x in rng.choice(nb, size=min(n_per_head, nb), replace=False))
            for i in sorted(base | pick):
                rows.append((b, h, i))
    return rows
