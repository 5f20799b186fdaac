"""Benchmark of the SeerAttention hot path on one MI355X.

One step = the whole prefill hot path on one batch of synthetic input:
  seer_gate_fwd (Q/K pooling, projections, block-level RoPE with the model's
  base 500000, causal block softmax, top-k mask)
  + seer_block_sparse_attn_fwd with the workload's block mask.
The default workload is the Llama-3.1-8B-shaped layer at 128k tokens with a
seeded 90%-sparse causal block mask (diagonal + sink + 4 vertical stripes +
random fill, per-head sparsity in [0.8, 0.97] with mean 0.9). The gate runs on
the same Q/K with random-init weights in top-k mode (k chosen for ~90% causal
sparsity); random weights cannot produce a trained gate's mask, so the mask
the attention consumes is the workload's seeded one, while the gate's full
cost is in the step. The dense causal kernel runs on the same inputs for the
speedup. Inputs are resident in HBM before timing starts.

`--workload gate_gt_s32k` runs the full gate path instead: planted Q/K at 32k,
random-init gate weights, the gate's threshold mask (T = 5e-4) feeding the
block-sparse attention inside the step, and the ground-truth kernel (dense
attention + 2D-maxpooled map) timed against the dense kernel.

Prints one JSON line. `value` = executed-tile FLOP of the sparse attention
(4*64*64*D per active causal tile) / step time, in TFLOP/s.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "block-sparse prefill ms, TFLOP/s & speedup vs dense at 128k/90% sparsity"
PEAK_BF16_TFLOPS = 2500.0        # MI355X dense bf16 MFMA (published)
PEAK_HBM_GBS = 8000.0
PEAK_FP32_MFMA_TFLOPS = 157.3     # MI355X dense fp32 matrix (published)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama8b_s128k_90")
    ap.add_argument("--dense-reps", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-train", action="store_true",
                    help="skip timing the ground-truth kernel and the gate's distillation step")
    ap.add_argument("--no-decode", action="store_true", help="skip timing the decode stage")
    ap.add_argument("--no-varlen", action="store_true", help="skip timing a packed varlen batch")
    ap.add_argument("--rope-theta", type=float, default=5e5,
                    help="RoPE base for the gate's block-level RoPE (0: none); Llama-3.1 uses 500000")
    ap.add_argument("--copy-gib", type=float, default=0.0,
                    help="run one plain device copy of this many GiB before the steps (counter calibration)")
    return ap.parse_args()


COUNTERS = os.path.join(ROOT, "profiles", "attn_sparse_llama8b_s128k_90_counters.md")
KERNEL_SRCS = [os.path.join(ROOT, "learned_block_sparse_attngate_amd", "csrc", f) for f in ("attn_kernels.hip", "tile_ops.h")]


def attention_source_digest():
    """sha256 over the attention kernels' source files (attn_kernels.hip, then
    tile_ops.h), which the committed counter summaries record."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SRCS:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per attention call from the committed FETCH_SIZE / WRITE_SIZE
    summary, or None if that summary is missing, is for another workload, or
    was taken on a different version of the attention kernels' source."""
    try:
        text = open(COUNTERS).read()
        src = attention_source_digest()
    except OSError:
        return None
    fields = dict(line.split(":", 1) for line in text.splitlines() if line.startswith("- ") and ":" in line)
    fields = {k[2:].strip(): v.strip().strip("`") for k, v in fields.items()}
    if fields.get("workload") != workload or fields.get("attention source sha256") != src:
        return None
    try:
        return int(fields["HBM bytes per call"])
    except (KeyError, ValueError):
        return None


MFMA_COUNTERS = os.path.join(ROOT, "profiles", "attn_sparse_llama8b_s128k_90_mfma_lds_counters.md")


def measured_mfma_busy(workload: str):
    """Fraction of the block-sparse call's kernel cycles its MFMA pipes were
    busy (rocprofv3 SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE x SIMDs) and
    the engine clock during it, from the committed counter summary; None if
    that summary is missing, for another workload, or for other kernel source."""
    import re
    try:
        text = open(MFMA_COUNTERS).read()
        src = attention_source_digest()
    except OSError:
        return None
    if workload not in text.splitlines()[0] or f"attention source sha256 `{src}`" not in text:
        return None
    busy = re.search(r"The MFMA pipes are busy ([0-9.]+)% of the kernel's cycles", text)
    clk = re.search(r"The engine clock during the kernel is ([0-9.]+) GHz", text)
    if not busy or not clk:
        return None
    return {"mfma_busy": round(float(busy.group(1)) / 100.0, 4), "engine_clock_ghz": float(clk.group(1)),
            "source": "profiles/attn_sparse_llama8b_s128k_90_mfma_lds_counters.md"}


def computed_peak():
    """Dense bf16 MFMA peak from the agent's compute-unit count and maximum
    engine clock as rocminfo reports them (4096 FLOP per clock per CU on
    gfx950), or None if rocminfo is unavailable."""
    import re
    import subprocess
    try:
        txt = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=30).stdout
    except Exception:                                          # pragma: no cover
        return None
    for agent in txt.split("Agent ")[1:]:
        if "gfx950" not in agent:
            continue
        cu = re.search(r"Compute Unit:\s+(\d+)", agent)
        mhz = re.search(r"Max Clock Freq\. \(MHz\):\s+(\d+)", agent)
        if cu and mhz:
            cus, clk = int(cu.group(1)), int(mhz.group(1))
            return {"cus": cus, "max_sclk_mhz": clk, "bf16_tflops": round(cus * 4096 * clk * 1e6 / 1e12, 1)}
    return None


def bench_decode(seer, torch, q, k, v, shape, stream, seed, reps: int = 50):
    """Decode stage on the same K/V cache: the newest token's query, a compressed
    K cache, a top-k decode gate keeping 10% of the blocks, and block-sparse
    decode attention; dense decode attention on the same cache for the speedup.
    The decode attention is bound by HBM reads of the selected K/V blocks."""
    import synth
    B, Hq, Hkv, S, D = shape.batch, shape.heads_q, shape.heads_kv, shape.seq_len, shape.head_dim
    nb = shape.nb
    dev = q.device
    qd = q[:, :, -1].contiguous()
    _, wk_np = synth.gen_gate_weights(Hq, D, D, seed + 200)
    wk = torch.from_numpy(wk_np).to(dev)
    kc = seer.seer_decode_compress_k(k, wk, Hq)
    k_dec = max(1, nb // 10)
    mask = torch.empty((B, Hq, nb), dtype=torch.uint8, device=dev)
    out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(seer.decode_attn_workspace_bytes(B, Hq, Hkv, S, D), dtype=torch.uint8, device=dev)

    def step():
        seer.seer_decode_compress_k(k, wk, Hq, kcomp=kc, block_begin=nb - 1)   # the block the new token joined
        seer.seer_decode_gate_fwd(qd, kc, S, Hkv, mode="topk", topk=k_dec, want_scores=False, block_mask=mask)
        seer.seer_decode_attn_fwd(qd, k, v, mask, out=out, workspace=ws)

    def sparse_attn():
        seer.seer_decode_attn_fwd(qd, k, v, mask, out=out, workspace=ws)

    def dense_attn():
        seer.seer_decode_attn_fwd(qd, k, v, None, out=out, workspace=ws)

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps          # microseconds

    step_us = timed(step)
    # the same step captured once as a HIP graph and replayed: the five
    # launches of a decode step without the per-launch host work
    step()
    torch.cuda.synchronize()
    ref = out.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    graph_us = timed(graph.replay)
    torch.cuda.synchronize()
    graph_same = bool(torch.equal(out, ref))
    sparse_us = timed(sparse_attn)
    dense_us = timed(dense_attn)
    m = mask.cpu().numpy().astype(bool).reshape(B, Hkv, Hq // Hkv, nb)
    union_blocks = int(m.any(axis=2).sum())               # blocks read: union over each KV group's heads
    blk_bytes = 2 * 64 * D * 2                            # K + V of one block, bf16
    sparse_bytes = union_blocks * blk_bytes + B * Hq * (nb + 4 * D)
    dense_bytes = B * Hkv * nb * blk_bytes + B * Hq * 4 * D
    print(f"[bench] decode step {step_us:.1f} us ({graph_us:.1f} us replayed as a graph, output "
          f"{'identical' if graph_same else 'DIFFERENT'}); decode attention sparse {sparse_us:.1f} us "
          f"({sparse_bytes / sparse_us / 1e3:.0f} GB/s), dense {dense_us:.1f} us "
          f"({dense_bytes / dense_us / 1e3:.0f} GB/s)", file=sys.stderr, flush=True)
    return {"workload": f"newest token of the {S}-token cache, top-k {k_dec} of {nb} blocks per head",
            "step_us": round(step_us, 2), "step_us_graph": round(graph_us, 2), "graph_output_identical": graph_same,
            "sparse_attention_us": round(sparse_us, 2),
            "dense_attention_us": round(dense_us, 2), "speedup_attention": round(dense_us / sparse_us, 3),
            "blocks_read_union": union_blocks, "blocks_selected": int(m.sum()),
            "roofline": {"bound": "hbm", "achieved": round(sparse_bytes / sparse_us / 1e3, 1),
                         "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(sparse_bytes / sparse_us / 1e3 / PEAK_HBM_GBS, 4),
                         "bytes_per_call": sparse_bytes},
            "dense_roofline_frac": round(dense_bytes / dense_us / 1e3 / PEAK_HBM_GBS, 4)}


def bench_varlen(seer, torch, dev, stream, seed, reps: int = 5):
    """Packed batches of Llama-3.1-8B-shaped sequences (no padding), each
    sequence with its own 90%-sparse seeded block mask, through the varlen
    block-sparse attention: 8 sequences of seeded lengths in [4k, 32k] tokens,
    and 64 sequences of 2048 tokens; TFLOP/s on executed tiles."""
    import synth
    rng = np.random.Generator(np.random.PCG64(seed + 300))
    batches = {"mixed_8x4k-32k": [int(x) for x in rng.integers(4096, 32769, size=8)],
               "uniform_64x2k": [2048] * 64}
    res = {}
    for bi, (name, lens) in enumerate(batches.items()):
        cu = [0] + [int(x) for x in np.cumsum(lens)]
        Hq, Hkv, D = 32, 8, 128
        T = cu[-1]
        g = torch.Generator(device=dev)
        g.manual_seed(seed + 301 + bi)
        q = torch.randn((Hq, T, D), generator=g, device=dev).to(torch.bfloat16)
        k = torch.randn((Hkv, T, D), generator=g, device=dev).to(torch.bfloat16)
        v = torch.randn((Hkv, T, D), generator=g, device=dev).to(torch.bfloat16)
        masks, tiles = [], 0
        for i, n in enumerate(lens):
            sh = synth.Shape(1, Hq, Hkv, n, D)
            m = synth.gen_block_mask(sh, seed + 310 + 100 * bi + i, 0.9).mask[0]
            nb = sh.nb
            tiles += int(np.count_nonzero(np.tril(np.ones((nb, nb), dtype=bool))[None] & m.astype(bool)))
            masks.append(m.reshape(-1))
        mask = torch.from_numpy(np.concatenate(masks)).to(dev)
        out = torch.empty((Hq, T, D), dtype=torch.bfloat16, device=dev)

        def run():
            seer.seer_block_sparse_attn_varlen_fwd(q, k, v, cu, mask, out=out)
        run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            run()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        tflops = tiles * 4.0 * 64 * 64 * D / ms / 1e9

        # the packed batch's gate (top-k 10% of each row's blocks, mask only)
        dg = 128
        wq = torch.randn((Hq, D, dg), generator=g, device=dev) / dg ** 0.5
        wk = torch.randn((Hq, 3 * D, dg), generator=g, device=dev) / dg ** 0.5
        gmask = torch.empty(mask.numel(), dtype=torch.uint8, device=dev)
        gws = torch.empty(max(seer.gate_varlen_workspace_bytes(cu, Hq, Hkv, D, dg, want_scores=False), 16),
                          dtype=torch.uint8, device=dev)
        k_top = max(1, (min(lens) // 64) // 10)

        def gate():
            seer.seer_gate_varlen_fwd(q, k, wq, wk, cu, mode="topk", topk=k_top, rope_theta=5e5, want_scores=False,
                                      block_mask=gmask, workspace=gws)
        gate()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            gate()
        e1.record(stream)
        torch.cuda.synchronize()
        gate_ms = e0.elapsed_time(e1) / reps
        print(f"[bench] varlen {name}: {len(lens)} sequences, {T} tokens, block-sparse attention {ms:.3f} ms "
              f"({tflops:.1f} TFLOP/s on executed tiles), gate {gate_ms:.3f} ms", file=sys.stderr, flush=True)
        res[name] = {"lengths": lens if len(set(lens)) > 1 else f"{len(lens)} x {lens[0]}", "tokens": T,
                     "sparse_attention_ms": round(ms, 4), "executed_tiles": tiles, "tflops": round(tflops, 2),
                     "gate_ms": round(gate_ms, 4), "gate_topk": k_top}
        del q, k, v, mask, out, gmask, gws
    return res


def mask_desc(sparsity) -> str:
    if isinstance(sparsity, tuple):
        lo, hi, mean = sparsity
        return f"seeded diag+sink+4 stripes+random, per-head s in [{lo},{hi}] with mean {mean}"
    return f"seeded diag+sink+4 stripes+random, s = {sparsity} for every head"


def topk_for_sparsity(nb: int, s: float) -> int:
    """Smallest k whose top-k causal mask has sparsity <= s."""
    total = nb * (nb + 1) // 2
    for k in range(1, nb + 1):
        kept = k * nb - k * (k - 1) // 2
        if 1.0 - kept / total <= s:
            return k
    return nb


def cpu_baseline(q, k, v, mask, shape, seconds: float):
    """Time the fp64 oracle on a bounded, seeded sample of query blocks."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:                                          # pragma: no cover
        threads = os.cpu_count() or 1
    rng = np.random.Generator(np.random.PCG64(12345))
    nb = shape.nb
    flops = 0.0
    rows_done = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        b = 0
        h = int(rng.integers(shape.heads_q))
        i = int(rng.integers(nb))
        oracle.attention_rows(q, k, v, mask, [(b, h, i)])
        tiles = int(np.count_nonzero(mask[b, h, i, :i + 1]))
        flops += 4.0 * 64 * 64 * shape.head_dim * tiles
        rows_done += 1
    el = time.perf_counter() - t0
    return {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "sample": f"{rows_done} random (head, query-block) rows of the same workload, fp64 NumPy, "
                      f"{el:.1f} s; rate = executed-tile FLOP / time"}


def cpu_model() -> str:
    """The host CPU's model name as lscpu reports it (/proc/cpuinfo if lscpu is absent)."""
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except Exception:                                          # pragma: no cover
        pass
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:                                            # pragma: no cover
        pass
    return "unknown"


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (got --gpus {args.gpus}); the library has no multi-GPU path",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import learned_block_sparse_attngate_amd as seer

    w = synth.WORKLOADS.get(args.workload)
    if w is None or not (isinstance(w["sparsity"], (float, tuple)) or w["sparsity"] == "gate"):
        usable = [k for k, v in synth.WORKLOADS.items() if isinstance(v["sparsity"], (float, tuple))
                  or v["sparsity"] == "gate"]
        print(f"bench.py needs a workload with a seeded or gate-made block mask, one of {usable} "
              f"(got {args.workload})", file=sys.stderr)
        sys.exit(2)
    # gate-made mask: planted Q/K, random-init weights, threshold mask from the gate feeds the attention
    gate_made = w["sparsity"] == "gate"
    seer.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = synth.WORKLOADS[args.workload]
    shape = w["shape"]
    B, Hq, Hkv, S, D = shape.batch, shape.heads_q, shape.heads_kv, shape.seq_len, shape.head_dim
    nb = shape.nb
    print(f"[bench] workload {args.workload}: B={B} Hq={Hq} Hkv={Hkv} S={S} D={D}; generating inputs",
          file=sys.stderr, flush=True)

    dg = w.get("gate_dim", 128)
    if gate_made:
        qb, kb, vb, _ = synth.gen_planted_qk(shape, w["seed"])
        mask_np = None                                  # the gate's mask, read back after the warm-up
    else:
        qb, kb, vb = synth.gen_qkv(shape, w["seed"])
        mask_np = synth.workload_mask(args.workload).mask
    wq_np, wk_np = synth.gen_gate_weights(Hq, D, dg, w["seed"] + 100)
    rope_theta = 0.0 if gate_made else args.rope_theta

    def to_dev_bf16(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v = to_dev_bf16(qb), to_dev_bf16(kb), to_dev_bf16(vb)
    wq, wk = torch.from_numpy(wq_np).to(dev), torch.from_numpy(wk_np).to(dev)
    out = torch.empty((B, Hq, S, D), dtype=torch.bfloat16, device=dev)
    gate_mask = torch.empty((B, Hq, nb, nb), dtype=torch.uint8, device=dev)
    # the step's gate call produces the block mask the attention consumes; the
    # fp32 scores are not stored (the distillation step recomputes them)
    gate_ws = torch.empty(seer.gate_workspace_bytes(B, Hq, Hkv, S, D, dg, want_scores=False), dtype=torch.uint8,
                          device=dev)
    k_gate = None if gate_made else topk_for_sparsity(nb, 0.9)
    mask = gate_mask if gate_made else torch.from_numpy(mask_np).to(dev)

    stream = torch.cuda.current_stream(dev)

    def gate():
        if gate_made:
            seer.seer_gate_fwd(q, k, wq, wk, mode="threshold", threshold=w["threshold"], want_scores=False,
                               block_mask=gate_mask, workspace=gate_ws)
        else:
            seer.seer_gate_fwd(q, k, wq, wk, mode="topk", topk=k_gate, rope_theta=rope_theta,
                               want_scores=False, block_mask=gate_mask, workspace=gate_ws)

    attn_ws = torch.empty(max(seer.attn_workspace_bytes(B, Hq, Hkv, S, D), 16), dtype=torch.uint8, device=dev)

    def attn():
        seer.seer_block_sparse_attn_fwd(q, k, v, mask, out=out, workspace=attn_ws)

    if args.copy_gib > 0:
        # a plain copy of known size: the counters' reading for it calibrates FETCH_SIZE / WRITE_SIZE
        n = int(args.copy_gib * (1 << 30)) // 4
        src_buf = torch.ones(n, dtype=torch.float32, device=dev)
        dst_buf = torch.empty_like(src_buf)
        dst_buf.copy_(src_buf)
        torch.cuda.synchronize()
        del src_buf, dst_buf
        print(f"[bench] copied {args.copy_gib} GiB device to device", file=sys.stderr, flush=True)

    print(f"[bench] warmup {args.warmup} steps", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        gate()
        attn()
    torch.cuda.synchronize()
    if gate_made:
        gate()
        torch.cuda.synchronize()
        mask_np = gate_mask.cpu().numpy()

    tiles = int(np.count_nonzero(np.tril(np.ones((nb, nb), dtype=bool)) & mask_np.astype(bool)))
    diag_tiles = int(np.count_nonzero(np.diagonal(mask_np, axis1=2, axis2=3)))
    causal_tiles = B * Hq * nb * (nb + 1) // 2
    flop_tile = 4.0 * 64 * 64 * D
    sparse_flop = tiles * flop_tile
    dense_flop = causal_tiles * flop_tile
    # useful work: a diagonal tile's causal part is 64 * 65 / 2 of its 64 * 64 entries
    useful_flop = (tiles - diag_tiles * 63.0 / 128.0) * flop_tile

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        gate()
        ev[i][1].record(stream)
        attn()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    gate_ms = [e[0].elapsed_time(e[1]) for e in ev]
    attn_ms = [e[1].elapsed_time(e[2]) for e in ev]
    step_ms = [a + g for a, g in zip(attn_ms, gate_ms)]
    print(f"[bench] timed {args.steps} steps: median step {np.median(step_ms):.3f} ms "
          f"(gate {np.median(gate_ms):.3f}, attention {np.median(attn_ms):.3f})", file=sys.stderr, flush=True)

    dense_ms = None
    if not args.no_dense:
        print("[bench] dense causal reference", file=sys.stderr, flush=True)
        seer.seer_block_sparse_attn_fwd(q, k, v, None, out=out)
        torch.cuda.synchronize()
        dts = []
        for _ in range(args.dense_reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            seer.seer_block_sparse_attn_fwd(q, k, v, None, out=out)
            e1.record(stream)
            torch.cuda.synchronize()
            dts.append(e0.elapsed_time(e1))
        dense_ms = float(np.median(dts))
        print(f"[bench] dense {dense_ms:.3f} ms ({dense_flop / dense_ms / 1e9:.1f} TFLOP/s)", file=sys.stderr,
              flush=True)

    gt_ms = distill_ms = None
    if not args.no_train:
        # training path: dense attention with the 2D-maxpooled map, then one
        # distillation step of the gate on that map (not part of `value`)
        print("[bench] ground-truth kernel and distillation step", file=sys.stderr, flush=True)
        gt = torch.empty((B, Hq, nb, nb), dtype=torch.float32, device=dev)
        gt_ws = torch.empty(seer.gt_workspace_bytes(B, Hq, Hkv, S, D), dtype=torch.uint8, device=dev)
        seer.seer_attn_maxpool_gt(q, k, v, out=out, gt=gt, workspace=gt_ws)
        torch.cuda.synchronize()
        dts = []
        for _ in range(args.dense_reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            seer.seer_attn_maxpool_gt(q, k, v, out=out, gt=gt, workspace=gt_ws)
            e1.record(stream)
            torch.cuda.synchronize()
            dts.append(e0.elapsed_time(e1))
        gt_ms = float(np.median(dts))
        del gt_ws
        d_ws = torch.empty(seer.distill_workspace_bytes(B, Hq, Hkv, S, D, dg), dtype=torch.uint8, device=dev)
        d_out = (torch.empty(1, dtype=torch.float32, device=dev), torch.empty_like(wq), torch.empty_like(wk))

        def distill():
            seer.seer_gate_distill_bwd(q, k, wq, wk, gt, rope_theta=rope_theta, loss=d_out[0],
                                       grad_wq=d_out[1], grad_wk=d_out[2], workspace=d_ws)
        distill()
        torch.cuda.synchronize()
        dts = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            distill()
            e1.record(stream)
            torch.cuda.synchronize()
            dts.append(e0.elapsed_time(e1))
        distill_ms = float(np.median(dts))
        print(f"[bench] dense + ground truth {gt_ms:.3f} ms, distillation step {distill_ms:.3f} ms "
              f"(loss {float(d_out[0].item()):.5f})", file=sys.stderr, flush=True)
        del d_ws, gt

    decode = None
    if not args.no_decode:
        decode = bench_decode(seer, torch, q, k, v, shape, stream, w["seed"])

    varlen = None
    if not args.no_varlen:
        varlen = bench_varlen(seer, torch, dev, stream, w["seed"])

    ms_step = float(np.mean(step_ms))
    attn_avg = float(np.mean(attn_ms))
    gate_avg = float(np.mean(gate_ms))
    s_real = 1.0 - tiles / causal_tiles
    achieved = sparse_flop / attn_avg / 1e9                     # TFLOP/s of the attention kernel
    peak = computed_peak()
    # the gate call's compulsory HBM bytes: Q and K read once (bf16) and the
    # u8 mask written once
    gate_bytes = 2 * B * S * D * (Hq + Hkv) + B * Hq * nb * nb
    # the gate's fp32 matrix work: the projections Q' = Qp W_q (D -> Dg per
    # query head) and K' = Kp W_k (3D -> Dg per W_k head), and the causal block
    # logits Q' K'^T. Its kernels run one after another (pool, projections,
    # logits, softmax / top-k), the HBM-bound ones moving the compulsory bytes
    # and the matrix ones doing this work, so the call takes at least
    # bytes / HBM peak + flop / fp32 matrix peak
    hwk = wk_np.shape[0]
    gate_flop = 2 * B * nb * dg * (Hq * D + hwk * 3 * D) + 2 * B * Hq * (nb * (nb + 1) // 2) * dg
    gate_bound_ms = gate_bytes / (PEAK_HBM_GBS * 1e6) + gate_flop / (PEAK_FP32_MFMA_TFLOPS * 1e9)
    rec = {
        "metric": METRIC,
        "value": round(sparse_flop / ms_step / 1e9, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "step_ms_median": round(float(np.median(step_ms)), 4),
        "step_ms_min": round(float(np.min(step_ms)), 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": B, "heads_q": Hq, "heads_kv": Hkv, "seq_len": S,
                   "head_dim": D, "block": 64, "gate_dim": dg,
                   "mask": (f"the gate's threshold mask (T = {w['threshold']}) on planted Q/K, random-init weights"
                            if gate_made else mask_desc(w["sparsity"])),
                   "realized_sparsity": round(s_real, 5), "executed_tiles": tiles,
                   "gate_mode": "threshold" if gate_made else "topk",
                   "gate_threshold": w["threshold"] if gate_made else None, "gate_topk": k_gate,
                   "gate_rope_theta": rope_theta},
        "breakdown_ms": {"gate": round(gate_avg, 4), "sparse_attention": round(attn_avg, 4),
                         "dense_attention": None if dense_ms is None else round(dense_ms, 4),
                         "dense_attention_with_gt_map": None if gt_ms is None else round(gt_ms, 4),
                         "gate_distillation_step": None if distill_ms is None else round(distill_ms, 4)},
        "speedup_vs_dense": None if dense_ms is None else {
            "kernel": round(dense_ms / attn_avg, 3),
            "with_gate": round(dense_ms / ms_step, 3),
            "target_0.8/(1-s)": round(0.8 / (1.0 - s_real), 3),
            "ideal_1/(1-s)": round(1.0 / (1.0 - s_real), 3)},
        "dense_tflops": None if dense_ms is None else round(dense_flop / dense_ms / 1e9, 2),
        "ground_truth": None if (gt_ms is None or dense_ms is None) else {
            "kernel": "seer_attn_maxpool_gt (dense attention + 2D-maxpooled map)",
            "ms": round(gt_ms, 4), "dense_ms": round(dense_ms, 4),
            "overhead_vs_dense": round(gt_ms / dense_ms - 1.0, 4),
            "map_shape": [B, Hq, nb, nb],
            "pages_overhead_vs_flashattention": "< 0.05 (explainer section 3.4, customized training kernel)"},
        "roofline": {"kernel": "seer_block_sparse_attn_fwd (one call: at 128k the two launches of the XCD-owned "
                               "chunk kernel, the second merging the partial outputs)",
                     "bound": "mfma", "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(args.workload),
                     "useful_tflops": round(useful_flop / attn_avg / 1e9, 2),
                     "attention_ms_median": round(float(np.median(attn_ms)), 4),
                     "attention_ms_min": round(float(np.min(attn_ms)), 4),
                     "frac_of_computed_peak": None if peak is None else round(achieved / peak["bf16_tflops"], 4),
                     "counters": measured_mfma_busy(args.workload)},
        "gate": {"kernel": "seer_gate_fwd (pool, projections, block RoPE, causal logits, softmax + top-k mask; "
                           "mask only, scores not stored)",
                 "ms": round(gate_avg, 4), "bound": "hbm",
                 "compulsory_bytes": gate_bytes,
                 "achieved": round(gate_bytes / gate_avg / 1e6, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                 "frac": round(gate_bytes / gate_avg / 1e6 / PEAK_HBM_GBS, 4),
                 "fp32_matrix_flop": gate_flop,
                 "time_bound_ms": round(gate_bound_ms, 4),
                 "time_bound": "compulsory bytes at the HBM peak plus the fp32 matrix work at its peak, in sequence",
                 "frac_of_time_bound": round(gate_bound_ms / gate_avg, 4)},
        "decode": decode,
        "varlen": varlen,
        "peak_computed": peak,
        "wall_s_timed": round(wall, 3),
    }
    if not args.no_cpu:
        print(f"[bench] cpu baseline (oracle, ~{args.cpu_seconds:.0f} s)", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(qb, kb, vb, mask_np, shape, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
