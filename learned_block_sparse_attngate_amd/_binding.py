"""ctypes binding of libseer.so (the C ABI in include/seer.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libseer.so. PyTorch supplies device memory and the current stream.
There is no fallback: if the library is missing or the GPU is not a gfx950,
the calls raise.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Union

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libseer.so")

SEER_OK = 0
SEER_ERR_INVALID_ARG = 1
SEER_ERR_SHAPE = 2
SEER_ERR_UNSUPPORTED = 3
SEER_ERR_WORKSPACE = 4
SEER_ERR_HIP = 5

SEER_MASK_THRESHOLD = 0
SEER_MASK_TOPK = 1
SEER_F32 = 0
SEER_BF16 = 1

BLOCK = 64

# Every symbol include/seer.h declares (checked by the CPU tests).
EXPORTED = (
    "seer_gate_workspace_size", "seer_gate_fwd",
    "seer_gate_distill_workspace_size", "seer_gate_distill_bwd",
    "seer_attn_workspace_size", "seer_block_sparse_attn_fwd",
    "seer_gt_workspace_size", "seer_attn_maxpool_gt",
    "seer_decode_compress_k", "seer_decode_gate_fwd", "seer_decode_attn_workspace_size", "seer_decode_attn_fwd",
    "seer_decode_attn_fwd_noalloc",
    "seer_varlen_map_elements", "seer_gate_varlen_workspace_size", "seer_gate_varlen_fwd",
    "seer_attn_varlen_workspace_size", "seer_block_sparse_attn_varlen_fwd", "seer_gt_varlen_workspace_size",
    "seer_attn_maxpool_gt_varlen",
    "seer_status_string", "seer_last_error", "seer_version",
)


class SeerShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads_q", ctypes.c_int32), ("heads_kv", ctypes.c_int32),
                ("seq_len", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("block", ctypes.c_int32)]


class SeerVarlen(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("heads_q", ctypes.c_int32), ("heads_kv", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("block", ctypes.c_int32), ("cu_seqlens", ctypes.POINTER(ctypes.c_int32))]


class SeerError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_status_name(status)}: {message}")
        self.status = status


_LIB = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libseer.so once and declare its signatures."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m learned_block_sparse_attngate_amd.build`")
    lib = ctypes.CDLL(path)
    vp, sz, i32, f32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_float
    shp = ctypes.POINTER(SeerShape)
    lib.seer_gate_workspace_size.argtypes = [shp, i32, i32, i32]
    lib.seer_gate_workspace_size.restype = sz
    lib.seer_gate_fwd.argtypes = [shp, i32, i32, f32, vp, vp, vp, vp, ctypes.c_int, f32, i32,
                                  ctypes.POINTER(i32), vp, vp, vp, sz, vp]
    lib.seer_gate_fwd.restype = ctypes.c_int
    lib.seer_gate_distill_workspace_size.argtypes = [shp, i32, i32]
    lib.seer_gate_distill_workspace_size.restype = sz
    lib.seer_gate_distill_bwd.argtypes = [shp, i32, i32, f32, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.seer_gate_distill_bwd.restype = ctypes.c_int
    lib.seer_attn_workspace_size.argtypes = [shp]
    lib.seer_attn_workspace_size.restype = sz
    lib.seer_block_sparse_attn_fwd.argtypes = [shp, vp, vp, vp, vp, vp, ctypes.c_int, vp, vp, sz, vp]
    lib.seer_block_sparse_attn_fwd.restype = ctypes.c_int
    lib.seer_gt_workspace_size.argtypes = [shp]
    lib.seer_gt_workspace_size.restype = sz
    lib.seer_attn_maxpool_gt.argtypes = [shp, vp, vp, vp, vp, ctypes.c_int, vp, vp, vp, sz, vp]
    lib.seer_attn_maxpool_gt.restype = ctypes.c_int
    lib.seer_decode_compress_k.argtypes = [shp, i32, vp, vp, i32, vp, i32, vp]
    lib.seer_decode_compress_k.restype = ctypes.c_int
    lib.seer_decode_gate_fwd.argtypes = [shp, i32, vp, vp, i32, ctypes.c_int, f32, i32, ctypes.POINTER(i32), vp, vp,
                                         vp]
    lib.seer_decode_gate_fwd.restype = ctypes.c_int
    lib.seer_decode_attn_workspace_size.argtypes = [shp]
    lib.seer_decode_attn_workspace_size.restype = sz
    lib.seer_decode_attn_fwd.argtypes = [shp, vp, vp, vp, vp, vp, ctypes.c_int, vp, vp, vp, sz, vp]
    lib.seer_decode_attn_fwd.restype = ctypes.c_int
    lib.seer_decode_attn_fwd_noalloc.argtypes = [shp, vp, vp, vp, vp, vp, ctypes.c_int, vp, vp, vp]
    lib.seer_decode_attn_fwd_noalloc.restype = ctypes.c_int
    vlp = ctypes.POINTER(SeerVarlen)
    lib.seer_varlen_map_elements.argtypes = [vlp]
    lib.seer_varlen_map_elements.restype = sz
    lib.seer_gate_varlen_workspace_size.argtypes = [vlp, i32, i32, i32]
    lib.seer_gate_varlen_workspace_size.restype = sz
    lib.seer_gate_varlen_fwd.argtypes = [vlp, i32, i32, f32, vp, vp, vp, vp, ctypes.c_int, f32, i32,
                                         ctypes.POINTER(i32), vp, vp, vp, sz, vp]
    lib.seer_gate_varlen_fwd.restype = ctypes.c_int
    lib.seer_attn_varlen_workspace_size.argtypes = [vlp]
    lib.seer_attn_varlen_workspace_size.restype = sz
    lib.seer_block_sparse_attn_varlen_fwd.argtypes = [vlp, vp, vp, vp, vp, vp, ctypes.c_int, vp, vp, sz, vp]
    lib.seer_block_sparse_attn_varlen_fwd.restype = ctypes.c_int
    lib.seer_gt_varlen_workspace_size.argtypes = [vlp]
    lib.seer_gt_varlen_workspace_size.restype = sz
    lib.seer_attn_maxpool_gt_varlen.argtypes = [vlp, vp, vp, vp, vp, ctypes.c_int, vp, vp, vp, sz, vp]
    lib.seer_attn_maxpool_gt_varlen.restype = ctypes.c_int
    lib.seer_status_string.argtypes = [ctypes.c_int]
    lib.seer_status_string.restype = ctypes.c_char_p
    lib.seer_last_error.argtypes = []
    lib.seer_last_error.restype = ctypes.c_char_p
    lib.seer_version.argtypes = []
    lib.seer_version.restype = ctypes.c_char_p
    _LIB = lib
    return lib


def _status_name(status: int) -> str:
    names = {0: "SEER_OK", 1: "SEER_ERR_INVALID_ARG", 2: "SEER_ERR_SHAPE", 3: "SEER_ERR_UNSUPPORTED",
             4: "SEER_ERR_WORKSPACE", 5: "SEER_ERR_HIP"}
    return names.get(status, f"status {status}")


def _check(status: int):
    if status != SEER_OK:
        msg = load_library().seer_last_error().decode(errors="replace")
        raise SeerError(status, msg)


def make_shape(batch, heads_q, heads_kv, seq_len, head_dim, block=BLOCK) -> SeerShape:
    return SeerShape(batch, heads_q, heads_kv, seq_len, head_dim, block)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name: str, dtype: torch.dtype, shape=None):
    """Validate one tensor before its pointer goes to the C ABI, which takes
    raw pointers and trusts their extents: type, dtype, exact shape and
    contiguity (the device is checked by _devices once every shape is).
    Raises TypeError / ValueError; nothing is launched."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name} must have shape {tuple(int(x) for x in shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _opt(t, name: str, dtype: torch.dtype, shape):
    if t is not None:
        _need(t, name, dtype, shape)


def _devices(dev: torch.device, **tensors):
    """Every given tensor is a CUDA (HIP) tensor on the device of q."""
    if dev.type != "cuda":
        raise TypeError(f"inputs must be CUDA (HIP) tensors, got device {dev}")
    for name, t in tensors.items():
        if t is not None and t.device != dev:
            raise ValueError(f"{name} is on {t.device}, expected {dev}")


def _out_dtype(dtype: torch.dtype, name: str = "out") -> int:
    if dtype == torch.bfloat16:
        return SEER_BF16
    if dtype == torch.float32:
        return SEER_F32
    raise TypeError(f"{name} must be bfloat16 or float32, got {dtype}")


def _check_out(out, lse, out_dtype, out_shape, lse_shape) -> int:
    """A caller-supplied out / lse must match the problem exactly; returns the C dtype of out."""
    if out is not None:
        if not isinstance(out, torch.Tensor):
            raise TypeError(f"out must be a torch.Tensor, got {type(out).__name__}")
        dt = _out_dtype(out.dtype)
        _need(out, "out", out.dtype, out_shape)
    else:
        dt = _out_dtype(out_dtype, "out_dtype")
    _opt(lse, "lse", torch.float32, lse_shape)
    return dt


def _dims(q, k, v, rank: int):
    """q [.., Hq, S, D] with k (and v) [.., Hkv, S, D] (rank 4: batch first;
    rank 3: packed heads-first), Hq a positive multiple of Hkv."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        if t is None:
            continue
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{n} must be a torch.Tensor, got {type(t).__name__}")
        if t.dim() != rank:
            raise ValueError(f"{n} must be {rank}-D, got shape {tuple(t.shape)}")
    hq, hkv = q.shape[-3], k.shape[-3]
    if hkv < 1 or hq % hkv != 0:
        raise ValueError(f"heads of q ({hq}) must be a positive multiple of the heads of k ({hkv})")
    kv_shape = tuple(q.shape[:-3]) + (hkv,) + tuple(q.shape[-2:])
    _need(q, "q", torch.bfloat16)
    _need(k, "k", torch.bfloat16, kv_shape)
    _opt(v, "v", torch.bfloat16, kv_shape)
    return tuple(q.shape), hkv


def _workspace(nbytes: int, device, workspace: Optional[torch.Tensor]):
    """The caller's workspace if it is large enough, else a new one."""
    if workspace is not None:
        if not isinstance(workspace, torch.Tensor) or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor")
        if workspace.device != device:
            raise ValueError(f"workspace is on {workspace.device}, expected {device}")
    if nbytes == 0:
        return workspace
    if workspace is not None and workspace.numel() * workspace.element_size() >= nbytes:
        return workspace
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def nblocks(seq_len: int) -> int:
    return -(-seq_len // BLOCK)


# ---------------------------------------------------------------------------
def _mask_args(mode: str, topk, heads_q: int):
    if mode not in ("topk", "threshold"):
        raise ValueError(f"mode must be 'threshold' or 'topk', got {mode!r}")
    m = SEER_MASK_TOPK if mode == "topk" else SEER_MASK_THRESHOLD
    per_head, k_uniform = None, 0
    if m == SEER_MASK_TOPK:
        if topk is None:
            raise ValueError("topk mode needs topk")
        if isinstance(topk, int):
            k_uniform = topk
        else:
            if len(topk) != heads_q:
                raise ValueError(f"per-head topk needs {heads_q} values")
            per_head = (ctypes.c_int32 * len(topk))(*[int(x) for x in topk])
    return m, k_uniform, per_head


def _gate_weights(w_q, w_k, heads_q, heads_kv, head_dim, wk_per_kv_head):
    if not isinstance(w_q, torch.Tensor) or w_q.dim() != 3:
        raise ValueError("w_q must be a 3-D tensor [Hq, D, Dg]")
    Dg = w_q.shape[-1]
    _need(w_q, "w_q", torch.float32, (heads_q, head_dim, Dg))
    _need(w_k, "w_k", torch.float32, (heads_kv if wk_per_kv_head else heads_q, 3 * head_dim, Dg))
    return Dg


def seer_gate_fwd(q: torch.Tensor, k: torch.Tensor, w_q: torch.Tensor, w_k: torch.Tensor, *,
                  mode: str = "threshold", threshold: float = 5e-4,
                  topk: Union[int, Sequence[int], None] = None, wk_per_kv_head: bool = False,
                  rope_theta: float = 0.0,
                  want_scores: bool = True, scores: Optional[torch.Tensor] = None,
                  block_mask: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """AttnGate scores and block mask. Returns (block_mask uint8, scores fp32 or None).

    rope_theta > 0 turns on the gate's block-level RoPE (q and k are then the
    model's pre-RoPE Q and K; rope_theta is the model's RoPE base)."""
    lib = load_library()
    (B, Hq, S, D), Hkv = _dims(q, k, None, 4)
    Dg = _gate_weights(w_q, w_k, Hq, Hkv, D, wk_per_kv_head)
    nb = nblocks(S)
    _opt(block_mask, "block_mask", torch.uint8, (B, Hq, nb, nb))
    _opt(scores, "scores", torch.float32, (B, Hq, nb, nb))
    m, k_uniform, per_head = _mask_args(mode, topk, Hq)
    dev = q.device
    _devices(dev, k=k, w_q=w_q, w_k=w_k, block_mask=block_mask, scores=scores)
    shape = make_shape(B, Hq, Hkv, S, D)
    if block_mask is None:
        block_mask = torch.empty((B, Hq, nb, nb), dtype=torch.uint8, device=dev)
    if want_scores and scores is None:
        scores = torch.empty((B, Hq, nb, nb), dtype=torch.float32, device=dev)
    if not want_scores:
        scores = None
    nbytes = lib.seer_gate_workspace_size(ctypes.byref(shape), Dg, int(wk_per_kv_head), int(scores is not None))
    workspace = _workspace(nbytes, dev, workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.seer_gate_fwd(ctypes.byref(shape), Dg, int(wk_per_kv_head), float(rope_theta),
                             _ptr(q), _ptr(k), _ptr(w_q), _ptr(w_k),
                             m, float(threshold), int(k_uniform), per_head, _ptr(scores), _ptr(block_mask),
                             _ptr(workspace), ws_bytes, _stream(dev)))
    return block_mask, scores


def seer_block_sparse_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                               block_mask: Optional[torch.Tensor] = None, *,
                               out: Optional[torch.Tensor] = None, out_dtype: torch.dtype = torch.bfloat16,
                               lse: Optional[torch.Tensor] = None, want_lse: bool = False,
                               workspace: Optional[torch.Tensor] = None):
    """Causal GQA block-sparse attention (block_mask=None: dense causal). Returns (out, lse or None)."""
    lib = load_library()
    (B, Hq, S, D), Hkv = _dims(q, k, v, 4)
    nb = nblocks(S)
    _opt(block_mask, "block_mask", torch.uint8, (B, Hq, nb, nb))
    dt = _check_out(out, lse, out_dtype, (B, Hq, S, D), (B, Hq, S))
    dev = q.device
    _devices(dev, k=k, v=v, block_mask=block_mask, out=out, lse=lse)
    shape = make_shape(B, Hq, Hkv, S, D)
    if out is None:
        out = torch.empty((B, Hq, S, D), dtype=out_dtype, device=dev)
    if want_lse and lse is None:
        lse = torch.empty((B, Hq, S), dtype=torch.float32, device=dev)
    ws_bytes = 0
    if block_mask is not None:
        workspace = _workspace(lib.seer_attn_workspace_size(ctypes.byref(shape)), dev, workspace)
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    else:
        workspace = None
    _check(lib.seer_block_sparse_attn_fwd(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(block_mask),
                                          _ptr(out), dt, _ptr(lse), _ptr(workspace), ws_bytes, _stream(dev)))
    return out, lse


def seer_attn_maxpool_gt(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *,
                         out: Optional[torch.Tensor] = None, out_dtype: torch.dtype = torch.bfloat16,
                         lse: Optional[torch.Tensor] = None, want_lse: bool = False,
                         gt: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """Dense causal attention plus the 2D-maxpooled map. Returns (out, lse or None, gt)."""
    lib = load_library()
    (B, Hq, S, D), Hkv = _dims(q, k, v, 4)
    nb = nblocks(S)
    dt = _check_out(out, lse, out_dtype, (B, Hq, S, D), (B, Hq, S))
    _opt(gt, "gt", torch.float32, (B, Hq, nb, nb))
    dev = q.device
    _devices(dev, k=k, v=v, out=out, lse=lse, gt=gt)
    shape = make_shape(B, Hq, Hkv, S, D)
    if out is None:
        out = torch.empty((B, Hq, S, D), dtype=out_dtype, device=dev)
    if want_lse and lse is None:
        lse = torch.empty((B, Hq, S), dtype=torch.float32, device=dev)
    if gt is None:
        gt = torch.empty((B, Hq, nb, nb), dtype=torch.float32, device=dev)
    workspace = _workspace(lib.seer_gt_workspace_size(ctypes.byref(shape)), dev, workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.seer_attn_maxpool_gt(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(out), dt, _ptr(lse),
                                    _ptr(gt), _ptr(workspace), ws_bytes, _stream(dev)))
    return out, lse, gt


def seer_decode_compress_k(k_cache: torch.Tensor, w_k: torch.Tensor, heads_q: int, *, wk_per_kv_head: bool = False,
                           block_begin: int = 0, kcomp: Optional[torch.Tensor] = None,
                           capacity_blocks: Optional[int] = None):
    """(Re)compute the compressed K cache of blocks >= block_begin. Returns kcomp
    [B, Hwk, capacity_blocks, D] fp32."""
    lib = load_library()
    if not isinstance(k_cache, torch.Tensor) or k_cache.dim() != 4:
        raise ValueError("k_cache must be a 4-D tensor [B, Hkv, S, D]")
    B, Hkv, S, D = k_cache.shape
    _need(k_cache, "k_cache", torch.bfloat16)
    if heads_q < 1 or heads_q % Hkv != 0:
        raise ValueError(f"heads_q ({heads_q}) must be a positive multiple of the cache's {Hkv} heads")
    nb = nblocks(S)
    hwk = Hkv if wk_per_kv_head else heads_q
    _need(w_k, "w_k", torch.float32, (hwk, 3 * D, D))
    if kcomp is not None:
        if not isinstance(kcomp, torch.Tensor) or kcomp.dim() != 4:
            raise ValueError("kcomp must be a 4-D tensor [B, Hwk, capacity_blocks, D]")
        _need(kcomp, "kcomp", torch.float32, (B, hwk, kcomp.shape[2], D))
    dev = k_cache.device
    _devices(dev, w_k=w_k, kcomp=kcomp)
    if kcomp is None:
        kcomp = torch.empty((B, hwk, capacity_blocks or nb, D), dtype=torch.float32, device=dev)
    shape = make_shape(B, heads_q, Hkv, S, D)
    _check(lib.seer_decode_compress_k(ctypes.byref(shape), int(wk_per_kv_head), _ptr(k_cache), _ptr(w_k),
                                      int(block_begin), _ptr(kcomp), int(kcomp.shape[2]), _stream(dev)))
    return kcomp


def seer_decode_gate_fwd(q: torch.Tensor, kcomp: torch.Tensor, seq_len: int, heads_kv: int, *,
                         wk_per_kv_head: bool = False, mode: str = "threshold", threshold: float = 5e-4,
                         topk: Union[int, Sequence[int], None] = None, want_scores: bool = True,
                         scores: Optional[torch.Tensor] = None, block_mask: Optional[torch.Tensor] = None):
    """Decode gate for one query per head. Returns (block_mask [B,Hq,nb] uint8, scores or None)."""
    lib = load_library()
    if not isinstance(q, torch.Tensor) or q.dim() != 3:
        raise ValueError("q must be a 3-D tensor [B, Hq, D]")
    B, Hq, D = q.shape
    _need(q, "q", torch.bfloat16)
    if heads_kv < 1 or Hq % heads_kv != 0:
        raise ValueError(f"heads of q ({Hq}) must be a positive multiple of heads_kv ({heads_kv})")
    nb = nblocks(seq_len)
    if not isinstance(kcomp, torch.Tensor) or kcomp.dim() != 4:
        raise ValueError("kcomp must be a 4-D tensor [B, Hwk, capacity_blocks, D]")
    hwk = heads_kv if wk_per_kv_head else Hq
    _need(kcomp, "kcomp", torch.float32, (B, hwk, kcomp.shape[2], D))
    _opt(block_mask, "block_mask", torch.uint8, (B, Hq, nb))
    _opt(scores, "scores", torch.float32, (B, Hq, nb))
    m, k_uniform, per_head = _mask_args(mode, topk, Hq)
    dev = q.device
    _devices(dev, kcomp=kcomp, block_mask=block_mask, scores=scores)
    if block_mask is None:
        block_mask = torch.empty((B, Hq, nb), dtype=torch.uint8, device=dev)
    if scores is None:
        scores = torch.empty((B, Hq, nb), dtype=torch.float32, device=dev)
    shape = make_shape(B, Hq, heads_kv, seq_len, D)
    _check(lib.seer_decode_gate_fwd(ctypes.byref(shape), int(wk_per_kv_head), _ptr(q), _ptr(kcomp),
                                    int(kcomp.shape[2]), m, float(threshold), int(k_uniform), per_head, _ptr(scores),
                                    _ptr(block_mask), _stream(dev)))
    return block_mask, (scores if want_scores else None)


def seer_decode_attn_fwd(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                         block_mask: Optional[torch.Tensor] = None, *, out: Optional[torch.Tensor] = None,
                         out_dtype: torch.dtype = torch.bfloat16, lse: Optional[torch.Tensor] = None,
                         want_lse: bool = False, want_gt: bool = False, gt: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None):
    """Decode attention of one query per head over the active blocks of the
    cache. Returns (out [B,Hq,D], lse or None, gt [B,Hq,nb] or None)."""
    lib = load_library()
    if not isinstance(q, torch.Tensor) or q.dim() != 3:
        raise ValueError("q must be a 3-D tensor [B, Hq, D]")
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        if not isinstance(t, torch.Tensor) or t.dim() != 4:
            raise ValueError(f"{n} must be a 4-D tensor [B, Hkv, S, D]")
    B, Hq, D = q.shape
    Hkv, S = k_cache.shape[1], k_cache.shape[2]
    if Hkv < 1 or Hq % Hkv != 0:
        raise ValueError(f"heads of q ({Hq}) must be a positive multiple of the cache's {Hkv} heads")
    _need(q, "q", torch.bfloat16)
    _need(k_cache, "k_cache", torch.bfloat16, (B, Hkv, S, D))
    _need(v_cache, "v_cache", torch.bfloat16, (B, Hkv, S, D))
    nb = nblocks(S)
    _opt(block_mask, "block_mask", torch.uint8, (B, Hq, nb))
    dt = _check_out(out, lse, out_dtype, (B, Hq, D), (B, Hq))
    _opt(gt, "gt", torch.float32, (B, Hq, nb))
    dev = q.device
    _devices(dev, k_cache=k_cache, v_cache=v_cache, block_mask=block_mask, out=out, lse=lse, gt=gt)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=out_dtype, device=dev)
    if want_lse and lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    if want_gt and gt is None:
        gt = torch.empty((B, Hq, nb), dtype=torch.float32, device=dev)
    shape = make_shape(B, Hq, Hkv, S, D)
    workspace = _workspace(lib.seer_decode_attn_workspace_size(ctypes.byref(shape)), dev, workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.seer_decode_attn_fwd(ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_mask),
                                    _ptr(out), dt, _ptr(lse), _ptr(gt), _ptr(workspace), ws_bytes, _stream(dev)))
    return out, lse, gt


NOALLOC_SCRATCH_BYTES = 16 << 20    # SEER_NOALLOC_SCRATCH_BYTES


def seer_decode_attn_fwd_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                                 block_mask: Optional[torch.Tensor], out: torch.Tensor, *,
                                 lse: Optional[torch.Tensor] = None, gt: Optional[torch.Tensor] = None):
    """Decode attention through the allocation-free entry point: the caller
    passes every output, the library uses its own fixed device scratch, and
    nothing is allocated. Same results as seer_decode_attn_fwd. Calls that
    overlap on one device share that scratch and must be serialized."""
    lib = load_library()
    if not isinstance(q, torch.Tensor) or q.dim() != 3:
        raise ValueError("q must be a 3-D tensor [B, Hq, D]")
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        if not isinstance(t, torch.Tensor) or t.dim() != 4:
            raise ValueError(f"{n} must be a 4-D tensor [B, Hkv, S, D]")
    B, Hq, D = q.shape
    Hkv, S = k_cache.shape[1], k_cache.shape[2]
    if Hkv < 1 or Hq % Hkv != 0:
        raise ValueError(f"heads of q ({Hq}) must be a positive multiple of the cache's {Hkv} heads")
    _need(q, "q", torch.bfloat16)
    _need(k_cache, "k_cache", torch.bfloat16, (B, Hkv, S, D))
    _need(v_cache, "v_cache", torch.bfloat16, (B, Hkv, S, D))
    nb = nblocks(S)
    _opt(block_mask, "block_mask", torch.uint8, (B, Hq, nb))
    if out is None:
        raise ValueError("the allocation-free call needs a caller-provided out")
    dt = _check_out(out, lse, out.dtype, (B, Hq, D), (B, Hq))
    _opt(gt, "gt", torch.float32, (B, Hq, nb))
    dev = q.device
    _devices(dev, k_cache=k_cache, v_cache=v_cache, block_mask=block_mask, out=out, lse=lse, gt=gt)
    shape = make_shape(B, Hq, Hkv, S, D)
    _check(lib.seer_decode_attn_fwd_noalloc(ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                            _ptr(block_mask), _ptr(out), dt, _ptr(lse), _ptr(gt), _stream(dev)))
    return out, lse, gt


def make_varlen(cu_seqlens: Sequence[int], heads_q: int, heads_kv: int, head_dim: int, block: int = BLOCK):
    """Varlen descriptor; the returned object keeps the host offsets alive."""
    arr = (ctypes.c_int32 * len(cu_seqlens))(*[int(x) for x in cu_seqlens])
    vl = SeerVarlen(len(cu_seqlens) - 1, heads_q, heads_kv, head_dim, block, arr)
    vl._keep = arr
    return vl


def gate_varlen_workspace_bytes(cu_seqlens: Sequence[int], heads_q: int, heads_kv: int, head_dim: int,
                                gate_dim: int, wk_per_kv_head: bool = False, want_scores: bool = True) -> int:
    """Workspace of seer_gate_varlen_fwd for this packed batch."""
    vl = make_varlen(cu_seqlens, heads_q, heads_kv, head_dim)
    return load_library().seer_gate_varlen_workspace_size(ctypes.byref(vl), gate_dim, int(wk_per_kv_head),
                                                          int(want_scores))


def varlen_map_offsets(cu_seqlens: Sequence[int], heads_q: int):
    """Element offset of each sequence's [Hq, nb_i, nb_i] block map, and the total."""
    offs, n = [], 0
    for a, b in zip(cu_seqlens[:-1], cu_seqlens[1:]):
        offs.append(n)
        nb = nblocks(b - a)
        n += heads_q * nb * nb
    return offs, n


def _varlen_dims(q, k, v, cu_seqlens):
    (Hq, T, D), Hkv = _dims(q, k, v, 3)
    cu = [int(x) for x in cu_seqlens]
    if len(cu) < 1 or cu[0] != 0 or cu[-1] != T or any(b < a for a, b in zip(cu[:-1], cu[1:])):
        raise ValueError(f"cu_seqlens must rise from 0 to the packed length {T}")
    return Hq, Hkv, T, D, cu, varlen_map_offsets(cu, Hq)[1]


def seer_gate_varlen_fwd(q: torch.Tensor, k: torch.Tensor, w_q: torch.Tensor, w_k: torch.Tensor,
                         cu_seqlens: Sequence[int], *, mode: str = "threshold", threshold: float = 5e-4,
                         topk: Union[int, Sequence[int], None] = None, wk_per_kv_head: bool = False,
                         rope_theta: float = 0.0, want_scores: bool = True, scores: Optional[torch.Tensor] = None,
                         block_mask: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """Gate of a packed batch (q [Hq,T,D], k [Hkv,T,D]). Returns (block_mask, scores or None),
    each sequence's [Hq, nb_i, nb_i] map concatenated (see varlen_map_offsets)."""
    lib = load_library()
    Hq, Hkv, T, D, cu, n_map = _varlen_dims(q, k, None, cu_seqlens)
    Dg = _gate_weights(w_q, w_k, Hq, Hkv, D, wk_per_kv_head)
    _opt(block_mask, "block_mask", torch.uint8, (n_map,))
    _opt(scores, "scores", torch.float32, (n_map,))
    m, k_uniform, per_head = _mask_args(mode, topk, Hq)
    dev = q.device
    _devices(dev, k=k, w_q=w_q, w_k=w_k, block_mask=block_mask, scores=scores)
    vl = make_varlen(cu, Hq, Hkv, D)
    if block_mask is None:
        block_mask = torch.empty(n_map, dtype=torch.uint8, device=dev)
    if want_scores and scores is None:
        scores = torch.empty(n_map, dtype=torch.float32, device=dev)
    if not want_scores:
        scores = None
    nbytes = lib.seer_gate_varlen_workspace_size(ctypes.byref(vl), Dg, int(wk_per_kv_head), int(scores is not None))
    workspace = _workspace(nbytes, dev, workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.seer_gate_varlen_fwd(ctypes.byref(vl), Dg, int(wk_per_kv_head), float(rope_theta), _ptr(q), _ptr(k),
                                    _ptr(w_q), _ptr(w_k), m, float(threshold), int(k_uniform), per_head, _ptr(scores),
                                    _ptr(block_mask), _ptr(workspace), ws_bytes, _stream(dev)))
    return block_mask, scores


def seer_block_sparse_attn_varlen_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: Sequence[int],
                                      block_mask: Optional[torch.Tensor] = None, *,
                                      out: Optional[torch.Tensor] = None, out_dtype: torch.dtype = torch.bfloat16,
                                      lse: Optional[torch.Tensor] = None, want_lse: bool = False,
                                      workspace: Optional[torch.Tensor] = None):
    """Causal GQA block-sparse attention of a packed batch (block_mask None: dense).
    Returns (out [Hq,T,D], lse [Hq,T] or None)."""
    lib = load_library()
    Hq, Hkv, T, D, cu, n_map = _varlen_dims(q, k, v, cu_seqlens)
    _opt(block_mask, "block_mask", torch.uint8, (n_map,))
    dt = _check_out(out, lse, out_dtype, (Hq, T, D), (Hq, T))
    dev = q.device
    _devices(dev, k=k, v=v, block_mask=block_mask, out=out, lse=lse)
    vl = make_varlen(cu, Hq, Hkv, D)
    if out is None:
        out = torch.empty((Hq, T, D), dtype=out_dtype, device=dev)
    if want_lse and lse is None:
        lse = torch.empty((Hq, T), dtype=torch.float32, device=dev)
    ws_need = lib.seer_attn_varlen_workspace_size(ctypes.byref(vl)) if block_mask is not None else 0
    workspace = _workspace(ws_need, dev, workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.seer_block_sparse_attn_varlen_fwd(ctypes.byref(vl), _ptr(q), _ptr(k), _ptr(v), _ptr(block_mask),
                                                 _ptr(out), dt, _ptr(lse), _ptr(workspace), ws_bytes, _stream(dev)))
    return out, lse


def seer_attn_maxpool_gt_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: Sequence[int], *,
                                out: Optional[torch.Tensor] = None, out_dtype: torch.dtype = torch.bfloat16,
                                lse: Optional[torch.Tensor] = None, want_lse: bool = False,
                                gt: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """Dense attention of a packed batch plus each sequence's 2D-maxpooled map. Returns (out, lse or None, gt)."""
    lib = load_library()
    Hq, Hkv, T, D, cu, n_map = _varlen_dims(q, k, v, cu_seqlens)
    dt = _check_out(out, lse, out_dtype, (Hq, T, D), (Hq, T))
    _opt(gt, "gt", torch.float32, (n_map,))
    dev = q.device
    _devices(dev, k=k, v=v, out=out, lse=lse, gt=gt)
    vl = make_varlen(cu, Hq, Hkv, D)
    if out is None:
        out = torch.empty((Hq, T, D), dtype=out_dtype, device=dev)
    if want_lse and lse is None:
        lse = torch.empty((Hq, T), dtype=torch.float32, device=dev)
    if gt is None:
        gt = torch.empty(n_map, dtype=torch.float32, device=dev)
    workspace = _workspace(lib.seer_gt_varlen_workspace_size(ctypes.byref(vl)), dev, workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.seer_attn_maxpool_gt_varlen(ctypes.byref(vl), _ptr(q), _ptr(k), _ptr(v), _ptr(out), dt, _ptr(lse),
                                           _ptr(gt), _ptr(workspace), ws_bytes, _stream(dev)))
    return out, lse, gt


def decode_attn_workspace_bytes(batch, heads_q, heads_kv, seq_len, head_dim) -> int:
    shape = make_shape(batch, heads_q, heads_kv, seq_len, head_dim)
    return load_library().seer_decode_attn_workspace_size(ctypes.byref(shape))


def seer_gate_distill_bwd(q: torch.Tensor, k: torch.Tensor, w_q: torch.Tensor, w_k: torch.Tensor,
                          gt: torch.Tensor, *, wk_per_kv_head: bool = False, rope_theta: float = 0.0,
                          loss: Optional[torch.Tensor] = None, grad_wq: Optional[torch.Tensor] = None,
                          grad_wk: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """One distillation step of the gate: KL(row-normalized gt || score) averaged
    over query-block rows, and its gradients. Returns (loss [1], grad_wq, grad_wk)."""
    lib = load_library()
    (B, Hq, S, D), Hkv = _dims(q, k, None, 4)
    Dg = _gate_weights(w_q, w_k, Hq, Hkv, D, wk_per_kv_head)
    nb = nblocks(S)
    _need(gt, "gt", torch.float32, (B, Hq, nb, nb))
    _opt(loss, "loss", torch.float32, (1,))
    _opt(grad_wq, "grad_wq", torch.float32, tuple(w_q.shape))
    _opt(grad_wk, "grad_wk", torch.float32, tuple(w_k.shape))
    dev = q.device
    _devices(dev, k=k, w_q=w_q, w_k=w_k, gt=gt, loss=loss, grad_wq=grad_wq, grad_wk=grad_wk)
    shape = make_shape(B, Hq, Hkv, S, D)
    if loss is None:
        loss = torch.empty(1, dtype=torch.float32, device=dev)
    if grad_wq is None:
        grad_wq = torch.empty_like(w_q)
    if grad_wk is None:
        grad_wk = torch.empty_like(w_k)
    nbytes = lib.seer_gate_distill_workspace_size(ctypes.byref(shape), Dg, int(wk_per_kv_head))
    workspace = _workspace(nbytes, dev, workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.seer_gate_distill_bwd(ctypes.byref(shape), Dg, int(wk_per_kv_head), float(rope_theta), _ptr(q),
                                     _ptr(k), _ptr(w_q), _ptr(w_k), _ptr(gt), _ptr(loss), _ptr(grad_wq),
                                     _ptr(grad_wk), _ptr(workspace), ws_bytes, _stream(dev)))
    return loss, grad_wq, grad_wk


def distill_workspace_bytes(batch, heads_q, heads_kv, seq_len, head_dim, gate_dim, wk_per_kv_head=False) -> int:
    shape = make_shape(batch, heads_q, heads_kv, seq_len, head_dim)
    return load_library().seer_gate_distill_workspace_size(ctypes.byref(shape), gate_dim, int(wk_per_kv_head))


def attn_workspace_bytes(batch, heads_q, heads_kv, seq_len, head_dim) -> int:
    shape = make_shape(batch, heads_q, heads_kv, seq_len, head_dim)
    return load_library().seer_attn_workspace_size(ctypes.byref(shape))


def gt_workspace_bytes(batch, heads_q, heads_kv, seq_len, head_dim) -> int:
    shape = make_shape(batch, heads_q, heads_kv, seq_len, head_dim)
    return load_library().seer_gt_workspace_size(ctypes.byref(shape))


def gate_workspace_bytes(batch, heads_q, heads_kv, seq_len, head_dim, gate_dim, wk_per_kv_head=False,
                         want_scores=True) -> int:
    shape = make_shape(batch, heads_q, heads_kv, seq_len, head_dim)
    return load_library().seer_gate_workspace_size(ctypes.byref(shape), gate_dim, int(wk_per_kv_head),
                                                   int(want_scores))


def version() -> str:
    return load_library().seer_version().decode()
