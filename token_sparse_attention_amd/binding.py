"""Thin ctypes binding of libmcs (include/mcs.h) for torch tensors.

Argument marshalling only: every step of the path runs in the HIP kernels of
libmcs.so.  PyTorch provides device memory and the current HIP stream.  If the
library has not been built, importing this module raises.

Tensor conventions: q, k, v, outputs and residuals are bf16 [B, H, N, D]
contiguous device tensors; perm int32 [B, H, N]; kv_idx int32 [B, H, G, K]
with G = ceil(N / C); lse float32 [B, H, N].
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("MCS_LIB", os.path.join(_HERE, "libmcs.so"))

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"libmcs.so not found at {LIB_PATH}: build it with "
        "`python -m token_sparse_attention_amd.build` (there is no CPU fallback)")

_lib = ctypes.CDLL(LIB_PATH)


class Dims(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("N", ctypes.c_int32), ("D", ctypes.c_int32)]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_F = ctypes.c_float

_SIGS = {
    "mcs_dense_attn": ([_P, _P, _P, _P, _P, Dims, _F, _P], _I32),
    "mcs_sparse_attn": ([_P, _P, _P, _P, _P, _P, _P, Dims, _I32, _I32, _F, _P], _I32),
    "mcs_dense_attn_f32out": ([_P, _P, _P, _P, _P, Dims, _F, _P], _I32),
    "mcs_sparse_attn_f32out": ([_P, _P, _P, _P, _P, _P, _P, Dims, _I32, _I32, _F, _P], _I32),
    "mcs_residual_update": ([_P, _P, _P, _I64, _P], _I32),
    "mcs_sparse_attn_ex": ([_P, _P, _P, _P, _P, _P, _P, _P, _I32, _P, Dims, _I32, _I32, _F, _P], _I32),
    "mcs_select_blocks": ([_P, _P, _P, _P, _P, Dims, _I32, _I32, _F, _P, _SZ, _P], _I32),
    "mcs_select_blocks_workspace": ([Dims], _SZ),
    "mcs_query_quality": ([_P, _P, _P, _P, _P, _P, _P, Dims, _P], _I32),
    "mcs_row_sums": ([_P, _P, _I64, _I64, _P], _I32),
    "mcs_kmeans": ([_P, _P, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _P, _SZ, _P], _I32),
    "mcs_kmeans_workspace": ([_I32, _I32], _SZ),
    "mcs_select": ([_P, _P, _P, _P, _P, Dims, _I32, _I32, _F, _P, _SZ, _P], _I32),
    "mcs_select_two_pass": ([_P, _P, _P, _P, _P, Dims, _I32, _I32, _F, _P, _SZ, _P], _I32),
    "mcs_select_workspace": ([Dims, _I32, _I32], _SZ),
    "mcs_select_workspace_all_heads": ([Dims, _I32, _I32], _SZ),
    "mcs_topk": ([_P, _P, _I64, _I32, _I32, _P], _I32),
    "mcs_group": ([_P, _P, Dims, _I32, _I32, _P, _SZ, _P], _I32),
    "mcs_group_workspace": ([Dims, _I32], _SZ),
    "mcs_group_noalloc": ([_P, _P, Dims, _I32, _I32, _P], _I32),
    "mcs_status_string": ([_I32], ctypes.c_char_p),
    "mcs_last_error": ([], ctypes.c_char_p),
    "mcs_version": ([], _I32),
}
for _name, (_args, _ret) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.argtypes = _args
    _fn.restype = _ret


class McsError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{_lib.mcs_status_string(status).decode()} ({status}): {detail}")
        self.status = status


def _check(status: int) -> None:
    if status != 0:
        raise McsError(status, _lib.mcs_last_error().decode())


def version() -> int:
    return _lib.mcs_version()


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _need(t: torch.Tensor, name: str, dtype, ndim: int) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims (got shape {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _like(t: torch.Tensor, name: str, dtype, shape, device) -> None:
    """t must be a contiguous tensor of this dtype and shape on this device: the
    kernels address it from the dimensions alone."""
    _need(t, name, dtype, len(shape))
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if t.device != device:
        raise ValueError(f"{name} must be on {device} (got {t.device})")


def dims_of(q: torch.Tensor) -> Dims:
    B, H, N, D = q.shape
    return Dims(B, H, N, D)


def num_groups(N: int, C: int) -> int:
    return -(-N // C)


def default_scale(D: int) -> float:
    return 1.0 / math.sqrt(D)


def heads_major(x: torch.Tensor) -> torch.Tensor:
    """[B, N, H, D] (the token-major layout of a transformer's projections) ->
    contiguous [B, H, N, D], the layout every call takes.  A torch copy, made
    once per tensor before the calls (outside the attention path)."""
    if x.dim() != 4:
        raise ValueError("expected a [B, N, H, D] tensor")
    return x.transpose(1, 2).contiguous()


def tokens_major(x: torch.Tensor) -> torch.Tensor:
    """Inverse of heads_major: [B, H, N, D] -> contiguous [B, N, H, D]."""
    if x.dim() != 4:
        raise ValueError("expected a [B, H, N, D] tensor")
    return x.transpose(1, 2).contiguous()


def _qkv(q, k, v=None):
    _need(q, "q", torch.bfloat16, 4)
    _like(k, "k", torch.bfloat16, q.shape, q.device)
    if v is not None:
        _like(v, "v", torch.bfloat16, q.shape, q.device)


def _out(q, out, out_dtype):
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    if not isinstance(out, torch.Tensor) or out.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("out must be a bf16 or float32 tensor")
    _like(out, "out", out.dtype, q.shape, q.device)
    return out


def dense_attn(q, k, v, scale=None, want_lse=False, out=None, lse=None, out_dtype=torch.bfloat16):
    """mcs_dense_attn(_f32out): softmax(scale q k^T) v per head, optionally the row LSE.

    The output is bf16 unless out (or out_dtype) is float32."""
    _qkv(q, k, v)
    B, H, N, D = q.shape
    scale = default_scale(D) if scale is None else scale
    out = _out(q, out, out_dtype)
    if want_lse and lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    elif want_lse:
        _like(lse, "lse", torch.float32, (B, H, N), q.device)
    fn = _lib.mcs_dense_attn_f32out if out.dtype == torch.float32 else _lib.mcs_dense_attn
    _check(fn(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse if want_lse else None), dims_of(q), scale,
              _stream(q)))
    return (out, lse) if want_lse else out


def sparse_attn(q, k, v, perm, kv_idx, C, residual=None, scale=None, out=None, out_dtype=torch.bfloat16):
    """mcs_sparse_attn(_f32out): each group of C queries attends to its K gathered keys (+ residual).

    The output is bf16 unless out (or out_dtype) is float32."""
    _qkv(q, k, v)
    B, H, N, D = q.shape
    _like(perm, "perm", torch.int32, (B, H, N), q.device)
    _need(kv_idx, "kv_idx", torch.int32, 4)
    if residual is not None:
        _like(residual, "residual", torch.bfloat16, q.shape, q.device)
    G = num_groups(N, C)
    if tuple(kv_idx.shape[:3]) != (B, H, G):
        raise ValueError(f"kv_idx must be [B, H, G={G}, K] (got {tuple(kv_idx.shape)})")
    if kv_idx.device != q.device:
        raise ValueError(f"kv_idx must be on {q.device} (got {kv_idx.device})")
    K = kv_idx.shape[3]
    scale = default_scale(D) if scale is None else scale
    out = _out(q, out, out_dtype)
    fn = _lib.mcs_sparse_attn_f32out if out.dtype == torch.float32 else _lib.mcs_sparse_attn
    _check(fn(_ptr(q), _ptr(k), _ptr(v), _ptr(perm), _ptr(kv_idx), _ptr(residual), _ptr(out), dims_of(q),
              C, K, scale, _stream(q)))
    return out


def sparse_attn_ex(q, k, v, perm, kv_idx, C, kv_count=None, residual=None, scale=None, want_lse=False,
                   out=None, out_dtype=torch.bfloat16):
    """mcs_sparse_attn_ex: sparse_attn with optional per-group key counts and the
    per-query LSE over the selected keys.  Returns out, or (out, lse)."""
    _qkv(q, k, v)
    B, H, N, D = q.shape
    _like(perm, "perm", torch.int32, (B, H, N), q.device)
    _need(kv_idx, "kv_idx", torch.int32, 4)
    G = num_groups(N, C)
    if tuple(kv_idx.shape[:3]) != (B, H, G) or kv_idx.device != q.device:
        raise ValueError(f"kv_idx must be [B, H, G={G}, K] on {q.device} (got {tuple(kv_idx.shape)})")
    if kv_count is not None:
        _like(kv_count, "kv_count", torch.int32, (B, H, G), q.device)
    if residual is not None:
        _like(residual, "residual", torch.bfloat16, q.shape, q.device)
    K = kv_idx.shape[3]
    scale = default_scale(D) if scale is None else scale
    out = _out(q, out, out_dtype)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if want_lse else None
    _check(_lib.mcs_sparse_attn_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(perm), _ptr(kv_idx), _ptr(kv_count),
                                   _ptr(residual), _ptr(out), int(out.dtype == torch.float32), _ptr(lse),
                                   dims_of(q), C, K, scale, _stream(q)))
    return (out, lse) if want_lse else out


def select_blocks(q, k, perm, C, K, scale=None, workspace=None):
    """mcs_select_blocks: mean-pooled block selection -> (kv_idx [B,H,G,K], kv_count [B,H,G])."""
    _qkv(q, k)
    B, H, N, D = q.shape
    _like(perm, "perm", torch.int32, (B, H, N), q.device)
    G = num_groups(N, C)
    scale = default_scale(D) if scale is None else scale
    kv_idx = torch.empty((B, H, G, K), dtype=torch.int32, device=q.device)
    kv_count = torch.empty((B, H, G), dtype=torch.int32, device=q.device)
    if workspace is None:
        need = int(_lib.mcs_select_blocks_workspace(dims_of(q)))
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check(_lib.mcs_select_blocks(_ptr(q), _ptr(k), _ptr(perm), _ptr(kv_idx), _ptr(kv_count), dims_of(q), C, K,
                                  scale, _ptr(workspace), workspace.numel(), _stream(q)))
    return kv_idx, kv_count


def query_quality(lse_dense, lse_sparse, o_dense, o_sparse):
    """mcs_query_quality: per-query recall, L1 distance and dense L1 norm (float32 [B,H,N] each)."""
    _need(o_dense, "o_dense", torch.float32, 4)
    B, H, N, D = o_dense.shape
    _like(o_sparse, "o_sparse", torch.float32, o_dense.shape, o_dense.device)
    _like(lse_dense, "lse_dense", torch.float32, (B, H, N), o_dense.device)
    _like(lse_sparse, "lse_sparse", torch.float32, (B, H, N), o_dense.device)
    recall, l1, l1_ref = (torch.empty((B, H, N), dtype=torch.float32, device=o_dense.device) for _ in range(3))
    _check(_lib.mcs_query_quality(_ptr(lse_dense), _ptr(lse_sparse), _ptr(o_dense), _ptr(o_sparse), _ptr(recall),
                                  _ptr(l1), _ptr(l1_ref), Dims(B, H, N, D), _stream(o_dense)))
    return recall, l1, l1_ref


def row_sums(x):
    """mcs_row_sums: fp64 sums of the rows of a contiguous float32 [rows, n] tensor."""
    _need(x, "x", torch.float32, 2)
    out = torch.empty(x.shape[0], dtype=torch.float64, device=x.device)
    _check(_lib.mcs_row_sums(_ptr(x), _ptr(out), x.shape[0], x.shape[1], _stream(x)))
    return out


def kmeans(x, init, rounds):
    """mcs_kmeans: Lloyd's k-means of the bf16 rows x [n, D] from the float32
    centres init [k, D] -> (labels [n], centers [k, D], inertia [rounds] fp64, sizes [k])."""
    _need(x, "x", torch.bfloat16, 2)
    n, D = x.shape
    _need(init, "init", torch.float32, 2)
    k = init.shape[0]
    if init.shape[1] != D or init.device != x.device:
        raise ValueError(f"init must be [k, {D}] on {x.device}")
    labels = torch.empty(n, dtype=torch.int32, device=x.device)
    centers = torch.empty((k, D), dtype=torch.float32, device=x.device)
    inertia = torch.empty(rounds, dtype=torch.float64, device=x.device)
    sizes = torch.empty(k, dtype=torch.int32, device=x.device)
    ws = torch.empty(max(int(_lib.mcs_kmeans_workspace(n, k)), 16), dtype=torch.uint8, device=x.device)
    _check(_lib.mcs_kmeans(_ptr(x), _ptr(init), n, D, k, rounds, _ptr(labels), _ptr(centers), _ptr(inertia),
                           _ptr(sizes), _ptr(ws), ws.numel(), _stream(x)))
    return labels, centers, inertia, sizes


def residual_update(o_dense, o_sparse, out=None):
    """mcs_residual_update: bf16(o_dense - o_sparse)."""
    _need(o_dense, "o_dense", torch.bfloat16, o_dense.dim())
    _like(o_sparse, "o_sparse", torch.bfloat16, o_dense.shape, o_dense.device)
    out = torch.empty_like(o_dense) if out is None else out
    _like(out, "out", torch.bfloat16, o_dense.shape, o_dense.device)
    _check(_lib.mcs_residual_update(_ptr(o_dense), _ptr(o_sparse), _ptr(out), o_dense.numel(),
                                    _stream(o_dense)))
    return out


def select_workspace_bytes(q_shape, C, K, all_heads=True) -> int:
    d = Dims(*q_shape)
    fn = _lib.mcs_select_workspace_all_heads if all_heads else _lib.mcs_select_workspace
    return int(fn(d, C, K))


def select(q, k, lse, perm, C, K, scale=None, out=None, workspace=None, max_workspace_bytes=2 << 30):
    """mcs_select: exact per-group top-K KV ids from recovered probabilities."""
    return _select(_lib.mcs_select, q, k, lse, perm, C, K, scale, out, workspace, max_workspace_bytes)


def select_two_pass(q, k, lse, perm, C, K, scale=None, out=None, workspace=None, max_workspace_bytes=2 << 30):
    """mcs_select_two_pass: the same selection as a mass kernel followed by a top-K kernel."""
    return _select(_lib.mcs_select_two_pass, q, k, lse, perm, C, K, scale, out, workspace, max_workspace_bytes)


def _select(fn, q, k, lse, perm, C, K, scale, out, workspace, max_workspace_bytes):
    _qkv(q, k)
    B, H, N, D = q.shape
    _like(lse, "lse", torch.float32, (B, H, N), q.device)
    _like(perm, "perm", torch.int32, (B, H, N), q.device)
    scale = default_scale(D) if scale is None else scale
    G = num_groups(N, C)
    out = torch.empty((B, H, G, K), dtype=torch.int32, device=q.device) if out is None else out
    _like(out, "out", torch.int32, (B, H, G, K), q.device)
    if workspace is not None:
        _like(workspace, "workspace", torch.uint8, (workspace.numel(),), q.device)
    else:
        per_head = select_workspace_bytes(q.shape, C, K, all_heads=False)
        nbytes = min(select_workspace_bytes(q.shape, C, K), max(per_head, max_workspace_bytes // per_head * per_head))
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    _check(fn(_ptr(q), _ptr(k), _ptr(lse), _ptr(perm), _ptr(out), dims_of(q), C, K, scale,
              _ptr(workspace), workspace.numel(), _stream(q)))
    return out


def topk(scores, K, out=None):
    """mcs_topk on float32 [rows, n] non-negative scores -> int32 [rows, K] ascending ids."""
    _need(scores, "scores", torch.float32, 2)
    rows, n = scores.shape
    out = torch.empty((rows, K), dtype=torch.int32, device=scores.device) if out is None else out
    _like(out, "out", torch.int32, (rows, K), scores.device)
    _check(_lib.mcs_topk(_ptr(scores), _ptr(out), rows, n, K, _stream(scores)))
    return out


def group_workspace_bytes(q_shape, C) -> int:
    return int(_lib.mcs_group_workspace(Dims(*q_shape), C))


def group(q, C, lanczos_steps=0, out=None, workspace=None):
    """mcs_group: median-split PDDP -> perm int32 [B, H, N]."""
    _need(q, "q", torch.bfloat16, 4)
    B, H, N, D = q.shape
    out = torch.empty((B, H, N), dtype=torch.int32, device=q.device) if out is None else out
    _like(out, "out", torch.int32, (B, H, N), q.device)
    if workspace is None:
        workspace = torch.empty(max(group_workspace_bytes(q.shape, C), 16), dtype=torch.uint8, device=q.device)
    else:
        _like(workspace, "workspace", torch.uint8, (workspace.numel(),), q.device)
    _check(_lib.mcs_group(_ptr(q), _ptr(out), dims_of(q), C, lanczos_steps, _ptr(workspace),
                          workspace.numel(), _stream(q)))
    return out


def group_noalloc(q, C, lanczos_steps=0, out=None):
    """mcs_group_noalloc: mcs_group with the library's static scratch (no workspace)."""
    _need(q, "q", torch.bfloat16, 4)
    B, H, N, D = q.shape
    out = torch.empty((B, H, N), dtype=torch.int32, device=q.device) if out is None else out
    _like(out, "out", torch.int32, (B, H, N), q.device)
    _check(_lib.mcs_group_noalloc(_ptr(q), _ptr(out), dims_of(q), C, lanczos_steps, _stream(q)))
    return out


def anchor_step(q, k, v, C, K, scale=None, lanczos_steps=0):
    """Anchor step: group, dense + LSE, select, sparse, residual.  Output is the dense output."""
    perm = group(q, C, lanczos_steps)
    o_dense, lse = dense_attn(q, k, v, scale, want_lse=True)
    kv_idx = select(q, k, lse, perm, C, K, scale)
    o_sparse = sparse_attn(q, k, v, perm, kv_idx, C, scale=scale)
    res = residual_update(o_dense, o_sparse)
    return {"out": o_dense, "perm": perm, "lse": lse, "kv_idx": kv_idx, "o_sparse": o_sparse, "residual": res}


def reuse_step(q, k, v, perm, kv_idx, residual, C, scale=None, out=None):
    """Reuse step: sparse attention with the cached groups, ids and residual."""
    return sparse_attn(q, k, v, perm, kv_idx, C, residual=residual, scale=scale, out=out)
