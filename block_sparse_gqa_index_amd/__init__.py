"""Python binding of libmsa.so — the MSA forward path on MI355X (gfx950).

Argument marshalling only: every step runs in the library's HIP kernels.  PyTorch
provides device memory and the current stream.  The functions carry the C names
(``msa_index_topk``, ``msa_sparse_attn_fwd``, ``msa_decode``, ...) and accept torch
tensors; outputs and workspaces are allocated here when not given.

If the library has not been built (``python block_sparse_gqa_index_amd/build.py``
or ``__graft_entry__.build()``) importing the binding fails loudly: there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmsa.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python block_sparse_gqa_index_amd/build.py`")

_lib = ctypes.CDLL(LIB_PATH)

MSA_OK, MSA_ERR_INVALID_ARG, MSA_ERR_UNSUPPORTED, MSA_ERR_WORKSPACE, MSA_ERR_HIP = range(5)

_P, _I64, _I32, _SZ, _F32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t, ctypes.c_float

_SIGS = {
    "msa_status_string": ([_I32], ctypes.c_char_p),
    "msa_last_error": ([], ctypes.c_char_p),
    "msa_index_topk_workspace": ([_I64, _I32, _I32, _I32, _I32], _SZ),
    "msa_index_topk": ([_P, _P, _I64, _I32, _I32, _I32, _I32, _P, _P, _SZ, _P], _I32),
    "msa_sparse_attn_fwd_workspace": ([_I64, _I32, _I32, _I32, _I32, _I32], _SZ),
    "msa_sparse_attn_fwd_workspace_min": ([_I64, _I32, _I32, _I32, _I32, _I32], _SZ),
    "msa_sparse_attn_fwd_windows": ([_I64, _I32, _I32, _I32, _I32, _I32, _SZ], _I64),
    "msa_sparse_attn_fwd": ([_P, _P, _P, _P, _I64, _I32, _I32, _I32, _I32, _I32, _F32, _P, _P, _P, _SZ, _P], _I32),
    "msa_sparse_attn_fwd_lse_idx": ([_P, _P, _P, _P, _P, _P, _I64, _I32, _I32, _I32, _I32, _I32, _I32, _F32, _P, _P,
                                     _P, _P, _SZ, _P], _I32),
    "msa_decode_workspace": ([_I32, _I32, _I32, _I32, _I32, _I32, _I32, _I64], _SZ),
    "msa_decode": ([_P, _P, _P, _P, _P, _P, _I32, _I64, _I64, _I32, _I32, _I32, _I32, _I32, _I32, _F32, _P, _P, _P, _P,
                    _SZ, _P], _I32),
    "msa_decode_noalloc": ([_P, _P, _P, _P, _P, _P, _I32, _I64, _I64, _I32, _I32, _I32, _I32, _I32, _I32, _F32, _P, _P,
                            _P, _P], _I32),
    "msa_index_block_scores": ([_P, _P, _I64, _I32, _I32, _I32, _P, _P], _I32),
    "msa_topk_from_scores": ([_P, _I64, _I32, _I64, _I32, _I32, _P, _P], _I32),
    "msa_set_profile_events": ([ctypes.POINTER(_P), _I32], _I32),
    "msa_set_profile_clock": ([_P, _I64], _I32),
    "msa_sparse_kl_fwd_workspace": ([_I64, _I32, _I32, _I32, _I32, _I32, _I32], _SZ),
    "msa_sparse_kl_fwd_workspace_min": ([_I64, _I32, _I32, _I32, _I32, _I32, _I32], _SZ),
    "msa_sparse_kl_fwd": ([_P, _P, _P, _P, _P, _P, _I64, _I32, _I32, _I32, _I32, _I32, _I32, _F32, _P, _P, _P, _P, _SZ,
                           _P], _I32),
    "msa_sparse_kl_fwd_from_lse_idx": ([_P, _P, _P, _P, _P, _P, _P, _I64, _I32, _I32, _I32, _I32, _I32, _I32, _F32,
                                        _P, _P, _P, _SZ, _P], _I32),
    "msa_sparse_attn_bwd_workspace": ([_I64, _I32, _I32, _I32, _I32, _I32], _SZ),
    "msa_sparse_attn_bwd_workspace_min": ([_I64, _I32, _I32, _I32, _I32, _I32], _SZ),
    "msa_sparse_attn_bwd": ([_P, _P, _P, _P, _P, _P, _P, _I64, _I32, _I32, _I32, _I32, _I32, _F32, _P, _P, _P, _P, _SZ,
                             _P], _I32),
    "msa_decode_paged": ([_P, _P, _P, _P, _F32, _F32, _P, _P, _I64, _I64, _P, _I32, _I64, _I32, _I32, _I32, _I32, _I32, _I32,
                          _F32, _P, _P, _P, _P, _SZ, _P], _I32),
    "msa_index_topk_varlen": ([_P, _P, _P, _I32, _I64, _I64, _I32, _I32, _I32, _I32, _P, _P], _I32),
    "msa_sparse_attn_fwd_varlen_workspace": ([_I64, _I32, _I32, _I32, _I32, _I32, _I32], _SZ),
    "msa_sparse_attn_fwd_varlen_workspace_min": ([_I64, _I32, _I32, _I32, _I32, _I32, _I32], _SZ),
    "msa_sparse_attn_fwd_varlen": ([_P, _P, _P, _P, _P, _I32, _I64, _I32, _I32, _I32, _I32, _I32, _F32, _P, _P, _P,
                                    _SZ, _P], _I32),
}
for _name, (_args, _res) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.argtypes = _args
    _fn.restype = _res

EXPORTED = tuple(_SIGS)


class MSAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib.msa_last_error().decode()
        super().__init__(f"{where}: {_lib.msa_status_string(status).decode()} ({msg})")


def _check(status: int, where: str) -> None:
    if status != MSA_OK:
        raise MSAError(status, where)


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _need(t: torch.Tensor, name: str, dtype, shape) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on the GPU")


def _ws(nbytes: int, device, workspace):
    if workspace is not None:
        return workspace
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


# ----------------------------------------------------------------- Index Branch
def msa_index_topk(q_idx: torch.Tensor, k_idx: torch.Tensor, k: int, B_k: int = 128,
                   block_idx: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Eq. 6-7: chosen blocks [N, H_kv, k] int32 (ascending, -1 padded, local block forced)."""
    N, H_kv, d_idx = q_idx.shape
    _need(q_idx, "q_idx", torch.bfloat16, (N, H_kv, d_idx))
    _need(k_idx, "k_idx", torch.bfloat16, (N, d_idx))
    if block_idx is None:
        block_idx = torch.empty((N, H_kv, k), dtype=torch.int32, device=q_idx.device)
    _need(block_idx, "block_idx", torch.int32, (N, H_kv, k))
    _check(_lib.msa_index_topk(_ptr(q_idx), _ptr(k_idx), N, H_kv, d_idx, B_k, k, _ptr(block_idx), None, 0,
                               _stream(stream)), "msa_index_topk")
    return block_idx


def msa_index_block_scores(q_idx: torch.Tensor, k_idx: torch.Tensor, B_k: int = 128, M: torch.Tensor | None = None,
                           stream=None) -> torch.Tensor:
    """Eq. 6: block scores M [N, H_kv, ceil(N/B_k)] fp32 (-inf where nothing is visible)."""
    N, H_kv, d_idx = q_idx.shape
    _need(q_idx, "q_idx", torch.bfloat16, (N, H_kv, d_idx))
    _need(k_idx, "k_idx", torch.bfloat16, (N, d_idx))
    B = (N + B_k - 1) // B_k
    if M is None:
        M = torch.empty((N, H_kv, B), dtype=torch.float32, device=q_idx.device)
    _need(M, "M", torch.float32, (N, H_kv, B))
    _check(_lib.msa_index_block_scores(_ptr(q_idx), _ptr(k_idx), N, H_kv, d_idx, B_k, _ptr(M), _stream(stream)),
           "msa_index_block_scores")
    return M


def msa_topk_from_scores(M: torch.Tensor, k: int, B_k: int = 128, block_idx: torch.Tensor | None = None,
                         stream=None) -> torch.Tensor:
    """Eq. 7 on given block scores M [N, H_kv, B] fp32."""
    N, H_kv, B = M.shape
    _need(M, "M", torch.float32, (N, H_kv, B))
    if block_idx is None:
        block_idx = torch.empty((N, H_kv, k), dtype=torch.int32, device=M.device)
    _need(block_idx, "block_idx", torch.int32, (N, H_kv, k))
    _check(_lib.msa_topk_from_scores(_ptr(M), N, H_kv, B, B_k, k, _ptr(block_idx), _stream(stream)),
           "msa_topk_from_scores")
    return block_idx


# ----------------------------------------------------------------- Main Branch
def msa_sparse_attn_fwd_workspace(N: int, H_q: int, H_kv: int, k: int, d_h: int = 128, B_k: int = 128,
                                  minimum: bool = False) -> int:
    fn = _lib.msa_sparse_attn_fwd_workspace_min if minimum else _lib.msa_sparse_attn_fwd_workspace
    return int(fn(N, H_q, H_kv, d_h, B_k, k))


def msa_sparse_attn_fwd_windows(N: int, H_q: int, H_kv: int, k: int, ws_bytes: int, d_h: int = 128,
                                B_k: int = 128) -> int:
    """Query windows a msa_sparse_attn_fwd call runs with a workspace of ws_bytes."""
    n = int(_lib.msa_sparse_attn_fwd_windows(N, H_q, H_kv, d_h, B_k, k, ws_bytes))
    if n < 0:
        raise ValueError("unsupported shape or workspace below the minimum")
    return n


def msa_sparse_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, block_idx: torch.Tensor,
                        B_k: int = 128, scale: float | None = None, o: torch.Tensor | None = None,
                        lse: torch.Tensor | None = None, workspace: torch.Tensor | None = None, stream=None):
    """Eq. 8 over the listed blocks.  Returns (o [N,H_q,d_h] fp32, lse [N,H_q] fp32)."""
    N, H_q, d_h = q.shape
    H_kv = k.shape[1]
    kk = block_idx.shape[2]
    _need(q, "q", torch.bfloat16, (N, H_q, d_h))
    _need(k, "k", torch.bfloat16, (N, H_kv, d_h))
    _need(v, "v", torch.bfloat16, (N, H_kv, d_h))
    _need(block_idx, "block_idx", torch.int32, (N, H_kv, kk))
    if scale is None:
        scale = d_h ** -0.5
    if o is None:
        o = torch.empty((N, H_q, d_h), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((N, H_q), dtype=torch.float32, device=q.device)
    _need(o, "o", torch.float32, (N, H_q, d_h))
    _need(lse, "lse", torch.float32, (N, H_q))
    ws = _ws(_lib.msa_sparse_attn_fwd_workspace(N, H_q, H_kv, d_h, B_k, kk), q.device, workspace)
    _check(_lib.msa_sparse_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(block_idx), N, H_q, H_kv, d_h, B_k, kk,
                                    float(scale), _ptr(o), _ptr(lse), _ptr(ws), ws.numel() * ws.element_size(),
                                    _stream(stream)), "msa_sparse_attn_fwd")
    return o, lse


def msa_sparse_attn_fwd_lse_idx(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, q_idx: torch.Tensor,
                                k_idx: torch.Tensor, block_idx: torch.Tensor, B_k: int = 128,
                                scale: float | None = None, o: torch.Tensor | None = None,
                                lse: torch.Tensor | None = None, lse_idx: torch.Tensor | None = None,
                                workspace: torch.Tensor | None = None, stream=None):
    """msa_sparse_attn_fwd that also emits LSE_idx [N, H_kv] (the index distribution's
    log partition over each row's selected tokens).  Returns (o, lse, lse_idx)."""
    N, H_q, d_h = q.shape
    H_kv = k.shape[1]
    kk = block_idx.shape[2]
    d_idx = q_idx.shape[2]
    _need(q, "q", torch.bfloat16, (N, H_q, d_h))
    _need(k, "k", torch.bfloat16, (N, H_kv, d_h))
    _need(v, "v", torch.bfloat16, (N, H_kv, d_h))
    _need(q_idx, "q_idx", torch.bfloat16, (N, H_kv, d_idx))
    _need(k_idx, "k_idx", torch.bfloat16, (N, d_idx))
    _need(block_idx, "block_idx", torch.int32, (N, H_kv, kk))
    if scale is None:
        scale = d_h ** -0.5
    if o is None:
        o = torch.empty((N, H_q, d_h), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((N, H_q), dtype=torch.float32, device=q.device)
    if lse_idx is None:
        lse_idx = torch.empty((N, H_kv), dtype=torch.float32, device=q.device)
    _need(o, "o", torch.float32, (N, H_q, d_h))
    _need(lse, "lse", torch.float32, (N, H_q))
    _need(lse_idx, "lse_idx", torch.float32, (N, H_kv))
    ws = _ws(_lib.msa_sparse_attn_fwd_workspace(N, H_q, H_kv, d_h, B_k, kk), q.device, workspace)
    _check(_lib.msa_sparse_attn_fwd_lse_idx(_ptr(q), _ptr(k), _ptr(v), _ptr(q_idx), _ptr(k_idx), _ptr(block_idx), N,
                                            H_q, H_kv, d_h, d_idx, B_k, kk, float(scale), _ptr(o), _ptr(lse),
                                            _ptr(lse_idx), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "msa_sparse_attn_fwd_lse_idx")
    return o, lse, lse_idx


# ----------------------------------------------------------------- Backward
def msa_sparse_attn_bwd_workspace(N: int, H_q: int, H_kv: int, k: int, d_h: int = 128, B_k: int = 128,
                                  minimum: bool = False) -> int:
    fn = _lib.msa_sparse_attn_bwd_workspace_min if minimum else _lib.msa_sparse_attn_bwd_workspace
    return int(fn(N, H_q, H_kv, d_h, B_k, k))


def msa_sparse_attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, lse: torch.Tensor,
                        dO: torch.Tensor, block_idx: torch.Tensor, B_k: int = 128, scale: float | None = None,
                        dq=None, dk=None, dv=None, workspace=None, stream=None):
    """Gradients of Eq. 8 (selection fixed).  Returns (dq [N,H_q,d_h], dk, dv [N,H_kv,d_h]) fp32."""
    N, H_q, d_h = q.shape
    H_kv = k.shape[1]
    kk = block_idx.shape[2]
    _need(q, "q", torch.bfloat16, (N, H_q, d_h))
    _need(k, "k", torch.bfloat16, (N, H_kv, d_h))
    _need(v, "v", torch.bfloat16, (N, H_kv, d_h))
    _need(o, "o", torch.float32, (N, H_q, d_h))
    _need(lse, "lse", torch.float32, (N, H_q))
    _need(dO, "dO", torch.bfloat16, (N, H_q, d_h))
    _need(block_idx, "block_idx", torch.int32, (N, H_kv, kk))
    if scale is None:
        scale = d_h ** -0.5
    dev = q.device
    if dq is None:
        dq = torch.empty((N, H_q, d_h), dtype=torch.float32, device=dev)
    if dk is None:
        dk = torch.empty((N, H_kv, d_h), dtype=torch.float32, device=dev)
    if dv is None:
        dv = torch.empty((N, H_kv, d_h), dtype=torch.float32, device=dev)
    _need(dq, "dq", torch.float32, (N, H_q, d_h))
    _need(dk, "dk", torch.float32, (N, H_kv, d_h))
    _need(dv, "dv", torch.float32, (N, H_kv, d_h))
    ws = _ws(_lib.msa_sparse_attn_bwd_workspace(N, H_q, H_kv, d_h, B_k, kk), dev, workspace)
    _check(_lib.msa_sparse_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dO), _ptr(block_idx), N, H_q,
                                    H_kv, d_h, B_k, kk, float(scale), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws),
                                    ws.numel() * ws.element_size(), _stream(stream)), "msa_sparse_attn_bwd")
    return dq, dk, dv


# ----------------------------------------------------------------- KL alignment
def msa_sparse_kl_fwd_workspace(N: int, H_q: int, H_kv: int, k: int, d_h: int = 128, d_idx: int = 64,
                                B_k: int = 128, minimum: bool = False) -> int:
    fn = _lib.msa_sparse_kl_fwd_workspace_min if minimum else _lib.msa_sparse_kl_fwd_workspace
    return int(fn(N, H_q, H_kv, d_h, d_idx, B_k, k))


def msa_sparse_kl_fwd(q: torch.Tensor, k: torch.Tensor, q_idx: torch.Tensor, k_idx: torch.Tensor,
                      block_idx: torch.Tensor, lse: torch.Tensor, B_k: int = 128, scale: float | None = None,
                      kl: torch.Tensor | None = None, lse_idx: torch.Tensor | None = None,
                      loss: torch.Tensor | None = None, workspace: torch.Tensor | None = None, stream=None):
    """Eq. 9-10 on the selected tokens.  Returns (kl [N,H_kv], lse_idx [N,H_kv], loss [1]) fp32."""
    N, H_q, d_h = q.shape
    H_kv, d_idx = q_idx.shape[1], q_idx.shape[2]
    kk = block_idx.shape[2]
    _need(q, "q", torch.bfloat16, (N, H_q, d_h))
    _need(k, "k", torch.bfloat16, (N, H_kv, d_h))
    _need(q_idx, "q_idx", torch.bfloat16, (N, H_kv, d_idx))
    _need(k_idx, "k_idx", torch.bfloat16, (N, d_idx))
    _need(block_idx, "block_idx", torch.int32, (N, H_kv, kk))
    _need(lse, "lse", torch.float32, (N, H_q))
    if scale is None:
        scale = d_h ** -0.5
    dev = q.device
    if kl is None:
        kl = torch.empty((N, H_kv), dtype=torch.float32, device=dev)
    if lse_idx is None:
        lse_idx = torch.empty((N, H_kv), dtype=torch.float32, device=dev)
    if loss is None:
        loss = torch.empty((1,), dtype=torch.float32, device=dev)
    _need(kl, "kl", torch.float32, (N, H_kv))
    _need(lse_idx, "lse_idx", torch.float32, (N, H_kv))
    _need(loss, "loss", torch.float32, (1,))
    ws = _ws(_lib.msa_sparse_kl_fwd_workspace(N, H_q, H_kv, d_h, d_idx, B_k, kk), dev, workspace)
    _check(_lib.msa_sparse_kl_fwd(_ptr(q), _ptr(k), _ptr(q_idx), _ptr(k_idx), _ptr(block_idx), _ptr(lse), N, H_q,
                                  H_kv, d_h, d_idx, B_k, kk, float(scale), _ptr(kl), _ptr(lse_idx), _ptr(loss),
                                  _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)), "msa_sparse_kl_fwd")
    return kl, lse_idx, loss


def msa_sparse_kl_fwd_from_lse_idx(q: torch.Tensor, k: torch.Tensor, q_idx: torch.Tensor, k_idx: torch.Tensor,
                                   block_idx: torch.Tensor, lse: torch.Tensor, lse_idx: torch.Tensor, B_k: int = 128,
                                   scale: float | None = None, kl: torch.Tensor | None = None,
                                   loss: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                                   stream=None):
    """Eq. 9-10 with LSE_idx given (as msa_sparse_attn_fwd_lse_idx emits it).
    Returns (kl [N,H_kv], loss [1]) fp32."""
    N, H_q, d_h = q.shape
    H_kv, d_idx = q_idx.shape[1], q_idx.shape[2]
    kk = block_idx.shape[2]
    _need(q, "q", torch.bfloat16, (N, H_q, d_h))
    _need(k, "k", torch.bfloat16, (N, H_kv, d_h))
    _need(q_idx, "q_idx", torch.bfloat16, (N, H_kv, d_idx))
    _need(k_idx, "k_idx", torch.bfloat16, (N, d_idx))
    _need(block_idx, "block_idx", torch.int32, (N, H_kv, kk))
    _need(lse, "lse", torch.float32, (N, H_q))
    _need(lse_idx, "lse_idx", torch.float32, (N, H_kv))
    if scale is None:
        scale = d_h ** -0.5
    dev = q.device
    if kl is None:
        kl = torch.empty((N, H_kv), dtype=torch.float32, device=dev)
    if loss is None:
        loss = torch.empty((1,), dtype=torch.float32, device=dev)
    _need(kl, "kl", torch.float32, (N, H_kv))
    _need(loss, "loss", torch.float32, (1,))
    ws = _ws(_lib.msa_sparse_kl_fwd_workspace(N, H_q, H_kv, d_h, d_idx, B_k, kk), dev, workspace)
    _check(_lib.msa_sparse_kl_fwd_from_lse_idx(_ptr(q), _ptr(k), _ptr(q_idx), _ptr(k_idx), _ptr(block_idx), _ptr(lse),
                                               _ptr(lse_idx), N, H_q, H_kv, d_h, d_idx, B_k, kk, float(scale),
                                               _ptr(kl), _ptr(loss), _ptr(ws), ws.numel() * ws.element_size(),
                                               _stream(stream)), "msa_sparse_kl_fwd_from_lse_idx")
    return kl, loss


# ----------------------------------------------------------------- Packed sequences
def msa_index_topk_varlen(q_idx: torch.Tensor, k_idx: torch.Tensor, cu_seqlens: torch.Tensor, max_len: int, k: int,
                          B_k: int = 128, block_idx: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Eq. 6-7 per packed sequence: block_idx [T, H_kv, k] int32, block numbers within each row's sequence."""
    T, H_kv, d_idx = q_idx.shape
    batch = cu_seqlens.shape[0] - 1
    _need(q_idx, "q_idx", torch.bfloat16, (T, H_kv, d_idx))
    _need(k_idx, "k_idx", torch.bfloat16, (T, d_idx))
    _need(cu_seqlens, "cu_seqlens", torch.int64, (batch + 1,))
    if block_idx is None:
        block_idx = torch.empty((T, H_kv, k), dtype=torch.int32, device=q_idx.device)
    _need(block_idx, "block_idx", torch.int32, (T, H_kv, k))
    _check(_lib.msa_index_topk_varlen(_ptr(q_idx), _ptr(k_idx), _ptr(cu_seqlens), batch, T, max_len, H_kv, d_idx,
                                      B_k, k, _ptr(block_idx), _stream(stream)), "msa_index_topk_varlen")
    return block_idx


def msa_sparse_attn_fwd_varlen_workspace(T: int, batch: int, H_q: int, H_kv: int, k: int, d_h: int = 128,
                                         B_k: int = 128, minimum: bool = False) -> int:
    fn = _lib.msa_sparse_attn_fwd_varlen_workspace_min if minimum else _lib.msa_sparse_attn_fwd_varlen_workspace
    return int(fn(T, batch, H_q, H_kv, d_h, B_k, k))


def msa_sparse_attn_fwd_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, block_idx: torch.Tensor,
                               cu_seqlens: torch.Tensor, B_k: int = 128, scale: float | None = None,
                               o: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                               workspace: torch.Tensor | None = None, stream=None):
    """Eq. 8 per packed sequence.  Returns (o [T,H_q,d_h] fp32, lse [T,H_q] fp32)."""
    T, H_q, d_h = q.shape
    H_kv = k.shape[1]
    kk = block_idx.shape[2]
    batch = cu_seqlens.shape[0] - 1
    _need(q, "q", torch.bfloat16, (T, H_q, d_h))
    _need(k, "k", torch.bfloat16, (T, H_kv, d_h))
    _need(v, "v", torch.bfloat16, (T, H_kv, d_h))
    _need(block_idx, "block_idx", torch.int32, (T, H_kv, kk))
    _need(cu_seqlens, "cu_seqlens", torch.int64, (batch + 1,))
    if scale is None:
        scale = d_h ** -0.5
    if o is None:
        o = torch.empty((T, H_q, d_h), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((T, H_q), dtype=torch.float32, device=q.device)
    _need(o, "o", torch.float32, (T, H_q, d_h))
    _need(lse, "lse", torch.float32, (T, H_q))
    ws = _ws(_lib.msa_sparse_attn_fwd_varlen_workspace(T, batch, H_q, H_kv, d_h, B_k, kk), q.device, workspace)
    _check(_lib.msa_sparse_attn_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(block_idx), _ptr(cu_seqlens), batch, T,
                                           H_q, H_kv, d_h, B_k, kk, float(scale), _ptr(o), _ptr(lse), _ptr(ws),
                                           ws.numel() * ws.element_size(), _stream(stream)),
           "msa_sparse_attn_fwd_varlen")
    return o, lse


# ----------------------------------------------------------------- Decode
def msa_decode_workspace(batch: int, H_q: int, H_kv: int, k: int, max_len: int, d_h: int = 128, d_idx: int = 64,
                         B_k: int = 128) -> int:
    return int(_lib.msa_decode_workspace(batch, H_q, H_kv, d_h, d_idx, B_k, k, max_len))


def msa_decode(q: torch.Tensor, q_idx: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
               k_idx_cache: torch.Tensor, cu_seqlens: torch.Tensor, max_len: int, k: int, B_k: int = 128,
               scale: float | None = None, block_idx=None, o=None, lse=None, workspace=None, stream=None):
    """One new token per sequence (already the last cache entry).  Returns (block_idx, o, lse)."""
    batch, H_q, d_h = q.shape
    H_kv, d_idx = q_idx.shape[1], q_idx.shape[2]
    T = k_cache.shape[0]
    _need(q, "q", torch.bfloat16, (batch, H_q, d_h))
    _need(q_idx, "q_idx", torch.bfloat16, (batch, H_kv, d_idx))
    _need(k_cache, "k_cache", torch.bfloat16, (T, H_kv, d_h))
    _need(v_cache, "v_cache", torch.bfloat16, (T, H_kv, d_h))
    _need(k_idx_cache, "k_idx_cache", torch.bfloat16, (T, d_idx))
    _need(cu_seqlens, "cu_seqlens", torch.int64, (batch + 1,))
    if scale is None:
        scale = d_h ** -0.5
    dev = q.device
    if block_idx is None:
        block_idx = torch.empty((batch, H_kv, k), dtype=torch.int32, device=dev)
    if o is None:
        o = torch.empty((batch, H_q, d_h), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((batch, H_q), dtype=torch.float32, device=dev)
    _need(block_idx, "block_idx", torch.int32, (batch, H_kv, k))
    _need(o, "o", torch.float32, (batch, H_q, d_h))
    _need(lse, "lse", torch.float32, (batch, H_q))
    ws = _ws(_lib.msa_decode_workspace(batch, H_q, H_kv, d_h, d_idx, B_k, k, max_len), dev, workspace)
    _check(_lib.msa_decode(_ptr(q), _ptr(q_idx), _ptr(k_cache), _ptr(v_cache), _ptr(k_idx_cache), _ptr(cu_seqlens),
                           batch, T, max_len, H_q, H_kv, d_h, d_idx, B_k, k, float(scale), _ptr(block_idx), _ptr(o),
                           _ptr(lse), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)), "msa_decode")
    return block_idx, o, lse


def msa_decode_noalloc(q: torch.Tensor, q_idx: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                       k_idx_cache: torch.Tensor, cu_seqlens: torch.Tensor, max_len: int, k: int, B_k: int = 128,
                       scale: float | None = None, block_idx=None, o=None, lse=None, stream=None):
    """msa_decode with the library's static scratch as its workspace (the C call
    allocates nothing; pass block_idx, o and lse to allocate nothing here either)."""
    batch, H_q, d_h = q.shape
    H_kv, d_idx = q_idx.shape[1], q_idx.shape[2]
    T = k_cache.shape[0]
    _need(q, "q", torch.bfloat16, (batch, H_q, d_h))
    _need(q_idx, "q_idx", torch.bfloat16, (batch, H_kv, d_idx))
    _need(k_cache, "k_cache", torch.bfloat16, (T, H_kv, d_h))
    _need(v_cache, "v_cache", torch.bfloat16, (T, H_kv, d_h))
    _need(k_idx_cache, "k_idx_cache", torch.bfloat16, (T, d_idx))
    _need(cu_seqlens, "cu_seqlens", torch.int64, (batch + 1,))
    if scale is None:
        scale = d_h ** -0.5
    dev = q.device
    if block_idx is None:
        block_idx = torch.empty((batch, H_kv, k), dtype=torch.int32, device=dev)
    if o is None:
        o = torch.empty((batch, H_q, d_h), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((batch, H_q), dtype=torch.float32, device=dev)
    _need(block_idx, "block_idx", torch.int32, (batch, H_kv, k))
    _need(o, "o", torch.float32, (batch, H_q, d_h))
    _need(lse, "lse", torch.float32, (batch, H_q))
    _check(_lib.msa_decode_noalloc(_ptr(q), _ptr(q_idx), _ptr(k_cache), _ptr(v_cache), _ptr(k_idx_cache),
                                   _ptr(cu_seqlens), batch, T, max_len, H_q, H_kv, d_h, d_idx, B_k, k, float(scale),
                                   _ptr(block_idx), _ptr(o), _ptr(lse), _stream(stream)), "msa_decode_noalloc")
    return block_idx, o, lse


def msa_decode_paged(q: torch.Tensor, q_idx: torch.Tensor, k_pages: torch.Tensor, v_pages: torch.Tensor,
                     k_scale: float, v_scale: float, k_idx_pages: torch.Tensor, block_table: torch.Tensor,
                     seqlens: torch.Tensor, max_len: int, k: int, B_k: int = 128, scale: float | None = None,
                     block_idx=None, o=None, lse=None, workspace=None, stream=None):
    """Decode over paged FP8 E4M3 K/V pages (uint8 codes) and bf16 index-key pages.
    Returns (block_idx, o, lse)."""
    batch, H_q, d_h = q.shape
    H_kv, d_idx = q_idx.shape[1], q_idx.shape[2]
    P = k_pages.shape[0]
    _need(q, "q", torch.bfloat16, (batch, H_q, d_h))
    _need(q_idx, "q_idx", torch.bfloat16, (batch, H_kv, d_idx))
    _need(k_pages, "k_pages", torch.uint8, (P, B_k, H_kv, d_h))
    _need(v_pages, "v_pages", torch.uint8, (P, B_k, H_kv, d_h))
    _need(k_idx_pages, "k_idx_pages", torch.bfloat16, (P, B_k, d_idx))
    _need(block_table, "block_table", torch.int32, (batch, block_table.shape[1]))
    _need(seqlens, "seqlens", torch.int64, (batch,))
    if scale is None:
        scale = d_h ** -0.5
    dev = q.device
    if block_idx is None:
        block_idx = torch.empty((batch, H_kv, k), dtype=torch.int32, device=dev)
    if o is None:
        o = torch.empty((batch, H_q, d_h), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((batch, H_q), dtype=torch.float32, device=dev)
    _need(block_idx, "block_idx", torch.int32, (batch, H_kv, k))
    _need(o, "o", torch.float32, (batch, H_q, d_h))
    _need(lse, "lse", torch.float32, (batch, H_q))
    ws = _ws(_lib.msa_decode_workspace(batch, H_q, H_kv, d_h, d_idx, B_k, k, max_len), dev, workspace)
    _check(_lib.msa_decode_paged(_ptr(q), _ptr(q_idx), _ptr(k_pages), _ptr(v_pages), float(k_scale), float(v_scale),
                                 _ptr(k_idx_pages), _ptr(block_table), block_table.shape[1], P, _ptr(seqlens), batch,
                                 max_len, H_q, H_kv, d_h, d_idx, B_k, k, float(scale), _ptr(block_idx), _ptr(o),
                                 _ptr(lse), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "msa_decode_paged")
    return block_idx, o, lse


def msa_set_profile_events(events=None) -> None:
    """Record caller-owned events at the phase boundaries of later msa_sparse_attn_fwd
    calls on this thread: 4 per query window (inverse index, KV-outer phase 1,
    combine, end), for the first len(events) // 4 windows; None clears.

    Takes torch.cuda.Event objects created with enable_timing=True.  An event whose
    handle does not exist yet is recorded once here on the current stream."""
    if events is None:
        _check(_lib.msa_set_profile_events(None, 0), "msa_set_profile_events")
        return
    if len(events) == 0 or len(events) % 4 != 0:
        raise ValueError("msa_set_profile_events takes 4 events per query window")
    for e in events:
        if not e.cuda_event:
            e.record()
    arr = (_P * len(events))(*[e.cuda_event for e in events])
    _check(_lib.msa_set_profile_events(arr, len(events)), "msa_set_profile_events")


def msa_set_profile_clock(clock: torch.Tensor | None = None) -> None:
    """Per-workgroup start / end clocks (100 MHz) of the persistent-grid kernels of
    later calls on this thread (phase 1 of msa_sparse_attn_fwd, the backward's main
    kernel; first query window only) into ``clock`` (int64 on the device, two per
    workgroup); None clears."""
    if clock is None:
        _check(_lib.msa_set_profile_clock(None, 0), "msa_set_profile_clock")
        return
    _need(clock, "clock", torch.int64, (clock.numel(),))
    _check(_lib.msa_set_profile_clock(_ptr(clock), clock.numel()), "msa_set_profile_clock")


def raw():
    """The ctypes handle (for tests of the C ABI itself)."""
    return _lib
