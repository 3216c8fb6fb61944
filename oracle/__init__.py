"""Python wrappers of the CPU oracle (``msa_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the test suite, ``__graft_entry__.smoke``
and the CPU-baseline leg of ``bench.py``; never by the library.  The oracle
follows the pages' definitions (MiniMax Sparse Attention paper review,
section 3, Eq. 4/6/7/8; reading notes section 5.1.1) in fp64 over the same
bf16 bytes the GPU consumes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "msa_oracle.c")
_LIB = os.path.join(_HERE, "libmsa_oracle.so")
_lib = None


def use_library(path: str | None) -> None:
    """Point the wrappers at another build of the oracle (mutation tests); None restores the default."""
    global _lib, _LIB_OVERRIDE
    _LIB_OVERRIDE = path
    _lib = None


_LIB_OVERRIDE = None


def build() -> str:
    """Compile the oracle with gcc (strict IEEE: no fast-math) into oracle/libmsa_oracle.so."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra",
           "-o", _LIB + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if _LIB_OVERRIDE is not None:
        lib = ctypes.CDLL(_LIB_OVERRIDE)
    else:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    i64, i32, dbl = ctypes.c_int64, ctypes.c_int, ctypes.c_double
    lib.msa_oracle_num_blocks.argtypes = [i64, i32]
    lib.msa_oracle_num_blocks.restype = i64
    lib.msa_oracle_threads.argtypes = []
    lib.msa_oracle_threads.restype = i32
    lib.msa_oracle_block_scores.argtypes = [P, P, i64, i32, i32, i32, P, i64, P]
    lib.msa_oracle_topk.argtypes = [P, P, i64, i32, i64, i32, i32, P]
    lib.msa_oracle_sparse_attn.argtypes = [P, P, P, P, i64, i32, i32, i32, i32, i32, dbl, P, i64, P, P]
    lib.msa_oracle_decode.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, i32, i32, i32, dbl,
                                      P, P, P, P, i64]
    lib.msa_oracle_decode_attn.argtypes = [P, P, P, P, i32, i32, i32, i32, i32, i32, dbl, P, P, P]
    lib.msa_oracle_sparse_kl.argtypes = [P, P, P, P, P, i64, i32, i32, i32, i32, i32, i32, dbl, P, i64, P, P]
    lib.msa_oracle_sparse_attn_bwd.argtypes = [P, P, P, P, P, i64, i32, i32, i32, i32, i32, dbl, P, P, P]
    lib.msa_oracle_sparse_attn_bwd_part.argtypes = [P, P, P, P, P, i64, i32, i32, i32, i32, i32, dbl, P, i64, P,
                                                    i64, i32, P, P]
    lib.msa_oracle_fp8_e4m3.argtypes = [ctypes.c_uint8]
    lib.msa_oracle_fp8_e4m3.restype = dbl
    lib.msa_oracle_decode_paged.argtypes = [P, P, P, P, dbl, dbl, P, P, i64, P, i32, i32, i32, i32, i32, i32, i32,
                                            dbl, P, P, P, P, P, i64]
    _lib = lib
    return lib


def _u16(x) -> np.ndarray:
    """bf16 tensor (torch) or uint16 array -> contiguous uint16 numpy array of the same bytes."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach()
            if x.device.type != "cpu":
                x = x.cpu()
            if x.dtype == torch.bfloat16:
                x = x.contiguous().view(torch.int16).numpy().view(np.uint16)
            else:
                x = x.contiguous().numpy()
    except ImportError:
        pass
    x = np.ascontiguousarray(x)
    if x.dtype != np.uint16:
        raise TypeError(f"expected bf16 bits as uint16, got {x.dtype}")
    return x


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _rows(rows, N):
    if rows is None:
        return None, N
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    if r.size and (r.min() < 0 or r.max() >= N):
        raise ValueError("row out of range")
    return r, r.size


def threads() -> int:
    return int(_load().msa_oracle_threads())


def num_blocks(N: int, B_k: int) -> int:
    return int(_load().msa_oracle_num_blocks(N, B_k))


def block_scores(q_idx, k_idx, B_k: int, rows=None) -> np.ndarray:
    """Eq. 6: M[n, r, b] (float64, -inf where block b has no visible token)."""
    qi, ki = _u16(q_idx), _u16(k_idx)
    N, H_kv, d_idx = qi.shape
    assert ki.shape == (N, d_idx)
    r, nrows = _rows(rows, N)
    B = num_blocks(N, B_k)
    M = np.empty((nrows, H_kv, B), dtype=np.float64)
    _load().msa_oracle_block_scores(_ptr(qi), _ptr(ki), N, H_kv, d_idx, B_k,
                                    None if r is None else _ptr(r), nrows, _ptr(M))
    return M


def topk(M, k: int, B_k: int, rows=None, N=None) -> np.ndarray:
    """Eq. 7 with the forced local block; M is [nrows, H_kv, B]; rows are positions."""
    Md = np.ascontiguousarray(M, dtype=np.float64)
    nrows, H_kv, B = Md.shape
    if rows is None:
        r = None
    else:
        r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        assert r.size == nrows
    out = np.empty((nrows, H_kv, k), dtype=np.int32)
    _load().msa_oracle_topk(_ptr(Md), None if r is None else _ptr(r), nrows, H_kv, B, B_k, k, _ptr(out))
    return out


def sparse_attn(q, k, v, block_idx, B_k: int, scale: float | None = None, rows=None):
    """Eq. 8 over the chosen blocks (causal); returns (o [nrows,H_q,d_h], lse [nrows,H_q]) float64."""
    qq, kk_, vv = _u16(q), _u16(k), _u16(v)
    N, H_q, d_h = qq.shape
    H_kv = kk_.shape[1]
    assert kk_.shape == (N, H_kv, d_h) and vv.shape == (N, H_kv, d_h)
    r, nrows = _rows(rows, N)
    bi = np.ascontiguousarray(np.asarray(block_idx), dtype=np.int32)
    assert bi.shape[0] == nrows and bi.shape[1] == H_kv
    kk = bi.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(d_h)
    o = np.empty((nrows, H_q, d_h), dtype=np.float64)
    lse = np.empty((nrows, H_q), dtype=np.float64)
    _load().msa_oracle_sparse_attn(_ptr(qq), _ptr(kk_), _ptr(vv), _ptr(bi), N, H_q, H_kv, d_h, B_k, kk,
                                   float(scale), None if r is None else _ptr(r), nrows, _ptr(o), _ptr(lse))
    return o, lse


def sparse_kl(q, k, q_idx, k_idx, block_idx, B_k: int, scale: float | None = None, rows=None):
    """Eq. 9-10 per (query, group) on the selected token set: returns (kl [nrows, H_kv],
    lse_idx [nrows, H_kv]) float64; the loss of Eq. 10 is kl.mean() over all rows."""
    qq, kk_, qi, ki = _u16(q), _u16(k), _u16(q_idx), _u16(k_idx)
    N, H_q, d_h = qq.shape
    H_kv, d_idx = qi.shape[1], qi.shape[2]
    assert kk_.shape == (N, H_kv, d_h) and ki.shape == (N, d_idx)
    r, nrows = _rows(rows, N)
    bi = np.ascontiguousarray(np.asarray(block_idx), dtype=np.int32)
    assert bi.shape[0] == nrows and bi.shape[1] == H_kv
    if scale is None:
        scale = 1.0 / np.sqrt(d_h)
    kl = np.empty((nrows, H_kv), dtype=np.float64)
    lse_idx = np.empty((nrows, H_kv), dtype=np.float64)
    _load().msa_oracle_sparse_kl(_ptr(qq), _ptr(kk_), _ptr(qi), _ptr(ki), _ptr(bi), N, H_q, H_kv, d_h, d_idx,
                                 B_k, bi.shape[2], float(scale), None if r is None else _ptr(r), nrows,
                                 _ptr(kl), _ptr(lse_idx))
    return kl, lse_idx


def sparse_attn_bwd(q, k, v, dO, block_idx, B_k: int, scale: float | None = None):
    """Gradients of Eq. 8 for upstream dO (selection fixed): returns (dq, dk, dv) float64."""
    qq, kk_, vv, gg = _u16(q), _u16(k), _u16(v), _u16(dO)
    N, H_q, d_h = qq.shape
    H_kv = kk_.shape[1]
    assert gg.shape == qq.shape and vv.shape == kk_.shape
    bi = np.ascontiguousarray(np.asarray(block_idx), dtype=np.int32)
    assert bi.shape[:2] == (N, H_kv)
    if scale is None:
        scale = 1.0 / np.sqrt(d_h)
    dq = np.empty((N, H_q, d_h), dtype=np.float64)
    dk = np.empty((N, H_kv, d_h), dtype=np.float64)
    dv = np.empty((N, H_kv, d_h), dtype=np.float64)
    _load().msa_oracle_sparse_attn_bwd(_ptr(qq), _ptr(kk_), _ptr(vv), _ptr(gg), _ptr(bi), N, H_q, H_kv, d_h, B_k,
                                       bi.shape[2], float(scale), _ptr(dq), _ptr(dk), _ptr(dv))
    return dq, dk, dv


def sparse_attn_bwd_part(q, k, v, dO, block_idx, B_k: int, rows=(), key_block: int = -1, group: int = 0,
                         scale: float | None = None):
    """The gradients of Eq. 8 restricted: dq [len(rows), H_q, d_h] of the listed query
    rows, and dk, dv [B_k, d_h] of key block `key_block` of KV head `group` (None when
    key_block < 0).  float64."""
    qq, kk_, vv, gg = _u16(q), _u16(k), _u16(v), _u16(dO)
    N, H_q, d_h = qq.shape
    H_kv = kk_.shape[1]
    assert gg.shape == qq.shape and vv.shape == kk_.shape
    bi = np.ascontiguousarray(np.asarray(block_idx), dtype=np.int32)
    assert bi.shape[:2] == (N, H_kv)
    if scale is None:
        scale = 1.0 / np.sqrt(d_h)
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    assert r.size == 0 or (r.min() >= 0 and r.max() < N)
    dq = np.empty((max(1, r.size), H_q, d_h), dtype=np.float64)
    dk = np.empty((B_k, d_h), dtype=np.float64)
    dv = np.empty((B_k, d_h), dtype=np.float64)
    _load().msa_oracle_sparse_attn_bwd_part(_ptr(qq), _ptr(kk_), _ptr(vv), _ptr(gg), _ptr(bi), N, H_q, H_kv, d_h,
                                            B_k, bi.shape[2], float(scale), _ptr(r), r.size, _ptr(dq),
                                            int(key_block), int(group), _ptr(dk), _ptr(dv))
    return dq[:r.size], (dk, dv) if key_block >= 0 else None


def decode(q, q_idx, k_cache, v_cache, k_idx_cache, cu_seqlens, k: int, B_k: int,
           scale: float | None = None, want_scores: bool = False):
    """One new token per sequence (the last cache entry).  Returns block_idx, o, lse[, M]."""
    qq, qi = _u16(q), _u16(q_idx)
    kc, vc, kic = _u16(k_cache), _u16(v_cache), _u16(k_idx_cache)
    try:
        import torch
        if isinstance(cu_seqlens, torch.Tensor):
            cu_seqlens = cu_seqlens.cpu().numpy()
    except ImportError:
        pass
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    batch, H_q, d_h = qq.shape
    H_kv, d_idx = qi.shape[1], qi.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(d_h)
    lens = np.diff(cu)
    Bmax = int((lens.max() + B_k - 1) // B_k) if batch else 0
    bi = np.empty((batch, H_kv, k), dtype=np.int32)
    o = np.empty((batch, H_q, d_h), dtype=np.float64)
    lse = np.empty((batch, H_q), dtype=np.float64)
    M = np.empty((batch, H_kv, Bmax), dtype=np.float64) if want_scores else None
    _load().msa_oracle_decode(_ptr(qq), _ptr(qi), _ptr(kc), _ptr(vc), _ptr(kic), _ptr(cu), batch, H_q, H_kv,
                              d_h, d_idx, B_k, k, float(scale), _ptr(bi), _ptr(o), _ptr(lse),
                              None if M is None else _ptr(M), Bmax)
    if want_scores:
        return bi, o, lse, M
    return bi, o, lse


def decode_attn(q, k_cache, v_cache, cu_seqlens, block_idx, B_k: int, scale: float | None = None):
    """Attention of each sequence's last token on a given selection block_idx [batch, H_kv, kk]."""
    qq, kc, vc = _u16(q), _u16(k_cache), _u16(v_cache)
    try:
        import torch
        if isinstance(cu_seqlens, torch.Tensor):
            cu_seqlens = cu_seqlens.cpu().numpy()
    except ImportError:
        pass
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    batch, H_q, d_h = qq.shape
    H_kv = kc.shape[1]
    bi = np.ascontiguousarray(np.asarray(block_idx), dtype=np.int32)
    kk = bi.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(d_h)
    o = np.empty((batch, H_q, d_h), dtype=np.float64)
    lse = np.empty((batch, H_q), dtype=np.float64)
    _load().msa_oracle_decode_attn(_ptr(qq), _ptr(kc), _ptr(vc), _ptr(cu), batch, H_q, H_kv, d_h, B_k, kk,
                                   float(scale), _ptr(bi), _ptr(o), _ptr(lse))
    return o, lse


def _cu(cu_seqlens) -> np.ndarray:
    try:
        import torch
        if isinstance(cu_seqlens, torch.Tensor):
            cu_seqlens = cu_seqlens.cpu().numpy()
    except ImportError:
        pass
    return np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))


def index_topk_varlen(q_idx, k_idx, cu_seqlens, k: int, B_k: int, want_scores: bool = False):
    """Packed sequences, each its own instance of Eq. 6-7 (positions count from the
    sequence start).  Returns block_idx [T, H_kv, k] with sequence-local block numbers
    [, per-sequence score arrays M_s]."""
    qi, ki = _u16(q_idx), _u16(k_idx)
    cu = _cu(cu_seqlens)
    T, H_kv, _ = qi.shape
    out = np.full((T, H_kv, k), -1, dtype=np.int32)
    Ms = []
    for s in range(cu.size - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        if b == a:
            Ms.append(None)
            continue
        M = block_scores(qi[a:b], ki[a:b], B_k)
        out[a:b] = topk(M, k, B_k)
        Ms.append(M)
    return (out, Ms) if want_scores else out


def sparse_attn_varlen(q, k, v, block_idx, cu_seqlens, B_k: int, scale: float | None = None):
    """Packed sequences, each its own instance of Eq. 8 over its rows of block_idx
    (sequence-local block numbers).  Returns (o [T,H_q,d_h], lse [T,H_q]) float64."""
    qq, kk_, vv = _u16(q), _u16(k), _u16(v)
    cu = _cu(cu_seqlens)
    bi = np.asarray(block_idx, dtype=np.int32)
    T, H_q, d_h = qq.shape
    o = np.zeros((T, H_q, d_h), dtype=np.float64)
    lse = np.full((T, H_q), -np.inf, dtype=np.float64)
    for s in range(cu.size - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        if b == a:
            continue
        o[a:b], lse[a:b] = sparse_attn(qq[a:b], kk_[a:b], vv[a:b], bi[a:b], B_k, scale)
    return o, lse


def fp8_e4m3(code: int) -> float:
    """OCP FP8 E4M3 code -> value."""
    return float(_load().msa_oracle_fp8_e4m3(code))


def _u8(x) -> np.ndarray:
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu()
            if x.dtype != torch.uint8:
                x = x.view(torch.uint8)
            return np.ascontiguousarray(x.numpy())
    except ImportError:
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.uint8))


def decode_paged(q, q_idx, k_pages, v_pages, k_scale: float, v_scale: float, kidx_pages, block_table, seqlens,
                 k: int, B_k: int, scale: float | None = None, want_scores: bool = False, block_idx=None):
    """Decode over paged caches (FP8 E4M3 K/V pages, bf16 index-key pages).  Returns
    block_idx, o, lse[, M] as ``decode``; a given ``block_idx`` [batch, H_kv, k] is
    used instead of the Top-k."""
    qq, qi, kip = _u16(q), _u16(q_idx), _u16(kidx_pages)
    kp, vp = _u8(k_pages), _u8(v_pages)
    bt = np.ascontiguousarray(np.asarray(block_table.cpu() if hasattr(block_table, "cpu") else block_table,
                                         dtype=np.int32))
    lens = np.ascontiguousarray(np.asarray(seqlens.cpu() if hasattr(seqlens, "cpu") else seqlens, dtype=np.int64))
    batch, H_q, d_h = qq.shape
    H_kv, d_idx = qi.shape[1], qi.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(d_h)
    Bmax = int((lens.max() + B_k - 1) // B_k) if batch else 0
    bi = np.empty((batch, H_kv, k), dtype=np.int32)
    o = np.empty((batch, H_q, d_h), dtype=np.float64)
    lse = np.empty((batch, H_q), dtype=np.float64)
    M = np.empty((batch, H_kv, Bmax), dtype=np.float64) if want_scores else None
    given = None
    if block_idx is not None:
        given = np.ascontiguousarray(np.asarray(block_idx.cpu() if hasattr(block_idx, "cpu") else block_idx,
                                                dtype=np.int32))
        assert given.shape == (batch, H_kv, k)
    _load().msa_oracle_decode_paged(_ptr(qq), _ptr(qi), _ptr(kp), _ptr(vp), float(k_scale), float(v_scale),
                                    _ptr(kip), _ptr(bt), bt.shape[1], _ptr(lens), batch, H_q, H_kv, d_h, d_idx, B_k,
                                    k, float(scale), None if given is None else _ptr(given), _ptr(bi), _ptr(o),
                                    _ptr(lse), None if M is None else _ptr(M), Bmax)
    if want_scores:
        return bi, o, lse, M
    return bi, o, lse
