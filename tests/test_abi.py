"""The C ABI: the library loads, exports every declared symbol, and rejects bad calls
on the host before anything is launched (no GPU is touched by these tests)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msa.h")
LIB = os.path.join(ROOT, "block_sparse_gqa_index_amd", "libmsa.so")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(msa_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from __graft_entry__ import load_builder
        load_builder().build()
    import block_sparse_gqa_index_amd as m
    return m


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert {"msa_index_topk", "msa_sparse_attn_fwd", "msa_decode"} <= set(names)
    raw = ctypes.CDLL(LIB)
    for n in names:
        assert hasattr(raw, n), n
    assert set(names) == set(lib.EXPORTED)


def test_no_oracle_or_torch_in_library():
    # The product path is the HIP library alone: it must not link the oracle.
    data = open(LIB, "rb").read() if os.path.exists(LIB) else b""
    assert b"msa_oracle_" not in data


def test_status_strings(lib):
    raw = lib.raw()
    for s, name in enumerate(["MSA_OK", "MSA_ERR_INVALID_ARG", "MSA_ERR_UNSUPPORTED", "MSA_ERR_WORKSPACE",
                              "MSA_ERR_HIP"]):
        assert raw.msa_status_string(s).decode() == name


def test_index_topk_rejects_bad_arguments(lib):
    raw = lib.raw()
    fake = 0x10000  # never dereferenced: every call below fails validation first
    call = lambda N=4096, H_kv=1, d_idx=64, B_k=128, k=8, q=fake, kk=fake, out=fake: raw.msa_index_topk(
        q, kk, N, H_kv, d_idx, B_k, k, out, None, 0, None)
    assert call(d_idx=32) == lib.MSA_ERR_UNSUPPORTED
    assert call(B_k=32) == lib.MSA_ERR_UNSUPPORTED
    assert call(B_k=256) == lib.MSA_ERR_UNSUPPORTED
    assert call(N=8192 * 64 + 1, B_k=64) == lib.MSA_ERR_UNSUPPORTED  # more than 8192 blocks
    assert call(k=0) == lib.MSA_ERR_UNSUPPORTED
    assert call(k=33) == lib.MSA_ERR_UNSUPPORTED
    assert call(N=-1) == lib.MSA_ERR_INVALID_ARG
    assert call(N=1 << 24) == lib.MSA_ERR_UNSUPPORTED
    assert call(H_kv=0) == lib.MSA_ERR_INVALID_ARG
    assert call(q=None) == lib.MSA_ERR_INVALID_ARG
    assert call(out=fake + 2) == lib.MSA_ERR_INVALID_ARG
    assert call(q=fake + 8) == lib.MSA_ERR_INVALID_ARG
    assert "misaligned" in raw.msa_last_error().decode()
    assert call(N=0, q=None, kk=None, out=None) == lib.MSA_OK  # empty call: nothing to do


def test_sparse_attn_rejects_bad_arguments(lib):
    raw = lib.raw()
    f = 0x10000

    def call(N=4096, H_q=8, H_kv=2, d_h=128, B_k=128, k=8, scale=0.088, ws=f, ws_bytes=1 << 40, o=f):
        return raw.msa_sparse_attn_fwd(f, f, f, f, N, H_q, H_kv, d_h, B_k, k, scale, o, f, ws, ws_bytes, None)

    assert call(d_h=64) == lib.MSA_ERR_UNSUPPORTED
    assert call(H_q=6, H_kv=4) == lib.MSA_ERR_INVALID_ARG
    assert call(H_q=24, H_kv=8) == lib.MSA_ERR_UNSUPPORTED  # G = 3
    assert call(scale=0.0) == lib.MSA_ERR_INVALID_ARG
    assert call(scale=float("nan")) == lib.MSA_ERR_INVALID_ARG
    assert call(ws=None) == lib.MSA_ERR_WORKSPACE
    need = raw.msa_sparse_attn_fwd_workspace_min(4096, 8, 2, 128, 128, 8)
    assert need > 0
    assert call(ws_bytes=need - 1) == lib.MSA_ERR_WORKSPACE
    assert call(ws=f + 16) == lib.MSA_ERR_INVALID_ARG  # workspace must be 256-byte aligned
    assert call(o=f + 4) == lib.MSA_ERR_INVALID_ARG
    assert call(N=0) == lib.MSA_OK


def test_workspace_sizes(lib):
    raw = lib.raw()
    assert raw.msa_index_topk_workspace(131072, 8, 64, 128, 16) == 0
    full = raw.msa_sparse_attn_fwd_workspace(131072, 64, 8, 128, 128, 16)
    small = raw.msa_sparse_attn_fwd_workspace_min(131072, 64, 8, 128, 128, 16)
    assert 0 < small < full <= (40 << 30)
    # one query window of 128 queries: partial rows of 128 bf16 + one fp32 lse each
    assert small >= 128 * 64 * 16 * (128 * 2 + 4)
    assert raw.msa_sparse_attn_fwd_workspace(131072, 64, 8, 64, 128, 16) == 0  # unsupported d_h
    assert raw.msa_decode_workspace(64, 64, 8, 128, 64, 128, 16, 131072) >= 64 * 8 * 1024 * 4
    assert raw.msa_decode_workspace(64, 64, 32, 128, 64, 128, 16, 131072) == 0  # H_kv > 16


def test_decode_rejects_bad_arguments(lib):
    raw = lib.raw()
    f = 0x10000

    def call(batch=4, max_len=1024, H_q=16, H_kv=2, d_h=128, d_idx=64, B_k=128, k=4, ws=f, ws_bytes=1 << 40,
             cu=f, T=4096):
        return raw.msa_decode(f, f, f, f, f, cu, batch, T, max_len, H_q, H_kv, d_h, d_idx, B_k, k, 0.088, f, f, f,
                              ws, ws_bytes, None)

    assert call(d_idx=128) == lib.MSA_ERR_UNSUPPORTED
    assert call(H_q=64, H_kv=2) == lib.MSA_ERR_UNSUPPORTED  # G = 32 > 16
    assert call(batch=-1) == lib.MSA_ERR_INVALID_ARG
    assert call(max_len=0) == lib.MSA_ERR_INVALID_ARG
    assert call(T=-1) == lib.MSA_ERR_INVALID_ARG
    assert call(cu=None) == lib.MSA_ERR_INVALID_ARG
    assert call(cu=f + 4) == lib.MSA_ERR_INVALID_ARG
    assert call(ws_bytes=16) == lib.MSA_ERR_WORKSPACE
    assert call(batch=0) == lib.MSA_OK


def test_kl_from_lse_idx_rejects_bad_arguments(lib):
    raw = lib.raw()
    f = 0x10000

    def call(N=4096, H_q=8, H_kv=2, d_idx=64, li=f, kl=f, ws=f, ws_bytes=1 << 40):
        return raw.msa_sparse_kl_fwd_from_lse_idx(f, f, f, f, f, f, li, N, H_q, H_kv, 128, d_idx, 128, 8, 0.088, kl,
                                                  f, ws, ws_bytes, None)

    assert call(d_idx=128) == lib.MSA_ERR_UNSUPPORTED
    assert call(H_q=128, H_kv=2) == lib.MSA_ERR_UNSUPPORTED  # G = 64 > 32
    assert call(li=None) == lib.MSA_ERR_INVALID_ARG
    assert call(li=f + 2) == lib.MSA_ERR_INVALID_ARG
    assert call(kl=None) == lib.MSA_ERR_INVALID_ARG
    assert call(ws_bytes=16) == lib.MSA_ERR_WORKSPACE
    assert call(N=0) == lib.MSA_OK


def test_forward_lse_idx_rejects_bad_arguments(lib):
    raw = lib.raw()
    f = 0x10000

    def call(N=4096, d_idx=64, qi=f, ki=f, li=f, ws=f, ws_bytes=1 << 40):
        return raw.msa_sparse_attn_fwd_lse_idx(f, f, f, qi, ki, f, N, 8, 2, 128, d_idx, 128, 8, 0.088, f, f, li,
                                               ws, ws_bytes, None)

    assert call(d_idx=128) == lib.MSA_ERR_UNSUPPORTED
    assert call(qi=None) == lib.MSA_ERR_INVALID_ARG
    assert call(li=None) == lib.MSA_ERR_INVALID_ARG
    assert call(ki=f + 8) == lib.MSA_ERR_INVALID_ARG  # k_idx needs 16 B
    assert call(ws_bytes=16) == lib.MSA_ERR_WORKSPACE
    assert call(N=0) == lib.MSA_OK


def test_profile_clock_hook_validates(lib):
    raw = lib.raw()
    assert raw.msa_set_profile_clock(None, 4) == lib.MSA_ERR_INVALID_ARG
    assert raw.msa_set_profile_clock(0x10004, 4) == lib.MSA_ERR_INVALID_ARG  # not 8-byte aligned
    assert raw.msa_set_profile_clock(0x10000, -2) == lib.MSA_ERR_INVALID_ARG
    assert raw.msa_set_profile_clock(None, 0) == lib.MSA_OK


def test_profile_events_hook_validates(lib):
    raw = lib.raw()
    assert raw.msa_set_profile_events(None, 3) == lib.MSA_ERR_INVALID_ARG
    assert raw.msa_set_profile_events(None, 4) == lib.MSA_ERR_INVALID_ARG
    import ctypes as C
    arr = (C.c_void_p * 4)(0x10, 0x20, None, 0x40)
    assert raw.msa_set_profile_events(arr, 4) == lib.MSA_ERR_INVALID_ARG  # null handle
    arr8 = (C.c_void_p * 8)(*range(0x10, 0x90, 0x10))
    assert raw.msa_set_profile_events(arr8, 6) == lib.MSA_ERR_INVALID_ARG  # not 4 per window
    assert raw.msa_set_profile_events(arr8, 4 * 1025) == lib.MSA_ERR_INVALID_ARG
    assert raw.msa_set_profile_events(None, 0) == lib.MSA_OK


def test_window_count_query(lib):
    raw = lib.raw()
    N, H_q, H_kv, k = 131072, 64, 8, 16
    full = raw.msa_sparse_attn_fwd_workspace(N, H_q, H_kv, 128, 128, k)
    small = raw.msa_sparse_attn_fwd_workspace_min(N, H_q, H_kv, 128, 128, k)
    assert raw.msa_sparse_attn_fwd_windows(N, H_q, H_kv, 128, 128, k, full) == 1
    assert raw.msa_sparse_attn_fwd_windows(N, H_q, H_kv, 128, 128, k, small) == N // 128
    assert raw.msa_sparse_attn_fwd_windows(N, H_q, H_kv, 128, 128, k, small - 1) == -1
    half = raw.msa_sparse_attn_fwd_windows(N, H_q, H_kv, 128, 128, k, full // 2 + small)
    assert 2 <= half <= 3
    assert raw.msa_sparse_attn_fwd_windows(0, H_q, H_kv, 128, 128, k, 0) == 0
    assert raw.msa_sparse_attn_fwd_windows(N, H_q, H_kv, 64, 128, k, full) == -1  # unsupported d_h
    # 1M tokens under the default workspace run in several windows.
    big = raw.msa_sparse_attn_fwd_workspace(1 << 20, H_q, H_kv, 128, 128, k)
    assert raw.msa_sparse_attn_fwd_windows(1 << 20, H_q, H_kv, 128, 128, k, big) > 1


def test_binding_fails_loudly_without_library(tmp_path):
    # Importing the binding from a copy without libmsa.so must raise, not fall back.
    import shutil
    import subprocess
    import sys
    pkg = tmp_path / "block_sparse_gqa_index_amd"
    pkg.mkdir()
    shutil.copy(os.path.join(ROOT, "block_sparse_gqa_index_amd", "__init__.py"), pkg / "__init__.py")
    r = subprocess.run([sys.executable, "-c", "import block_sparse_gqa_index_amd"], cwd=tmp_path,
                       capture_output=True, text=True)
    assert r.returncode != 0 and "libmsa.so is missing" in r.stderr


def test_varlen_rejects_bad_arguments(lib):
    raw = lib.raw()
    f = 0x10000

    def idx(batch=3, T=4096, max_len=2048, H_kv=2, d_idx=64, B_k=128, k=8, cu=f, q=f):
        return raw.msa_index_topk_varlen(q, f, cu, batch, T, max_len, H_kv, d_idx, B_k, k, f, None)

    assert idx(batch=-1) == lib.MSA_ERR_INVALID_ARG
    assert idx(max_len=4097) == lib.MSA_ERR_INVALID_ARG  # longer than T
    assert idx(max_len=0) == lib.MSA_ERR_INVALID_ARG
    assert idx(cu=None) == lib.MSA_ERR_INVALID_ARG
    assert idx(cu=f + 4) == lib.MSA_ERR_INVALID_ARG
    assert idx(d_idx=128) == lib.MSA_ERR_UNSUPPORTED
    assert idx(T=8192 * 128, max_len=128, batch=2) == lib.MSA_ERR_UNSUPPORTED  # blocks + batch > 8192
    assert idx(batch=0, cu=None, q=None) == lib.MSA_OK

    def attn(batch=3, T=4096, H_q=8, H_kv=2, d_h=128, k=8, ws=f, ws_bytes=1 << 40, cu=f, scale=0.088):
        return raw.msa_sparse_attn_fwd_varlen(f, f, f, f, cu, batch, T, H_q, H_kv, d_h, 128, k, scale, f, f, ws,
                                              ws_bytes, None)

    assert attn(d_h=64) == lib.MSA_ERR_UNSUPPORTED
    assert attn(cu=None) == lib.MSA_ERR_INVALID_ARG
    assert attn(scale=-1.0) == lib.MSA_ERR_INVALID_ARG
    assert attn(ws=None) == lib.MSA_ERR_WORKSPACE
    need = raw.msa_sparse_attn_fwd_varlen_workspace_min(4096, 3, 8, 2, 128, 128, 8)
    # the sequence tables sit in front of the per-window buffers
    assert need > raw.msa_sparse_attn_fwd_workspace_min(4096, 8, 2, 128, 128, 8)
    assert attn(ws_bytes=need - 1) == lib.MSA_ERR_WORKSPACE
    assert attn(batch=0) == lib.MSA_OK
    assert raw.msa_sparse_attn_fwd_varlen_workspace(4096, 0, 8, 2, 128, 128, 8) == 0


def test_sparse_kl_rejects_bad_arguments(lib):
    raw = lib.raw()
    f = 0x10000

    def call(N=4096, H_q=8, H_kv=2, d_h=128, d_idx=64, k=8, scale=0.088, ws=f, ws_bytes=1 << 40, lse=f, loss=f,
             B_k=128):
        return raw.msa_sparse_kl_fwd(f, f, f, f, f, lse, N, H_q, H_kv, d_h, d_idx, B_k, k, scale, f, f, loss, ws,
                                     ws_bytes, None)

    assert call(B_k=32) == lib.MSA_ERR_UNSUPPORTED

    assert call(d_idx=32) == lib.MSA_ERR_UNSUPPORTED
    assert call(H_q=128, H_kv=2) == lib.MSA_ERR_UNSUPPORTED  # G = 64 > 32
    assert call(lse=None) == lib.MSA_ERR_INVALID_ARG
    assert call(loss=None) == lib.MSA_ERR_INVALID_ARG
    assert call(scale=0.0) == lib.MSA_ERR_INVALID_ARG
    assert call(ws=None) == lib.MSA_ERR_WORKSPACE
    need = raw.msa_sparse_kl_fwd_workspace_min(4096, 8, 2, 128, 64, 128, 8)
    assert 0 < need < raw.msa_sparse_kl_fwd_workspace(4096, 8, 2, 128, 64, 128, 8)
    assert call(ws_bytes=need - 1) == lib.MSA_ERR_WORKSPACE
    assert call(N=0) == lib.MSA_OK
    # partials are 32 bytes per (query, group, slot): far below the attention's rows
    full_kl = raw.msa_sparse_kl_fwd_workspace(131072, 64, 8, 128, 64, 128, 16)
    assert 0 < full_kl < raw.msa_sparse_attn_fwd_workspace(131072, 64, 8, 128, 128, 16) // 8


def test_decode_paged_rejects_bad_arguments(lib):
    raw = lib.raw()
    f = 0x10000

    def call(batch=4, max_len=1024, H_q=16, H_kv=2, k=4, ks=0.01, vs=0.01, max_blocks=8, bt=f, lens=f,
             ws=f, ws_bytes=1 << 40, B_k=128, num_pages=64):
        return raw.msa_decode_paged(f, f, f, f, ks, vs, f, bt, max_blocks, num_pages, lens, batch, max_len, H_q,
                                    H_kv, 128, 64, B_k, k, 0.088, f, f, f, ws, ws_bytes, None)

    assert call(B_k=32, max_blocks=32) == lib.MSA_ERR_UNSUPPORTED

    assert call(ks=0.0) == lib.MSA_ERR_INVALID_ARG
    assert call(vs=float("inf")) == lib.MSA_ERR_INVALID_ARG
    assert call(max_blocks=7) == lib.MSA_ERR_INVALID_ARG  # ceil(1024 / 128) = 8 blocks per row needed
    assert call(num_pages=0) == lib.MSA_ERR_INVALID_ARG
    assert call(bt=None) == lib.MSA_ERR_INVALID_ARG
    assert call(lens=f + 4) == lib.MSA_ERR_INVALID_ARG
    assert call(H_q=64, H_kv=2) == lib.MSA_ERR_UNSUPPORTED
    assert call(ws_bytes=16) == lib.MSA_ERR_WORKSPACE
    assert call(batch=0) == lib.MSA_OK


def test_backward_rejects_bad_arguments(lib):
    raw = lib.raw()
    f = 0x10000

    def call(N=4096, H_q=8, H_kv=2, d_h=128, B_k=128, k=8, ws=f, ws_bytes=1 << 40, o=f, dq=f):
        return raw.msa_sparse_attn_bwd(f, f, f, o, f, f, f, N, H_q, H_kv, d_h, B_k, k, 0.088, dq, f, f, ws,
                                       ws_bytes, None)

    assert call(B_k=32) == lib.MSA_ERR_UNSUPPORTED
    assert call(H_q=128, H_kv=2) == lib.MSA_ERR_UNSUPPORTED
    assert call(o=None) == lib.MSA_ERR_INVALID_ARG
    assert call(dq=f + 4) == lib.MSA_ERR_INVALID_ARG
    assert call(ws=None) == lib.MSA_ERR_WORKSPACE
    need = raw.msa_sparse_attn_bwd_workspace_min(4096, 8, 2, 128, 128, 8)
    assert 0 < need < raw.msa_sparse_attn_bwd_workspace(4096, 8, 2, 128, 128, 8)
    assert call(ws_bytes=need - 1) == lib.MSA_ERR_WORKSPACE
    assert call(N=0) == lib.MSA_OK


def test_noalloc_decode_rejects_shapes_beyond_its_static_scratch(lib):
    raw = lib.raw()
    f = 0x10000  # never dereferenced: the size check comes before any pointer or device use
    # 512 sequences of 1M tokens need 128 MiB of block scores: above the 32 MiB scratch.
    st = raw.msa_decode_noalloc(f, f, f, f, f, f, 512, 512 << 20, 1 << 20, 64, 8, 128, 64, 128, 16, 0.088, f, f, f,
                                None)
    assert st == lib.MSA_ERR_WORKSPACE
    assert "static" in raw.msa_last_error().decode()
    assert raw.msa_decode_noalloc(f, f, f, f, f, f, 0, 0, 0, 64, 8, 128, 64, 128, 16, 0.088, f, f, f,
                                  None) == lib.MSA_OK
    assert raw.msa_decode_noalloc(f, f, f, f, f, f, 4, 16384, 4096, 64, 8, 64, 64, 128, 16, 0.088, f, f, f,
                                  None) == lib.MSA_ERR_UNSUPPORTED  # d_h = 64
    assert raw.msa_decode_noalloc(f, f, f, f, f, f, 4, -1, 4096, 64, 8, 128, 64, 128, 16, 0.088, f, f, f,
                                  None) == lib.MSA_ERR_INVALID_ARG  # T < 0
