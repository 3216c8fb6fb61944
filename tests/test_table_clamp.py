"""The clamps the kernels apply to the caller's device tables (packed offsets,
paged lengths and page numbers), compiled for the host from the same header the
kernels include and driven with malformed tables: every span and page the kernels
would touch stays inside the buffers, and well-formed tables pass unchanged."""
import ctypes
import os
import subprocess

import numpy as np
import pytest

HDR_DIR = os.path.join(os.path.dirname(__file__), "..", "block_sparse_gqa_index_amd", "csrc")

DRIVER = r"""
#include "table_clamp.h"
extern "C" {
// Spans of every sequence as the index and decode kernels read them.
void spans(const int64_t* cu, int batch, int64_t T, int64_t* start, int64_t* len) {
  for (int s = 0; s < batch; ++s) {
    const msa::PackedSpan p = msa::packed_span(cu[s], cu[s + 1], T);
    start[s] = p.start;
    len[s] = p.len;
  }
}
// The attention's sanitised table, from the running maximum as its scan forms it.
void sanitize(const int64_t* cu, int batch, int64_t T, int64_t* out) {
  int64_t pmax = INT64_MIN;
  for (int s = 0; s <= batch; ++s) {
    if (cu[s] > pmax) pmax = cu[s];
    out[s] = msa::sanitized_offset(pmax, s, batch, T);
  }
}
int64_t paged_len(int64_t raw, int64_t max_blocks, int64_t bk) { return msa::paged_len(raw, max_blocks, bk); }
int64_t page_number(int64_t raw, int64_t num_pages) { return msa::page_number(raw, num_pages); }
}
"""


@pytest.fixture(scope="module")
def clamp(tmp_path_factory):
    d = tmp_path_factory.mktemp("clamp")
    src = d / "driver.cpp"
    src.write_text(DRIVER)
    so = d / "libclamp.so"
    subprocess.run(["g++", "-std=c++17", "-O2", "-fPIC", "-shared", "-I", HDR_DIR, "-o", str(so), str(src)],
                   check=True)
    lib = ctypes.CDLL(str(so))
    P, I, L = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    lib.spans.argtypes = [P, I, L, P, P]
    lib.sanitize.argtypes = [P, I, L, P]
    lib.paged_len.argtypes = [L, L, L]
    lib.paged_len.restype = L
    lib.page_number.argtypes = [L, L]
    lib.page_number.restype = L
    return lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _spans(lib, cu, T):
    cu = np.ascontiguousarray(cu, dtype=np.int64)
    b = cu.size - 1
    start, ln = np.empty(b, np.int64), np.empty(b, np.int64)
    lib.spans(_ptr(cu), b, T, _ptr(start), _ptr(ln))
    return start, ln


def _sanitize(lib, cu, T):
    cu = np.ascontiguousarray(cu, dtype=np.int64)
    out = np.empty_like(cu)
    lib.sanitize(_ptr(cu), cu.size - 1, T, _ptr(out))
    return out


def _tables(seed, n=400):
    g = np.random.default_rng(seed)
    big = np.iinfo(np.int64)
    for _ in range(n):
        batch = int(g.integers(1, 12))
        T = int(g.integers(0, 5000))
        kind = g.integers(0, 4)
        if kind == 0:    # arbitrary values around [0, T]
            cu = g.integers(-3 * T - 5, 3 * T + 5, size=batch + 1)
        elif kind == 1:  # extremes
            cu = g.choice([big.min, big.max, -1, 0, T, T + 1], size=batch + 1)
        elif kind == 2:  # decreasing
            cu = np.sort(g.integers(-T, 2 * T + 1, size=batch + 1))[::-1].copy()
        else:            # well formed but for one entry
            cu = np.concatenate([[0], np.sort(g.integers(0, T + 1, size=batch - 1)), [T]])
            cu[g.integers(0, batch + 1)] = g.integers(-10 * T - 10, 10 * T + 10)
        yield batch, T, cu.astype(np.int64)


def test_packed_spans_stay_inside_the_buffers(clamp):
    for batch, T, cu in _tables(1):
        start, ln = _spans(clamp, cu, T)
        assert np.all(start >= 0) and np.all(ln >= 0) and np.all(start + ln <= T), (cu, T)


def test_sanitized_offsets_partition_the_tokens(clamp):
    for batch, T, cu in _tables(2):
        out = _sanitize(clamp, cu, T)
        assert out[0] == 0 and out[-1] == T, (cu, T, out)
        assert np.all(np.diff(out) >= 0), (cu, T, out)
        # Block counts of the partition stay within ceil(T / B_k) + batch.
        for bk in (64, 128):
            nb = (np.diff(out) + bk - 1) // bk
            assert nb.sum() <= (T + bk - 1) // bk + batch


def test_well_formed_tables_pass_unchanged(clamp):
    g = np.random.default_rng(3)
    for _ in range(300):
        batch = int(g.integers(1, 20))
        T = int(g.integers(0, 100000))
        cu = np.concatenate([[0], np.sort(g.integers(0, T + 1, size=batch - 1)), [T]]).astype(np.int64)
        start, ln = _spans(clamp, cu, T)
        np.testing.assert_array_equal(start, cu[:-1])
        np.testing.assert_array_equal(ln, np.diff(cu))
        np.testing.assert_array_equal(_sanitize(clamp, cu, T), cu)


def test_paged_lengths_and_pages_are_clamped(clamp):
    big = np.iinfo(np.int64)
    for raw in (big.min, -5, -1, 0, 1, 127, 128, 1023, 1024, 1025, 10 ** 12, big.max):
        L = clamp.paged_len(int(raw), 8, 128)
        assert 0 <= L <= 8 * 128
        if 0 <= raw <= 1024:
            assert L == raw
    for raw in (-(2 ** 31), -1, 0, 5, 63, 64, 2 ** 31 - 1):
        p = clamp.page_number(int(raw), 64)
        assert 0 <= p < 64
        if 0 <= raw < 64:
            assert p == raw
