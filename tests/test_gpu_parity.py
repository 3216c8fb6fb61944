"""GPU parity at sizes the oracle finishes in seconds: full rows, several tiles, ragged tails.

Every call goes through the C ABI (via the ctypes binding); the oracle sees host
copies of the same bf16 bytes.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.parity import check_attn, check_block_idx, check_exact_twin_ties

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def msa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_gqa_index_amd as m
    return m


def _inputs(N, H_q, H_kv, k, seed, mode="literal", needles=0):
    return synth.small_prefill(N=N, H_q=H_q, H_kv=H_kv, k=k, seed=seed, mode=mode, needles=needles, device=DEV)


INDEX_SHAPES = [  # N, H_kv, k
    (4096, 1, 8),
    (1000, 2, 4),
    (129, 3, 2),
    (1, 1, 8),
    (128, 2, 1),
    (5000, 4, 16),
    (3000, 2, 32),
    (700, 8, 16),
    (2047, 5, 9),
]


@pytest.mark.parametrize("N,H_kv,k", INDEX_SHAPES)
def test_block_scores_match_oracle(msa, N, H_kv, k):
    inp = _inputs(N, H_kv, H_kv, k, seed=100 + N, needles=0)
    M = msa.msa_index_block_scores(inp.q_idx, inp.k_idx)
    torch.cuda.synchronize()
    Mo = oracle.block_scores(inp.q_idx, inp.k_idx, 128)
    Mg = M.double().cpu().numpy()
    fin = np.isfinite(Mo)
    assert np.array_equal(np.isfinite(Mg), fin)
    assert np.all(Mg[~fin] == -np.inf)
    err = np.abs(Mg[fin] - Mo[fin]) / np.maximum(1.0, np.abs(Mo[fin]))
    assert err.max() <= 1e-5, err.max()


@pytest.mark.parametrize("N,H_kv,k", [(4096, 1, 8), (3000, 3, 16), (2000, 2, 32), (300, 2, 5), (129, 1, 1),
                                      (9000, 2, 17)])
def test_topk_from_scores_bit_exact(msa, N, H_kv, k):
    """Selection on given fp32 scores with many exact ties: bit-exact against the oracle."""
    g = torch.Generator().manual_seed(N * 7 + k)
    B = (N + 127) // 128
    M = (torch.randint(-6, 7, (N, H_kv, B), generator=g).float() * 0.25)
    bi = msa.msa_topk_from_scores(M.to(DEV), k)
    torch.cuda.synchronize()
    ref = oracle.topk(M.double().numpy(), k, 128)
    np.testing.assert_array_equal(bi.cpu().numpy(), ref)


def _check_index(msa, inp, k):
    bi = msa.msa_index_topk(inp.q_idx, inp.k_idx, k)
    torch.cuda.synchronize()
    N = inp.q_idx.shape[0]
    M = oracle.block_scores(inp.q_idx, inp.k_idx, 128)
    tie = check_block_idx(bi.cpu().numpy(), M, np.arange(N), k, 128)
    return bi, tie


@pytest.mark.parametrize("mode", ["literal", "structured"])
@pytest.mark.parametrize("N,H_kv,k", INDEX_SHAPES)
def test_index_topk_matches_oracle(msa, N, H_kv, k, mode):
    inp = _inputs(N, H_kv, H_kv, k, seed=200 + N + k, mode=mode, needles=1 if N >= 1000 else 0)
    _check_index(msa, inp, k)


def _twin_blocks(k_idx, B_k, n_blocks):
    """Make block b an exact copy of block b - 1 for every odd b < n_blocks (full blocks only)."""
    k_idx = k_idx.clone()
    for b in range(1, n_blocks, 2):
        k_idx[b * B_k:(b + 1) * B_k] = k_idx[(b - 1) * B_k:b * B_k]
    return k_idx


@pytest.mark.parametrize("B_k", [128, 64])
@pytest.mark.parametrize("N,H_kv,k", [(2048, 2, 4), (4096, 3, 8), (5000, 2, 16), (3000, 1, 2), (6000, 2, 32)])
def test_index_topk_exact_ties_go_to_lower_block(msa, N, H_kv, k, B_k):
    """Duplicated index-key blocks make exact ties in block score, so the k-th slot
    falls between two equal blocks on most rows.  Where the tie is the only freedom
    (every other block clearly above or below it), the fused kernel must pick the
    lower block, bit-exactly as the oracle does; all other rows follow the usual rule."""
    inp = _inputs(N, H_kv, H_kv, k, seed=7 + N + k + B_k)
    nb = N // B_k
    kidx = _twin_blocks(inp.k_idx, B_k, nb)
    bi = msa.msa_index_topk(inp.q_idx, kidx, k, B_k=B_k)
    Mg = msa.msa_index_block_scores(inp.q_idx, kidx, B_k=B_k)
    torch.cuda.synchronize()
    M = oracle.block_scores(inp.q_idx, kidx, B_k)
    # The GPU's own fp32 scores of twin blocks are equal wherever both are fully visible.
    Mg = Mg.cpu().numpy()
    for b in range(1, nb, 2):
        past = np.arange(N) >= (b + 1) * B_k
        assert np.array_equal(Mg[past, :, b - 1], Mg[past, :, b]), f"GPU scores of twin blocks {b - 1}, {b} differ"
    bi = bi.cpu().numpy()
    check_block_idx(bi, M, np.arange(N), k, B_k)
    n_tied = check_exact_twin_ties(bi, M, np.arange(N), k, B_k)
    assert n_tied >= N * H_kv // 8, f"only {n_tied} rows had an isolated exact tie"


ATTN_SHAPES = [  # N, H_q, H_kv, k
    (4096, 4, 1, 8),
    (1000, 16, 2, 4),
    (700, 8, 8, 3),
    (300, 4, 2, 16),
    (1, 8, 1, 4),
    (129, 32, 1, 2),
    (2600, 16, 1, 5),
    (512, 64, 4, 4),
    (3000, 8, 1, 16),  # one GPU's share of the 128K workload when the 8 groups are split
]


@pytest.mark.parametrize("N,H_q,H_kv,k", ATTN_SHAPES)
def test_sparse_attn_on_oracle_selection(msa, N, H_q, H_kv, k):
    """The main branch alone, on the oracle's own block_idx."""
    inp = _inputs(N, H_q, H_kv, k, seed=300 + N)
    M = oracle.block_scores(inp.q_idx, inp.k_idx, 128)
    bi = oracle.topk(M, k, 128)
    o, lse = msa.msa_sparse_attn_fwd(inp.q, inp.k, inp.v, torch.from_numpy(bi).to(DEV))
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.sparse_attn(inp.q, inp.k, inp.v, bi, 128)
    check_attn(o.cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, f"N={N} H_q={H_q} H_kv={H_kv} k={k}")


def test_sparse_attn_arbitrary_block_sets(msa):
    """-1 entries, future blocks (no visible token), empty rows and unordered lists."""
    N, H_q, H_kv, k = 1500, 8, 2, 5
    inp = _inputs(N, H_q, H_kv, k, seed=11)
    g = np.random.default_rng(3)
    B = (N + 127) // 128
    bi = np.full((N, H_kv, k), -1, dtype=np.int32)
    for i in range(N):
        for r in range(H_kv):
            c = g.choice(B, size=g.integers(0, k + 1), replace=False)
            bi[i, r, :len(c)] = c
    bi[5] = -1                      # no block at all
    bi[900, 0] = [11, 10, -1, 9, -1]  # only future blocks for query 900 (local block 7)
    o, lse = msa.msa_sparse_attn_fwd(inp.q, inp.k, inp.v, torch.from_numpy(bi).to(DEV))
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.sparse_attn(inp.q, inp.k, inp.v, bi, 128)
    assert np.all(np.isinf(lse_ref[5])) and np.all(np.isinf(lse_ref[900, :4]))
    check_attn(o.cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, "arbitrary sets")


def test_sparse_attn_scale_argument(msa):
    N, H_q, H_kv, k = 600, 4, 2, 3
    inp = _inputs(N, H_q, H_kv, k, seed=12)
    bi = oracle.topk(oracle.block_scores(inp.q_idx, inp.k_idx, 128), k, 128)
    o, lse = msa.msa_sparse_attn_fwd(inp.q, inp.k, inp.v, torch.from_numpy(bi).to(DEV), scale=0.03)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.sparse_attn(inp.q, inp.k, inp.v, bi, 128, scale=0.03)
    check_attn(o.cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, "scale 0.03")


@pytest.mark.parametrize("mode", ["literal", "structured"])
def test_end_to_end_tiny_workload(msa, mode):
    """The whole path on the 4K workload (H_q=4, H_kv=1, k=8): selection, then attention."""
    inp = synth.make_prefill(synth.CONFIGS["c0"], mode, device=DEV)
    k = 8
    bi, tie = _check_index(msa, inp, k)
    o, lse = msa.msa_sparse_attn_fwd(inp.q, inp.k, inp.v, bi)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.sparse_attn(inp.q, inp.k, inp.v, bi.cpu().numpy(), 128)
    check_attn(o.cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, f"c0 {mode}")


def test_query_windows_and_reruns_are_bitwise_identical(msa):
    """Small workspaces split the queries into windows; results must not change at all."""
    N, H_q, H_kv, k = 3000, 16, 2, 6
    inp = _inputs(N, H_q, H_kv, k, seed=13, needles=2)
    bi = msa.msa_index_topk(inp.q_idx, inp.k_idx, k)
    bi2 = msa.msa_index_topk(inp.q_idx, inp.k_idx, k)
    o1, l1 = msa.msa_sparse_attn_fwd(inp.q, inp.k, inp.v, bi)
    wmin = msa.msa_sparse_attn_fwd_workspace(N, H_q, H_kv, k, minimum=True)
    ws = torch.empty(wmin, dtype=torch.uint8, device=DEV)
    o2, l2 = msa.msa_sparse_attn_fwd(inp.q, inp.k, inp.v, bi, workspace=ws)
    o3, l3 = msa.msa_sparse_attn_fwd(inp.q, inp.k, inp.v, bi)
    torch.cuda.synchronize()
    assert torch.equal(bi, bi2)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o1, o3) and torch.equal(l1, l3)


def test_profile_events_per_query_window(msa):
    """The measurement hook records 4 events per query window for as many windows as
    it was given; a windowed call's phases then add up to its whole duration."""
    N, H_q, H_kv, k = 3000, 16, 2, 6
    inp = _inputs(N, H_q, H_kv, k, seed=14, needles=2)
    bi = msa.msa_index_topk(inp.q_idx, inp.k_idx, k)
    wmin = msa.msa_sparse_attn_fwd_workspace(N, H_q, H_kv, k, minimum=True)
    ws = torch.empty(wmin, dtype=torch.uint8, device=DEV)
    n_win = msa.msa_sparse_attn_fwd_windows(N, H_q, H_kv, k, wmin)
    assert n_win == (N + 127) // 128
    assert msa.msa_sparse_attn_fwd_windows(N, H_q, H_kv, k,
                                           msa.msa_sparse_attn_fwd_workspace(N, H_q, H_kv, k)) == 1
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4 * n_win)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    msa.msa_set_profile_events(ev)
    try:
        start.record(stream)
        o, lse = msa.msa_sparse_attn_fwd(inp.q, inp.k, inp.v, bi, workspace=ws)
        end.record(stream)
    finally:
        msa.msa_set_profile_events(None)
    torch.cuda.synchronize()
    phases = [ev[4 * w + p].elapsed_time(ev[4 * w + p + 1]) for w in range(n_win) for p in range(3)]
    assert all(t >= 0 for t in phases)
    gaps = [ev[4 * w + 3].elapsed_time(ev[4 * w + 4]) for w in range(n_win - 1)]
    assert all(t >= 0 for t in gaps)  # windows run in order on the stream
    total = start.elapsed_time(end)
    assert sum(phases) <= total * 1.05 + 0.01
    o_ref, l_ref = msa.msa_sparse_attn_fwd(inp.q, inp.k, inp.v, bi)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)


def test_empty_inputs(msa):
    z = torch.empty((0, 2, 64), dtype=torch.bfloat16, device=DEV)
    bi = msa.msa_index_topk(z, torch.empty((0, 64), dtype=torch.bfloat16, device=DEV), 4)
    assert bi.shape == (0, 2, 4)
    q = torch.empty((0, 8, 128), dtype=torch.bfloat16, device=DEV)
    kv = torch.empty((0, 2, 128), dtype=torch.bfloat16, device=DEV)
    o, lse = msa.msa_sparse_attn_fwd(q, kv, kv, torch.empty((0, 2, 4), dtype=torch.int32, device=DEV))
    assert o.shape == (0, 8, 128) and lse.shape == (0, 8)


DECODE_CASES = [  # lengths, H_q, H_kv, k
    ([1, 100, 128, 129, 1000, 5000], 16, 2, 4),
    ([4096, 3000, 256, 640], 64, 8, 16),
    ([2000, 70], 8, 8, 32),
    ([384] * 3, 16, 1, 3),
]


@pytest.mark.parametrize("mode", ["literal", "structured"])
@pytest.mark.parametrize("case", range(len(DECODE_CASES)))
def test_decode_matches_oracle(msa, case, mode):
    lengths, H_q, H_kv, k = DECODE_CASES[case]
    cfg = synth.DecodeConfig("t", batch=len(lengths), H_q=H_q, H_kv=H_kv, k=k, len_lo_blocks=1, len_hi_blocks=1,
                             seed=500 + case)
    d = synth.make_decode(cfg, mode, device=DEV, lengths=lengths)
    bi, o, lse = msa.msa_decode(d.q, d.q_idx, d.k_cache, d.v_cache, d.k_idx_cache, d.cu_seqlens, max(lengths), k)
    torch.cuda.synchronize()
    bi_ref, o_ref, lse_ref, M = oracle.decode(d.q, d.q_idx, d.k_cache, d.v_cache, d.k_idx_cache, d.cu_seqlens, k,
                                              128, want_scores=True)
    pos = np.array(lengths) - 1
    bi_gpu = bi.cpu().numpy()
    tie = check_block_idx(bi_gpu, M, pos, k, 128)
    if tie.any():  # attention compared on the GPU's own selection
        o_ref, lse_ref = oracle.decode_attn(d.q, d.k_cache, d.v_cache, d.cu_seqlens, bi_gpu, 128)
    check_attn(o.cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, f"decode case {case}")


def _twin_cache_blocks(k_idx_cache, lengths, B_k):
    """In every sequence of a packed cache, make full block b an exact copy of block
    b - 1 for odd b."""
    out = k_idx_cache.clone()
    t0 = 0
    for L in lengths:
        for b in range(1, L // B_k, 2):
            out[t0 + b * B_k:t0 + (b + 1) * B_k] = out[t0 + (b - 1) * B_k:t0 + b * B_k]
        t0 += L
    return out


@pytest.mark.parametrize("B_k", [128, 64])
@pytest.mark.parametrize("k", [2, 4, 16, 32])
def test_decode_exact_ties_go_to_lower_block(msa, k, B_k):
    """Duplicated cached index-key blocks: the decode Top-k must give an exact boundary
    tie to the lower block, bit-exactly as the oracle does."""
    batch, H_q, H_kv = 48, 16, 8
    cfg = synth.DecodeConfig("t", batch=batch, H_q=H_q, H_kv=H_kv, k=k, len_lo_blocks=24, len_hi_blocks=48,
                             B_k=B_k, seed=560 + k + B_k)
    d = synth.make_decode(cfg, device=DEV)
    kidx = _twin_cache_blocks(d.k_idx_cache, d.lengths, B_k)
    bi, o, lse = msa.msa_decode(d.q, d.q_idx, d.k_cache, d.v_cache, kidx, d.cu_seqlens, max(d.lengths), k,
                                B_k=B_k)
    torch.cuda.synchronize()
    _, _, _, M = oracle.decode(d.q, d.q_idx, d.k_cache, d.v_cache, kidx, d.cu_seqlens, k, B_k, want_scores=True)
    pos = np.array(d.lengths) - 1
    bi = bi.cpu().numpy()
    check_block_idx(bi, M, pos, k, B_k)
    n_tied = check_exact_twin_ties(bi, M, pos, k, B_k)
    assert n_tied >= batch * H_kv // 4, f"only {n_tied} rows had an isolated exact tie"
