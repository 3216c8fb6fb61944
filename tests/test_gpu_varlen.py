"""GPU parity of the packed variable-length prefill entry points against the oracle.

Each sequence of a packed batch is its own instance of the method (positions,
blocks and the local block count from its start); the oracle runs them one by one.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.parity import check_attn, check_block_idx

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def msa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_gqa_index_amd as m
    return m


VARLEN_CASES = [  # lengths, H_q, H_kv, k
    ([1000, 129, 1, 2047], 16, 2, 4),
    ([128, 0, 300, 4096, 77], 4, 1, 8),
    ([700, 700, 700], 8, 8, 16),
    ([2500, 64, 1300], 32, 1, 32),
    ([5, 3, 1, 257, 0, 0, 900], 16, 4, 3),
    ([3000], 8, 1, 16),
]


def _packed(lengths, H_q, H_kv, k, seed, mode="literal"):
    return synth.packed_prefill(lengths, H_q, H_kv, k, seed, mode, device=DEV)


def _check_index_varlen(msa, p, k):
    lengths = p.lengths
    bi = msa.msa_index_topk_varlen(p.q_idx, p.k_idx, p.cu_seqlens, max(lengths), k)
    torch.cuda.synchronize()
    bi_h = bi.cpu().numpy()
    _, Ms = oracle.index_topk_varlen(p.q_idx, p.k_idx, p.cu_seqlens, k, 128, want_scores=True)
    cu = p.cu_seqlens.cpu().tolist()
    ties = np.zeros(bi_h.shape[:2], dtype=bool)
    for s, L in enumerate(lengths):
        if L == 0:
            continue
        a, b = cu[s], cu[s + 1]
        ties[a:b] = check_block_idx(bi_h[a:b], Ms[s], np.arange(L), k, 128)
    return bi, ties


@pytest.mark.parametrize("mode", ["literal", "structured"])
@pytest.mark.parametrize("case", range(len(VARLEN_CASES)))
def test_index_topk_varlen_matches_oracle(msa, case, mode):
    lengths, H_q, H_kv, k = VARLEN_CASES[case]
    p = _packed(lengths, H_kv, H_kv, k, seed=700 + 10 * case)
    _check_index_varlen(msa, p, k)


@pytest.mark.parametrize("case", range(len(VARLEN_CASES)))
def test_sparse_attn_varlen_on_oracle_selection(msa, case):
    lengths, H_q, H_kv, k = VARLEN_CASES[case]
    p = _packed(lengths, H_q, H_kv, k, seed=800 + 10 * case)
    bi = oracle.index_topk_varlen(p.q_idx, p.k_idx, p.cu_seqlens, k, 128)
    o, lse = msa.msa_sparse_attn_fwd_varlen(p.q, p.k, p.v, torch.from_numpy(bi).to(DEV), p.cu_seqlens)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.sparse_attn_varlen(p.q, p.k, p.v, bi, p.cu_seqlens, 128)
    check_attn(o.cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, f"varlen case {case}")


@pytest.mark.parametrize("mode", ["literal", "structured"])
def test_varlen_end_to_end(msa, mode):
    lengths, H_q, H_kv, k = [1500, 40, 2600, 128, 129], 16, 2, 8
    p = _packed(lengths, H_q, H_kv, k, seed=901, mode=mode)
    bi, ties = _check_index_varlen(msa, p, k)
    o, lse = msa.msa_sparse_attn_fwd_varlen(p.q, p.k, p.v, bi, p.cu_seqlens)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.sparse_attn_varlen(p.q, p.k, p.v, bi.cpu().numpy(), p.cu_seqlens, 128)
    check_attn(o.cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, f"varlen e2e {mode}")


def test_varlen_arbitrary_block_sets(msa):
    """-1 entries, blocks past the sequence's end or the query's local block, empty rows."""
    lengths, H_q, H_kv, k = [600, 1100, 260], 8, 2, 5
    p = _packed(lengths, H_q, H_kv, k, seed=902)
    T = sum(lengths)
    g = np.random.default_rng(4)
    bi = np.full((T, H_kv, k), -1, dtype=np.int32)
    for i in range(T):
        for r in range(H_kv):
            c = g.choice(12, size=g.integers(0, k + 1), replace=False)  # up to block 11 > any sequence's last
            bi[i, r, :len(c)] = c
    bi[3] = -1
    o, lse = msa.msa_sparse_attn_fwd_varlen(p.q, p.k, p.v, torch.from_numpy(bi).to(DEV), p.cu_seqlens)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.sparse_attn_varlen(p.q, p.k, p.v, bi, p.cu_seqlens, 128)
    assert np.all(np.isinf(lse_ref[3]))
    check_attn(o.cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, "varlen arbitrary sets")


def test_single_sequence_varlen_equals_fixed_path(msa):
    N, H_q, H_kv, k = 2900, 16, 2, 6
    p = _packed([N], H_q, H_kv, k, seed=903)
    bi_v = msa.msa_index_topk_varlen(p.q_idx, p.k_idx, p.cu_seqlens, N, k)
    bi_f = msa.msa_index_topk(p.q_idx, p.k_idx, k)
    o_v, l_v = msa.msa_sparse_attn_fwd_varlen(p.q, p.k, p.v, bi_f, p.cu_seqlens)
    o_f, l_f = msa.msa_sparse_attn_fwd(p.q, p.k, p.v, bi_f)
    torch.cuda.synchronize()
    assert torch.equal(bi_v, bi_f)
    assert torch.equal(l_v, l_f)
    # Same arithmetic per row; the list stride differs (one spare block per
    # sequence), which may only reorder nothing: outputs must agree to the bit.
    assert torch.equal(o_v, o_f)


def test_varlen_windows_across_sequences_are_bitwise_identical(msa):
    """The minimum workspace runs 128-query windows that straddle sequence boundaries."""
    lengths, H_q, H_kv, k = [300, 77, 1000, 513], 8, 2, 6
    p = _packed(lengths, H_q, H_kv, k, seed=904)
    T = sum(lengths)
    bi = msa.msa_index_topk_varlen(p.q_idx, p.k_idx, p.cu_seqlens, max(lengths), k)
    o1, l1 = msa.msa_sparse_attn_fwd_varlen(p.q, p.k, p.v, bi, p.cu_seqlens)
    wmin = msa.msa_sparse_attn_fwd_varlen_workspace(T, len(lengths), H_q, H_kv, k, minimum=True)
    assert 0 < wmin < msa.msa_sparse_attn_fwd_varlen_workspace(T, len(lengths), H_q, H_kv, k)
    ws = torch.empty(wmin, dtype=torch.uint8, device=DEV)
    o2, l2 = msa.msa_sparse_attn_fwd_varlen(p.q, p.k, p.v, bi, p.cu_seqlens, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    o_ref, lse_ref = oracle.sparse_attn_varlen(p.q, p.k, p.v, bi.cpu().numpy(), p.cu_seqlens, 128)
    check_attn(o2.cpu().numpy(), l2.cpu().numpy(), o_ref, lse_ref, "varlen min workspace")


def test_varlen_empty(msa):
    cu = torch.zeros(3, dtype=torch.int64, device=DEV)
    z = torch.empty((0, 2, 64), dtype=torch.bfloat16, device=DEV)
    bi = msa.msa_index_topk_varlen(z, torch.empty((0, 64), dtype=torch.bfloat16, device=DEV), cu, 0, 4)
    assert bi.shape == (0, 2, 4)
    q = torch.empty((0, 8, 128), dtype=torch.bfloat16, device=DEV)
    kv = torch.empty((0, 2, 128), dtype=torch.bfloat16, device=DEV)
    o, lse = msa.msa_sparse_attn_fwd_varlen(q, kv, kv, torch.empty((0, 2, 4), dtype=torch.int32, device=DEV), cu)
    assert o.shape == (0, 8, 128) and lse.shape == (0, 8)
