"""GPU parity of the split-form selection (msa_topk_from_scores) on long score rows.

Rows here hold 1,000 to 8,191 causal blocks, so both kernels (rows of up to 32
register-held chunks of 64 blocks, and longer rows streamed from memory) and the
fallback of each for rows with too many candidates run; the oracle checks sampled
rows (it takes explicit row positions).  Scores are drawn on the device from a
seeded generator.
"""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def msa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_gqa_index_amd as m
    return m


def _sample_rows(N, n, seed):
    g = np.random.default_rng(seed)
    rows = np.concatenate([g.choice(N, size=n, replace=False), np.arange(N - 32, N)])
    return np.unique(rows)


def _check_rows(bi, M, rows, k, B_k):
    r = torch.from_numpy(rows).to(M.device)
    ref = oracle.topk(M[r].double().cpu().numpy(), k, B_k, rows=rows)
    np.testing.assert_array_equal(bi[r].cpu().numpy(), ref)


@pytest.mark.parametrize("k", [9, 16, 32])
def test_long_rows_random(msa, k):
    N, H_kv, BK = 76000, 2, 64  # up to 1,187 causal blocks: 19 chunks of 64
    B = (N + BK - 1) // BK
    g = torch.Generator(device=DEV).manual_seed(5000 + k)
    M = torch.randn((N, H_kv, B), generator=g, device=DEV)
    bi = msa.msa_topk_from_scores(M, k, B_k=BK)
    torch.cuda.synchronize()
    _check_rows(bi, M, _sample_rows(N, 200, k), k, BK)


# 76,000 tokens: up to 19 chunks (register-held rows); 200,000: up to 49 (streamed).
@pytest.mark.parametrize("N", [76000, 200000])
@pytest.mark.parametrize("k", [16, 32])
def test_few_lanes_own_the_best_blocks(msa, k, N):
    """Blocks b with b % 64 < k - 2 outscore all others: with k = 32 the rows near the
    end have more than 512 blocks at or above the lane-best bound (the fallback)."""
    H_kv, BK = 1, 64
    B = (N + BK - 1) // BK
    g = torch.Generator(device=DEV).manual_seed(6000 + k)
    M = torch.randn((N, H_kv, B), generator=g, device=DEV)
    hot = (torch.arange(B, device=DEV) % 64) < k - 2
    M[:, :, hot] += 100.0
    bi = msa.msa_topk_from_scores(M, k, B_k=BK)
    torch.cuda.synchronize()
    _check_rows(bi, M, _sample_rows(N, 200, 60 + k), k, BK)
    del M
    torch.cuda.empty_cache()


@pytest.mark.parametrize("N", [76000, 200000])
def test_ties_and_neg_inf_long_rows(msa, N):
    """Scores on a coarse grid (many exact ties) with some -inf entries."""
    H_kv, BK, k = 1, 64, 32
    B = (N + BK - 1) // BK
    g = torch.Generator(device=DEV).manual_seed(6100)
    M = torch.randint(-4, 5, (N, H_kv, B), generator=g, device=DEV).float() * 0.5
    M[torch.rand((N, H_kv, B), generator=g, device=DEV) < 0.3] = -float("inf")
    bi = msa.msa_topk_from_scores(M, k, B_k=BK)
    torch.cuda.synchronize()
    _check_rows(bi, M, _sample_rows(N, 200, 61), k, BK)
    del M
    torch.cuda.empty_cache()


def test_neg_inf_short_rows(msa):
    """Rows whose causal prefix is mostly -inf: -inf blocks fill the selection last."""
    N, H_kv, k = 3000, 2, 8
    B = (N + 127) // 128
    g = torch.Generator().manual_seed(6200)
    M = torch.randn((N, H_kv, B), generator=g)
    M[torch.rand((N, H_kv, B), generator=g) < 0.8] = -float("inf")
    bi = msa.msa_topk_from_scores(M.to(DEV), k)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bi.cpu().numpy(), oracle.topk(M.double().numpy(), k, 128))


def test_rows_at_block_limit(msa):
    """8,192 blocks (B_k = 64, N = 524,288): rows of up to 128 chunks of 64 blocks."""
    N, H_kv, BK, k = 524288, 1, 64, 32
    B = N // BK
    g = torch.Generator(device=DEV).manual_seed(6300)
    M = torch.randn((N, H_kv, B), generator=g, device=DEV)
    bi = msa.msa_topk_from_scores(M, k, B_k=BK)
    torch.cuda.synchronize()
    _check_rows(bi, M, _sample_rows(N, 100, 63), k, BK)
    del M
    torch.cuda.empty_cache()


def test_signed_zeros_tie(msa):
    """-0.0 and +0.0 compare equal, so a tie between them goes to the lower block like
    any other tie (scores drawn from {-1, -0, +0, 1})."""
    N, H_kv, k = 5000, 2, 8
    B = (N + 127) // 128
    g = torch.Generator().manual_seed(6400)
    M = torch.tensor([-1.0, -0.0, 0.0, 1.0])[torch.randint(0, 4, (N, H_kv, B), generator=g)]
    assert (torch.signbit(M) & (M == 0)).any() and (~torch.signbit(M) & (M == 0)).any()
    bi = msa.msa_topk_from_scores(M.to(DEV), k)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bi.cpu().numpy(), oracle.topk(M.double().numpy(), k, 128))
