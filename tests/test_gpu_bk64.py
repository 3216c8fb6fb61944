"""GPU parity with 64-key blocks (B_k = 64: twice the blocks, as in the pages'
Table 1 rows with 2048 and 8192 blocks), against the oracle run with B_k = 64."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.parity import check_attn, check_block_idx

pytestmark = pytest.mark.gpu

DEV = "cuda"
BK = 64


@pytest.fixture(scope="module")
def msa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_gqa_index_amd as m
    return m


def _inputs(N, H_q, H_kv, k, seed, mode="literal", needles=0):
    return synth.small_prefill(N=N, H_q=H_q, H_kv=H_kv, k=k, seed=seed, mode=mode, needles=needles, B_k=BK,
                               device=DEV)


SHAPES = [  # N, H_q, H_kv, k
    (4096, 4, 1, 8),
    (1000, 16, 2, 4),
    (129, 8, 1, 2),
    (65, 4, 2, 3),
    (3000, 8, 1, 32),
    (2047, 16, 4, 16),
    (700, 8, 8, 9),
]


@pytest.mark.parametrize("N,H_q,H_kv,k", SHAPES)
def test_block_scores_bk64(msa, N, H_q, H_kv, k):
    inp = _inputs(N, H_kv, H_kv, k, seed=1300 + N)
    M = msa.msa_index_block_scores(inp.q_idx, inp.k_idx, B_k=BK)
    torch.cuda.synchronize()
    Mo = oracle.block_scores(inp.q_idx, inp.k_idx, BK)
    Mg = M.double().cpu().numpy()
    fin = np.isfinite(Mo)
    assert np.array_equal(np.isfinite(Mg), fin)
    err = np.abs(Mg[fin] - Mo[fin]) / np.maximum(1.0, np.abs(Mo[fin]))
    assert err.max() <= 1e-5


@pytest.mark.parametrize("mode", ["literal", "structured"])
@pytest.mark.parametrize("N,H_q,H_kv,k", SHAPES)
def test_index_and_attention_bk64(msa, N, H_q, H_kv, k, mode):
    inp = _inputs(N, H_q, H_kv, k, seed=1400 + N + k, mode=mode, needles=1 if N >= 2000 else 0)
    bi = msa.msa_index_topk(inp.q_idx, inp.k_idx, k, B_k=BK)
    o, lse = msa.msa_sparse_attn_fwd(inp.q, inp.k, inp.v, bi, B_k=BK)
    torch.cuda.synchronize()
    M = oracle.block_scores(inp.q_idx, inp.k_idx, BK)
    check_block_idx(bi.cpu().numpy(), M, np.arange(N), k, BK)
    o_ref, lse_ref = oracle.sparse_attn(inp.q, inp.k, inp.v, bi.cpu().numpy(), BK)
    check_attn(o.cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, f"B_k=64 N={N} {mode}")


def test_topk_from_scores_bk64(msa):
    N, H_kv, k = 3000, 2, 16
    g = torch.Generator().manual_seed(77)
    B = (N + BK - 1) // BK
    M = torch.randint(-6, 7, (N, H_kv, B), generator=g).float() * 0.25
    bi = msa.msa_topk_from_scores(M.to(DEV), k, B_k=BK)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bi.cpu().numpy(), oracle.topk(M.double().numpy(), k, BK))


def test_varlen_bk64(msa):
    lengths, H_q, H_kv, k = [1000, 65, 0, 2500, 64], 8, 2, 6
    p = synth.packed_prefill(lengths, H_q, H_kv, k, seed=1500, device=DEV)
    bi = msa.msa_index_topk_varlen(p.q_idx, p.k_idx, p.cu_seqlens, max(lengths), k, B_k=BK)
    o, lse = msa.msa_sparse_attn_fwd_varlen(p.q, p.k, p.v, bi, p.cu_seqlens, B_k=BK)
    torch.cuda.synchronize()
    bi_h = bi.cpu().numpy()
    _, Ms = oracle.index_topk_varlen(p.q_idx, p.k_idx, p.cu_seqlens, k, BK, want_scores=True)
    cu = p.cu_seqlens.cpu().tolist()
    for s, L in enumerate(lengths):
        if L:
            check_block_idx(bi_h[cu[s]:cu[s + 1]], Ms[s], np.arange(L), k, BK)
    o_ref, lse_ref = oracle.sparse_attn_varlen(p.q, p.k, p.v, bi_h, p.cu_seqlens, BK)
    check_attn(o.cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, "varlen B_k=64")


@pytest.mark.parametrize("case", range(3))
def test_decode_bk64(msa, case):
    lengths, H_q, H_kv, k = [([1, 64, 65, 129, 1000, 5000], 16, 2, 4), ([4096, 3000, 256, 640], 64, 8, 32),
                             ([777, 130], 8, 8, 16)][case]
    cfg = synth.DecodeConfig("t", batch=len(lengths), H_q=H_q, H_kv=H_kv, k=k, len_lo_blocks=1, len_hi_blocks=1,
                             B_k=BK, seed=1600 + case)
    d = synth.make_decode(cfg, device=DEV, lengths=lengths)
    bi, o, lse = msa.msa_decode(d.q, d.q_idx, d.k_cache, d.v_cache, d.k_idx_cache, d.cu_seqlens, max(lengths), k,
                                B_k=BK)
    torch.cuda.synchronize()
    bi_ref, o_ref, lse_ref, M = oracle.decode(d.q, d.q_idx, d.k_cache, d.v_cache, d.k_idx_cache, d.cu_seqlens, k,
                                              BK, want_scores=True)
    bi_gpu = bi.cpu().numpy()
    tie = check_block_idx(bi_gpu, M, np.array(lengths) - 1, k, BK)
    if tie.any():
        o_ref, lse_ref = oracle.decode_attn(d.q, d.k_cache, d.v_cache, d.cu_seqlens, bi_gpu, BK)
    check_attn(o.cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, f"decode B_k=64 case {case}")


@pytest.mark.parametrize("N,H_q,H_kv,k", [(3000, 8, 2, 12), (700, 16, 1, 5), (129, 4, 4, 2), (2100, 32, 1, 32)])
def test_sparse_kl_bk64(msa, N, H_q, H_kv, k):
    """The KL alignment pass over 64-key blocks (Eq. 9-10), on the GPU's own selection."""
    from tests.test_gpu_kl import _check_kl
    inp = synth.small_prefill(N=N, H_q=H_q, H_kv=H_kv, k=k, seed=1900 + N, B_k=BK, needles=1 if N >= 2000 else 0,
                              device=DEV)
    bi = msa.msa_index_topk(inp.q_idx, inp.k_idx, k, B_k=BK)
    _, lse = msa.msa_sparse_attn_fwd(inp.q, inp.k, inp.v, bi, B_k=BK)
    kl, lse_idx, loss = msa.msa_sparse_kl_fwd(inp.q, inp.k, inp.q_idx, inp.k_idx, bi, lse, B_k=BK)
    wmin = msa.msa_sparse_kl_fwd_workspace(N, H_q, H_kv, k, B_k=BK, minimum=True)
    ws = torch.empty(wmin, dtype=torch.uint8, device=DEV)
    kl2, li2, loss2 = msa.msa_sparse_kl_fwd(inp.q, inp.k, inp.q_idx, inp.k_idx, bi, lse, B_k=BK, workspace=ws)
    torch.cuda.synchronize()
    kl_ref, li_ref = oracle.sparse_kl(inp.q, inp.k, inp.q_idx, inp.k_idx, bi.cpu().numpy(), BK)
    _check_kl(kl, lse_idx, loss, kl_ref, li_ref, f"B_k=64 N={N} H_q={H_q} H_kv={H_kv} k={k}")
    assert torch.equal(kl, kl2) and torch.equal(lse_idx, li2)


@pytest.mark.parametrize("N,H_q,H_kv,k", [(1000, 16, 2, 4), (129, 8, 1, 2), (65, 4, 4, 3), (2600, 32, 1, 9),
                                         (3000, 4, 2, 32)])
def test_backward_bk64(msa, N, H_q, H_kv, k):
    """Gradients of Eq. 8 over 64-key blocks (selection fixed, taken from the oracle), and
    the same dK, dV bit for bit from a rerun with the minimum workspace."""
    from tests.test_gpu_backward import check_grads
    inp = synth.small_prefill(N=N, H_q=H_q, H_kv=H_kv, k=k, seed=2000 + N, B_k=BK, needles=1 if N >= 2000 else 0,
                              device=DEV)
    bi = oracle.topk(oracle.block_scores(inp.q_idx, inp.k_idx, BK), k, BK)
    bi_d = torch.from_numpy(bi).to(DEV)
    o, lse = msa.msa_sparse_attn_fwd(inp.q, inp.k, inp.v, bi_d, B_k=BK)
    g = torch.Generator(device=DEV).manual_seed(N)
    dO = torch.randn(inp.q.shape, generator=g, device=DEV).to(torch.bfloat16)
    grads = msa.msa_sparse_attn_bwd(inp.q, inp.k, inp.v, o, lse, dO, bi_d, B_k=BK)
    wmin = msa.msa_sparse_attn_bwd_workspace(N, H_q, H_kv, k, B_k=BK, minimum=True)
    ws = torch.empty(wmin, dtype=torch.uint8, device=DEV)
    g2 = msa.msa_sparse_attn_bwd(inp.q, inp.k, inp.v, o, lse, dO, bi_d, B_k=BK, workspace=ws)
    torch.cuda.synchronize()
    ref = oracle.sparse_attn_bwd(inp.q, inp.k, inp.v, dO, bi, BK)
    check_grads(grads, ref, f"B_k=64 N={N} H_q={H_q} H_kv={H_kv} k={k}")
    check_grads(g2, ref, f"B_k=64 min workspace N={N}")


@pytest.mark.parametrize("case", range(3))
def test_decode_paged_bk64(msa, case):
    """Paged FP8 decode over 64-token pages (one page per block, in random order): a
    128-key scoring tile spans two pages."""
    lengths, H_q, H_kv, k = [([1, 64, 65, 129, 1000, 5000], 16, 2, 4), ([4096, 3000, 256, 640], 64, 8, 32),
                             ([777, 130, 191], 8, 8, 16)][case]
    cfg = synth.DecodeConfig("t", batch=len(lengths), H_q=H_q, H_kv=H_kv, k=k, len_lo_blocks=1, len_hi_blocks=1,
                             B_k=BK, seed=2100 + case)
    p = synth.make_decode_paged(cfg, "structured" if case == 1 else "literal", device=DEV, lengths=lengths)
    bi, o, lse = msa.msa_decode_paged(p.q, p.q_idx, p.k_pages, p.v_pages, p.k_scale, p.v_scale, p.kidx_pages,
                                      p.block_table, p.seqlens, max(lengths), k, B_k=BK)
    torch.cuda.synchronize()
    bi_ref, o_ref, lse_ref, M = oracle.decode_paged(p.q, p.q_idx, p.k_pages, p.v_pages, p.k_scale, p.v_scale,
                                                    p.kidx_pages, p.block_table, p.seqlens, k, BK, want_scores=True)
    bi_gpu = bi.cpu().numpy()
    tie = check_block_idx(bi_gpu, M, np.array(lengths) - 1, k, BK)
    if tie.any():
        _, o_ref, lse_ref = oracle.decode_paged(p.q, p.q_idx, p.k_pages, p.v_pages, p.k_scale, p.v_scale,
                                                p.kidx_pages, p.block_table, p.seqlens, k, BK, block_idx=bi_gpu)
    check_attn(o.cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, f"paged B_k=64 case {case}")
