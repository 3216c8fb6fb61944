"""GPU parity of the paged FP8 decode against the oracle (same FP8 codes, same page
table), plus equality with the contiguous bf16 decode when the cached values are
exactly FP8-representable."""
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


PAGED_CASES = [  # lengths, H_q, H_kv, k
    ([1, 100, 128, 129, 1000, 5000], 16, 2, 4),
    ([4096, 3000, 256, 640], 64, 8, 16),
    ([2000, 70], 8, 8, 32),
    ([384] * 3, 16, 1, 3),
    ([777, 1280], 4, 4, 8),
]


def _run(msa, p, k):
    max_len = max(p.lengths)
    return msa.msa_decode_paged(p.q, p.q_idx, p.k_pages, p.v_pages, p.k_scale, p.v_scale, p.kidx_pages,
                                p.block_table, p.seqlens, max_len, k)


@pytest.mark.parametrize("mode", ["literal", "structured"])
@pytest.mark.parametrize("case", range(len(PAGED_CASES)))
def test_decode_paged_matches_oracle(msa, case, mode):
    lengths, H_q, H_kv, k = PAGED_CASES[case]
    cfg = synth.DecodeConfig("t", batch=len(lengths), H_q=H_q, H_kv=H_kv, k=k, len_lo_blocks=1, len_hi_blocks=1,
                             seed=900 + case)
    p = synth.make_decode_paged(cfg, mode, device=DEV, lengths=lengths)
    bi, o, lse = _run(msa, p, k)
    torch.cuda.synchronize()
    bi_ref, o_ref, lse_ref, M = oracle.decode_paged(p.q, p.q_idx, p.k_pages, p.v_pages, p.k_scale, p.v_scale,
                                                    p.kidx_pages, p.block_table, p.seqlens, k, 128,
                                                    want_scores=True)
    bi_gpu = bi.cpu().numpy()
    tie = check_block_idx(bi_gpu, M, np.array(lengths) - 1, k, 128)
    if tie.any():  # attention compared on the GPU's own (valid) selection
        _, o_ref, lse_ref = oracle.decode_paged(p.q, p.q_idx, p.k_pages, p.v_pages, p.k_scale, p.v_scale,
                                                p.kidx_pages, p.block_table, p.seqlens, k, 128, block_idx=bi_gpu)
    check_attn(o.cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, f"paged case {case} {mode}")


def test_decode_paged_equals_contiguous_when_exact(msa):
    """K/V exactly FP8-representable and scales 1: the paged FP8 decode and the
    contiguous bf16 decode see the same numbers and run the same arithmetic, so
    they agree bit for bit."""
    lengths, H_q, H_kv, k = [3000, 129, 1024, 1], 16, 2, 6
    cfg = synth.DecodeConfig("t", batch=4, H_q=H_q, H_kv=H_kv, k=k, len_lo_blocks=1, len_hi_blocks=1, seed=950)
    p = synth.make_decode_paged(cfg, device=DEV, lengths=lengths, unit_scale=True)
    d = p.contiguous
    bi_p, o_p, l_p = _run(msa, p, k)
    bi_c, o_c, l_c = msa.msa_decode(d.q.to(DEV), d.q_idx.to(DEV), d.k_cache.to(DEV), d.v_cache.to(DEV),
                                    d.k_idx_cache.to(DEV), d.cu_seqlens.to(DEV), max(lengths), k)
    torch.cuda.synchronize()
    assert torch.equal(bi_p, bi_c)
    assert torch.equal(o_p, o_c) and torch.equal(l_p, l_c)


@pytest.mark.parametrize("B_k", [128, 64])
@pytest.mark.parametrize("k", [4, 16, 32])
def test_decode_paged_exact_ties_go_to_lower_block(msa, k, B_k):
    """Index-key pages duplicated pairwise (the page of odd block b holds the keys of
    block b - 1): exact boundary ties must go to the lower block, bit-exactly."""
    batch, H_q, H_kv = 48, 16, 8
    cfg = synth.DecodeConfig("t", batch=batch, H_q=H_q, H_kv=H_kv, k=k, len_lo_blocks=24, len_hi_blocks=48,
                             B_k=B_k, seed=960 + k + B_k)
    p = synth.make_decode_paged(cfg, device=DEV)
    table = p.block_table.cpu()
    for s, L in enumerate(p.lengths):
        for b in range(1, L // B_k, 2):
            p.kidx_pages[int(table[s, b])] = p.kidx_pages[int(table[s, b - 1])]
    bi, o, lse = msa.msa_decode_paged(p.q, p.q_idx, p.k_pages, p.v_pages, p.k_scale, p.v_scale, p.kidx_pages,
                                      p.block_table, p.seqlens, max(p.lengths), k, B_k=B_k)
    torch.cuda.synchronize()
    _, _, _, M = oracle.decode_paged(p.q, p.q_idx, p.k_pages, p.v_pages, p.k_scale, p.v_scale, p.kidx_pages,
                                     p.block_table, p.seqlens, k, B_k, want_scores=True)
    pos = np.array(p.lengths) - 1
    bi = bi.cpu().numpy()
    check_block_idx(bi, M, pos, k, B_k)
    n_tied = check_exact_twin_ties(bi, M, pos, k, B_k)
    assert n_tied >= batch * H_kv // 4, f"only {n_tied} rows had an isolated exact tie"
