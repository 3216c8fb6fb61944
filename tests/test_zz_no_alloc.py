"""The allocation-free decode entry point (static scratch) against msa_decode with a
caller workspace: two calls in a row, the second smaller, both bit-identical."""
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def msa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_gqa_index_amd as m
    return m


def _case(msa, lengths, H_q, H_kv, k, B_k, seed):
    cfg = synth.DecodeConfig("t", batch=len(lengths), H_q=H_q, H_kv=H_kv, k=k, len_lo_blocks=1, len_hi_blocks=1,
                             B_k=B_k, seed=seed)
    d = synth.make_decode(cfg, device=DEV, lengths=lengths)
    max_len = max(lengths)
    ref = msa.msa_decode(d.q, d.q_idx, d.k_cache, d.v_cache, d.k_idx_cache, d.cu_seqlens, max_len, k, B_k=B_k)
    bi = torch.full((len(lengths), H_kv, k), -7, dtype=torch.int32, device=DEV)
    o = torch.full((len(lengths), H_q, 128), float("nan"), dtype=torch.float32, device=DEV)
    lse = torch.full((len(lengths), H_q), float("nan"), dtype=torch.float32, device=DEV)
    got = msa.msa_decode_noalloc(d.q, d.q_idx, d.k_cache, d.v_cache, d.k_idx_cache, d.cu_seqlens, max_len, k,
                                 B_k=B_k, block_idx=bi, o=o, lse=lse)
    torch.cuda.synchronize()
    for a, b, name in zip(got, ref, ("block_idx", "o", "lse")):
        assert torch.equal(a, b), f"{name} differs from msa_decode"


def test_noalloc_decode_matches_workspace_decode_twice(msa):
    # A larger call first, then a smaller one that reuses the same static scratch.
    _case(msa, [4096, 3000, 640, 129, 8192, 1], 64, 8, 16, 128, seed=1200)
    _case(msa, [700, 256], 16, 2, 4, 64, seed=1201)


def test_noalloc_decode_rejects_shapes_beyond_the_scratch(msa):
    raw = msa.raw()
    f = 0x10000  # never dereferenced: the size check fails first
    st = raw.msa_decode_noalloc(f, f, f, f, f, f, 512, 512 << 20, 1 << 20, 64, 8, 128, 64, 128, 16, 0.088, f, f, f,
                                None)
    assert st == msa.MSA_ERR_WORKSPACE
    assert "static" in raw.msa_last_error().decode()
