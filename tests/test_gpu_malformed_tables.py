"""Device tables that break their documented form (packed offsets out of range or
decreasing, paged lengths past the table row, page numbers out of range) are read
through the library's clamps: every call finishes, and its results equal those of
the same call on the well-formed table the clamps map it to (bitwise).  The clamp
arithmetic itself is pinned on the CPU (test_table_clamp.py); these tables stay
within what the clamps cover, so no access can leave the buffers."""
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


def _cu(vals):
    return torch.tensor(vals, dtype=torch.int64, device=DEV)


def test_varlen_offsets_out_of_range(msa):
    lengths, H_q, H_kv, k = [1000, 129, 2047, 300], 16, 2, 4
    print(f"[malformed] varlen lengths {lengths}", flush=True)
    p = synth.packed_prefill(lengths, H_q, H_kv, k, 951, device=DEV)
    T = sum(lengths)
    cu = p.cu_seqlens.cpu().tolist()
    # First entry below 0 and last past T: both calls read the well-formed spans.
    bad = _cu([-50] + cu[1:-1] + [T + 999])
    bi = msa.msa_index_topk_varlen(p.q_idx, p.k_idx, p.cu_seqlens, max(lengths), k)
    bi_bad = msa.msa_index_topk_varlen(p.q_idx, p.k_idx, bad, max(lengths), k)
    o, lse = msa.msa_sparse_attn_fwd_varlen(p.q, p.k, p.v, bi, p.cu_seqlens)
    o_bad, lse_bad = msa.msa_sparse_attn_fwd_varlen(p.q, p.k, p.v, bi, bad)
    torch.cuda.synchronize()
    assert torch.equal(bi, bi_bad)
    assert torch.equal(o, o_bad) and torch.equal(lse, lse_bad)


def test_varlen_attention_sanitises_decreasing_offsets(msa):
    """The attention copies the table as 0, the running maximum clamped into [0, T],
    T: [7, c2, c1, c3 + 5, 3] becomes [0, c2, c2, c3 + 5, T]."""
    lengths, H_q, H_kv, k = [700, 900, 1300, 400], 8, 2, 6
    print(f"[malformed] varlen decreasing, lengths {lengths}", flush=True)
    p = synth.packed_prefill(lengths, H_q, H_kv, k, 952, device=DEV)
    T = sum(lengths)
    c = p.cu_seqlens.cpu().tolist()
    bad = _cu([7, c[2], c[1], c[3] + 5, 3])
    good = _cu([0, c[2], c[2], c[3] + 5, T])
    glen = [c[2], 0, c[3] + 5 - c[2], T - c[3] - 5]
    bi = msa.msa_index_topk_varlen(p.q_idx, p.k_idx, good, max(glen), k)
    o, lse = msa.msa_sparse_attn_fwd_varlen(p.q, p.k, p.v, bi, good)
    o_bad, lse_bad = msa.msa_sparse_attn_fwd_varlen(p.q, p.k, p.v, bi, bad)
    torch.cuda.synchronize()
    assert torch.equal(o, o_bad) and torch.equal(lse, lse_bad)


def test_decode_offsets_out_of_range(msa):
    cfg = synth.DecodeConfig("malformed", batch=3, H_q=16, H_kv=2, k=4, len_lo_blocks=1, len_hi_blocks=8,
                             seed=953)
    lengths = [300, 1000, 129]
    print(f"[malformed] decode lengths {lengths}", flush=True)
    d = synth.make_decode(cfg, device=DEV, lengths=lengths)
    T = d.k_cache.shape[0]
    c = d.cu_seqlens.cpu().tolist()
    max_len = max(lengths)
    ref = msa.msa_decode(d.q, d.q_idx, d.k_cache, d.v_cache, d.k_idx_cache, d.cu_seqlens, max_len, cfg.k)
    bad = _cu([-9, c[1], c[2], T + 12345])
    got = msa.msa_decode(d.q, d.q_idx, d.k_cache, d.v_cache, d.k_idx_cache, bad, max_len, cfg.k)
    # Decreasing offsets: sequences 0 and 1 become empty (start clamped past their
    # end), sequence 2 reads tokens 5 .. T-1, i.e. a one-sequence cache from row 5.
    dec = _cu([c[2], c[1], 5, T + 1])
    got2 = msa.msa_decode(d.q, d.q_idx, d.k_cache, d.v_cache, d.k_idx_cache, dec, T, cfg.k)
    one = msa.msa_decode(d.q[2:], d.q_idx[2:], d.k_cache[5:], d.v_cache[5:], d.k_idx_cache[5:],
                         _cu([0, T - 5]), T, cfg.k)
    torch.cuda.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a, b)
    bi2, o2, lse2 = got2
    assert torch.all(bi2[:2] == -1) and torch.all(torch.isinf(lse2[:2])) and torch.all(lse2[:2] < 0)
    assert torch.equal(bi2[2:], one[0]) and torch.equal(o2[2:], one[1]) and torch.equal(lse2[2:], one[2])


def test_decode_paged_lengths_and_pages_out_of_range(msa):
    cfg = synth.DecodeConfig("malformed_paged", batch=3, H_q=16, H_kv=2, k=4, len_lo_blocks=1, len_hi_blocks=8,
                             seed=954)
    lengths = [700, 256, 1000]
    print(f"[malformed] paged decode lengths {lengths}", flush=True)
    p = synth.make_decode_paged(cfg, device=DEV, lengths=lengths)
    P = p.k_pages.shape[0]
    max_blocks = p.block_table.shape[1]
    B_k = cfg.B_k
    max_len = max_blocks * B_k
    good_t = p.block_table.clone()
    good_t[good_t < 0] = 0  # unused entries: a valid page, read once a length covers them
    good_l = p.seqlens.clone()
    bad_t = good_t.clone()
    bad_l = p.seqlens.clone()
    bad_t[0, 0] = -5
    good_t[0, 0] = 0
    bad_t[2, 1] = P + 100
    good_t[2, 1] = P - 1
    bad_l[1] = 10 ** 12          # past the table row: read as max_blocks * B_k tokens
    good_l[1] = max_blocks * B_k
    args = (p.q, p.q_idx, p.k_pages, p.v_pages, p.k_scale, p.v_scale, p.kidx_pages)
    ref = msa.msa_decode_paged(*args, good_t, good_l, max_len, cfg.k)
    got = msa.msa_decode_paged(*args, bad_t, bad_l, max_len, cfg.k)
    torch.cuda.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a, b)
