"""GPU parity at the full workload sizes (32K, 128K and 1M prefill, 128K with B_k = 64,
a packed batch of 128K tokens; 64-sequence decode),
in the launch configuration the benchmark times, on sampled rows the oracle computes
one by one.  The sample holds rows with fewer than k causal blocks, uniform rows, the
last rows of the sequence and rows right after needle blocks."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.parity import check_attn, check_block_idx

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

DEV = "cuda"


@pytest.fixture(scope="module")
def msa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_gqa_index_amd as m
    return m


def sample_rows(cfg, needles, n_uniform, seed):
    g = np.random.default_rng(seed)
    N, B_k, k = cfg.N, cfg.B_k, cfg.k
    rows = set(range(0, min(N, k * B_k), 37))                      # fewer than k causal blocks
    rows |= set(g.choice(N, size=n_uniform, replace=False).tolist())  # uniform
    rows |= set(range(max(0, N - 24), N))                          # last rows
    for b in needles[0][:4] if needles and needles[0] else []:
        rows |= {min(N - 1, (b + 1) * B_k), min(N - 1, (b + 1) * B_k + 77)}
    return np.array(sorted(rows), dtype=np.int64)


def _run_prefill(msa, name, mode, n_uniform):
    cfg = synth.CONFIGS[name]
    print(f"[full] {name} {mode}: generating inputs", flush=True)
    inp = synth.make_prefill(cfg, mode, device=DEV)
    k = cfg.k
    bi = msa.msa_index_topk(inp.q_idx, inp.k_idx, k, B_k=cfg.B_k)
    o, lse = msa.msa_sparse_attn_fwd(inp.q, inp.k, inp.v, bi, B_k=cfg.B_k)
    torch.cuda.synchronize()
    rows = sample_rows(cfg, inp.needles, n_uniform, cfg.seed)
    print(f"[full] {name} {mode}: oracle on {len(rows)} rows", flush=True)
    ridx = torch.from_numpy(rows).to(DEV)
    bi_s = bi[ridx].cpu().numpy()
    M = oracle.block_scores(inp.q_idx.cpu(), inp.k_idx.cpu(), cfg.B_k, rows=rows)
    tie = check_block_idx(bi_s, M, rows, k, cfg.B_k)
    # Main branch alone, at full size, on the GPU's own selection.
    q_h, k_h, v_h = inp.q.cpu(), inp.k.cpu(), inp.v.cpu()
    o_ref, lse_ref = oracle.sparse_attn(q_h, k_h, v_h, bi_s, cfg.B_k, rows=rows)
    stats = check_attn(o[ridx].cpu().numpy(), lse[ridx].cpu().numpy(), o_ref, lse_ref, f"{name} {mode}")
    # Rows away from near ties use exactly the oracle's selection.
    exact = oracle.topk(M, k, cfg.B_k, rows=rows)
    np.testing.assert_array_equal(bi_s[~tie], exact[~tie])
    print(f"[full] {name} {mode}: {len(rows)} rows, {int(tie.sum())} near-tie rows, {stats}", flush=True)


@pytest.mark.parametrize("mode", ["literal", "structured"])
def test_prefill_32k(msa, mode):
    _run_prefill(msa, "c1", mode, n_uniform=512)


@pytest.mark.parametrize("mode", ["literal", "structured"])
def test_prefill_128k(msa, mode):
    _run_prefill(msa, "c2", mode, n_uniform=256)


@pytest.mark.parametrize("mode", ["literal", "structured"])
def test_prefill_1m(msa, mode):
    _run_prefill(msa, "c4", mode, n_uniform=48)


@pytest.mark.parametrize("mode", ["literal", "structured"])
def test_prefill_128k_bk64(msa, mode):
    _run_prefill(msa, "c2_bk64", mode, n_uniform=128)


@pytest.mark.parametrize("mode", ["literal", "structured"])
def test_packed_batch_128k(msa, mode):
    """The packed variable-length batch the benchmark times (9 sequences, 131072
    tokens), checked per sequence on sampled rows."""
    vcfg = synth.VARLEN_CONFIGS["c2_varlen"]
    lengths = synth.varlen_lengths(vcfg)
    print(f"[full] {vcfg.name} {mode}: generating {len(lengths)} sequences", flush=True)
    p = synth.packed_prefill(lengths, vcfg.H_q, vcfg.H_kv, vcfg.k, vcfg.seed, mode, device=DEV)
    k, B_k = vcfg.k, vcfg.B_k
    bi = msa.msa_index_topk_varlen(p.q_idx, p.k_idx, p.cu_seqlens, max(lengths), k, B_k=B_k)
    o, lse = msa.msa_sparse_attn_fwd_varlen(p.q, p.k, p.v, bi, p.cu_seqlens, B_k=B_k)
    torch.cuda.synchronize()
    cu = p.cu_seqlens.cpu().tolist()
    for s, L in enumerate(lengths):
        a = cu[s]
        scfg = synth.PrefillConfig(f"seq{s}", N=L, H_q=vcfg.H_q, H_kv=vcfg.H_kv, k=k, B_k=B_k)
        rows = sample_rows(scfg, None, min(24, L), vcfg.seed + s)
        ridx = torch.from_numpy(rows + a).to(DEV)
        bi_s = bi[ridx].cpu().numpy()
        sl = slice(a, a + L)
        M = oracle.block_scores(p.q_idx[sl].cpu(), p.k_idx[sl].cpu(), B_k, rows=rows)
        tie = check_block_idx(bi_s, M, rows, k, B_k)
        o_ref, lse_ref = oracle.sparse_attn(p.q[sl].cpu(), p.k[sl].cpu(), p.v[sl].cpu(), bi_s, B_k, rows=rows)
        stats = check_attn(o[ridx].cpu().numpy(), lse[ridx].cpu().numpy(), o_ref, lse_ref,
                           f"{vcfg.name} {mode} sequence {s}")
        exact = oracle.topk(M, k, B_k, rows=rows)
        np.testing.assert_array_equal(bi_s[~tie], exact[~tie])
        print(f"[full] {vcfg.name} {mode} sequence {s} (L={L}): {len(rows)} rows, {stats}", flush=True)


@pytest.mark.parametrize("name", ["c3", "c3_128k"])
@pytest.mark.parametrize("mode", ["literal", "structured"])
def test_decode_64_sequences(msa, name, mode):
    cfg = synth.CONFIGS[name]
    print(f"[full] {name} {mode}: generating caches", flush=True)
    d = synth.make_decode(cfg, mode, device=DEV)
    max_len = max(d.lengths)
    bi, o, lse = msa.msa_decode(d.q, d.q_idx, d.k_cache, d.v_cache, d.k_idx_cache, d.cu_seqlens, max_len, cfg.k)
    torch.cuda.synchronize()
    print(f"[full] {name} {mode}: oracle on all {cfg.batch} sequences", flush=True)
    h = lambda t: t.cpu()
    bi_ref, o_ref, lse_ref, M = oracle.decode(h(d.q), h(d.q_idx), h(d.k_cache), h(d.v_cache), h(d.k_idx_cache),
                                              d.cu_seqlens, cfg.k, cfg.B_k, want_scores=True)
    bi_g = bi.cpu().numpy()
    tie = check_block_idx(bi_g, M, np.array(d.lengths) - 1, cfg.k, cfg.B_k)
    np.testing.assert_array_equal(bi_g[~tie], bi_ref[~tie])
    if tie.any():  # compare attention on the GPU's own selection
        o_ref, lse_ref = oracle.decode_attn(h(d.q), h(d.k_cache), h(d.v_cache), d.cu_seqlens, bi_g, cfg.B_k)
    stats = check_attn(o.cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, f"{name} {mode}")
    print(f"[full] {name} {mode}: {int(tie.sum())} near-tie rows, {stats}", flush=True)
